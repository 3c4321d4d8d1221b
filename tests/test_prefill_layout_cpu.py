"""CPU checks of the prefill kernel's index arithmetic (csrc/prefill.hip,
prefill32_kernel), re-stated here and run on every lane, register, thread and
stage:

* the 32 x 32 x 16 MFMA lane layout: the key that the kernel masks at score
  register (tile kt, register r) of lane (j, h) is the key the S^T product
  puts there, and the P^T operand a lane supplies for k-step s (its score
  registers 8s .. 8s + 7) meets, at every k-index, the V^T slot that holds
  the same key (bits 2 and 3 of the key swapped within a k-step);
* the V^T staging (store_v32): every (key, d) element of a stage is written
  exactly once, to the slot of its key in row d, and K (store_k32) fills
  every row and 16-byte chunk exactly once;
* the register loads with blocks of at least a stage: the per-thread offsets
  fixed for the loop reach every (key, chunk) of K and (key pair, d range) of
  V once, and V rows past the visible range re-read the last visible row,
  inside the same block;
* the first masked stage: no stage before it holds a key after any query of
  the wave, and it is the first that does;
* the pipeline: at every iteration the LDS holds K of the next stage and V of
  the current one, each written in an earlier iteration into a buffer no one
  reads in the iteration that writes it, and the block of every register
  load is the block of its stage.
"""

import numpy as np
import pytest

KKT = 64  # keys per stage


def swap23(x):
    return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1)


def mfma32_b(k, j):
    """lane and element of B[k][j] (16 x 32 operand, 8 consecutive k)."""
    return j + 32 * (k // 8), k % 8


def mfma32_d(i, j):
    """(lane, register) of D[i][j] for the 32 x 32 accumulator."""
    h = (i // 4) % 2
    r = 4 * (i // 8) + i % 4
    return j + 32 * h, r


def test_accumulator_layout_inverts():
    seen = set()
    for i in range(32):
        for j in range(32):
            lane, r = mfma32_d(i, j)
            h = lane // 32
            assert lane % 32 == j
            assert 8 * (r // 4) + 4 * h + r % 4 == i  # the kernel's reading
            seen.add((lane, r))
    assert len(seen) == 1024


def score_key(kt, r, h):
    """the key at score register (kt, r) of a lane in half h (kernel's mask)."""
    return 32 * kt + ((r & 15) >> 2) * 8 + 4 * h + (r & 3)


def test_scores_hold_the_keys_the_mask_names():
    # S^T = K Q^T: row i of tile kt is K row 32 kt + i of the stage
    for kt in range(2):
        for i in range(32):
            for j in range(32):
                lane, r = mfma32_d(i, j)
                assert score_key(kt, r, lane // 32) == 32 * kt + i
    # the mask's constant c(i) for flat index i = 16 kt + r equals key - 4h
    for h in range(2):
        for idx in range(32):
            c = (idx >> 4) * 32 + ((idx & 15) >> 2) * 8 + (idx & 3)
            assert c == score_key(idx >> 4, idx & 15, h) - 4 * h


def test_p_operand_meets_its_v_slot():
    # k-step s of O^T += V^T P^T: lane (j, h) gives B[8h + e][j] = its score
    # register 8s + e; the A operand V^T[d][k] is read at slot 16 s + 8h + e.
    slot_of_key = {key: (key & ~15) + swap23(key & 15) for key in range(KKT)}
    key_of_slot = {v: k for k, v in slot_of_key.items()}
    assert sorted(slot_of_key.values()) == list(range(KKT))
    for s in range(KKT // 16):
        for h in range(2):
            for e in range(8):
                flat = 8 * s + e
                key = score_key(flat >> 4, flat & 15, h)
                k_index = 8 * h + e
                lane_b, elem_b = mfma32_b(k_index, 0)
                assert (lane_b // 32, elem_b) == (h, e)
                slot = 16 * s + k_index
                assert key_of_slot[slot] == key
    # an even key and its odd neighbour stay adjacent (one dword per pair)
    for key in range(0, KKT, 2):
        assert slot_of_key[key + 1] == slot_of_key[key] + 1 and slot_of_key[key] % 2 == 0


@pytest.mark.parametrize("D", [128, 64])
def test_stage_stores_cover_the_stage_once(D):
    threads = 512
    KROW, VROW = 2 * D + 16, 2 * KKT + 16
    kchunks = KKT * D // 8 // threads
    vgroups = threads // 32
    VW = D // vgroups
    kmem, vmem = {}, {}
    for t in range(threads):
        for i in range(kchunks):
            c = t + i * threads
            key, ch = c // (D // 8), c % (D // 8)
            addr = key * KROW + ch * 16
            assert addr not in kmem and addr + 16 <= KKT * KROW
            kmem[addr] = (key, ch)
        pair, dg = t % 32, t // 32
        key0 = 2 * pair
        slot = (key0 & ~15) + swap23(key0 & 15)
        for w in range(VW // 2):
            d = dg * VW + 2 * w
            for dd in (d, d + 1):
                addr = dd * VROW + slot * 2
                assert addr not in vmem and addr + 4 <= D * VROW
                # low half: key0, high half: key0 + 1, both at element dd
                vmem[addr] = (dd, key0)
    assert sorted(kmem.values()) == [(k, c) for k in range(KKT) for c in range(D // 8)]
    got = sorted(vmem.values())
    assert got == sorted((d, k) for d in range(D) for k in range(0, KKT, 2))
    # the A operand read of V^T (row dt*32 + j, slots 16 s + 8h .. + 7) stays in its row
    for dt in range(D // 32):
        for j in range(32):
            for s in range(KKT // 16):
                for h in range(2):
                    off = (dt * 32 + j) * VROW + (s * 16 + h * 8) * 2
                    assert off // VROW == dt * 32 + j and off % VROW + 16 <= 2 * KKT


@pytest.mark.parametrize("D,H_kv,bs", [(128, 8, 256), (64, 4, 64), (128, 2, 1024)])
def test_register_loads_with_scalar_bases(D, H_kv, bs):
    threads = 512
    row_e = H_kv * D
    kchunks = KKT * D // 8 // threads
    VW = D // (threads // 32)
    rng = np.random.default_rng(7)
    for kmax in [1, 63, 64, 65, 200, 511, 1000]:
        n = (kmax + KKT - 1) // KKT
        for st in range(n):
            kb = st * KKT
            blk = int(rng.integers(0, 50))
            base_row = (blk * bs) + (kb & (bs - 1))  # the stage's first cache row
            kseen, vseen = set(), set()
            for t in range(threads):
                for i in range(kchunks):
                    c = t + i * threads
                    koff = (c // (D // 8)) * row_e + (c % (D // 8)) * 8
                    row, col = divmod(base_row * row_e + koff, row_e)
                    key = row - base_row
                    # inside the stage's block
                    assert row // bs == blk and 0 <= key < KKT
                    kseen.add((key, col))
                pair, dg = t % 32, t // 32
                for s in range(2):
                    voff = (2 * pair + s) * row_e + dg * VW
                    vlast = (kmax - 1 - kb) * row_e + dg * VW
                    off = voff if kb + 2 * pair + s < kmax else vlast
                    row, col = divmod(base_row * row_e + off, row_e)
                    assert row // bs == blk  # same block as the stage
                    key = row - base_row
                    want = min(kb + 2 * pair + s, kmax - 1) - kb
                    assert key == want
                    vseen.add((2 * pair + s, col))
            assert kseen == {(k, 8 * c) for k in range(KKT) for c in range(D // 8)}
            assert vseen == {(k, VW * g) for k in range(KKT) for g in range(threads // 32)}


def test_first_masked_stage():
    for off in range(0, 300, 7):
        for wmin in range(-70, 200, 3):
            diag_st = max(off + wmin + 1, 0) // KKT
            first = next(st for st in range(10000) if st * KKT + KKT - 1 > off + wmin)
            assert diag_st == first


def test_pipeline_buffers_and_blocks():
    for n in range(1, 12):
        for bs_stages in (1, 2, 4):  # blocks of 1, 2, 4 stages
            def block(stage):
                return 100 + stage // bs_stages

            kbuf, vbuf = [None, None], [None, None]
            # prologue
            kbuf[0], vbuf[0] = 0, 0
            kr_stage, vr_stage = min(1, n - 1), min(1, n - 1)
            kbuf[1] = kr_stage  # K of stage 1
            kr_stage = min(2, n - 1)
            bk = block(min(2, n - 1))
            raw_next = block(min(3, n - 1))
            for st in range(n):
                # the iteration reads K of st + 1 and V of st
                if st + 1 < n:
                    assert kbuf[(st + 1) & 1] == st + 1
                assert vbuf[st & 1] == st
                reads = {("k", (st + 1) & 1), ("v", st & 1)}
                # staging: block bookkeeping, stores, loads
                bk_now = raw_next
                raw_next = block(min(st + 4, n - 1))
                bv, bk = bk, bk_now
                assert ("k", st & 1) not in reads and ("v", (st + 1) & 1) not in reads
                kbuf[st & 1] = kr_stage
                vbuf[(st + 1) & 1] = vr_stage
                if st + 2 < n:
                    assert kr_stage == st + 2
                if st + 1 < n:
                    assert vr_stage == st + 1
                kr_stage, vr_stage = min(st + 3, n - 1), min(st + 2, n - 1)
                assert bk == block(kr_stage) and bv == block(vr_stage)
