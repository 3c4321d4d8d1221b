"""CPU checks of the decode kernels' index arithmetic (csrc/decode.hip),
re-stated here and run on every lane, chunk position and item:

* matrix-core decode (compute_chunk_mf): the K rows and the V^T token pairs
  that each lane writes to its wave's LDS region are exactly what the MFMA
  operand reads expect: every K operand lane reads one token row's 8
  consecutive elements, the S^T accumulator's (tile, lane group, register)
  is the token the kernel masks and weights, and every V^T operand element
  is V[token][d] for the token the P^T operand holds at that k-index; no
  two writes overlap;
* dispatch order (decode_order_kernel): whatever order the rank atomics are
  taken in, the written order is a permutation of the work items (each
  (sequence, partition) once, -1 after them), never written outside the
  array, laid out as a snake over rounds of one item per CU.
"""

import numpy as np
import pytest


def mf_layout(D):
    LPT, U, ROW = D // 8, D // 16, 2 * D
    TILE = 16 * ROW
    VROW = 80
    VT = 2 * 16 * 2 * D  # V^T region after two K tiles
    TPI = 64 // LPT      # tokens per load instruction

    def token_of_load(u, r):
        return u * TPI + r

    mem = {}

    def put(addr, label):
        assert addr not in mem, "two writes to byte %d" % addr
        assert 0 <= addr < VT + D * VROW
        mem[addr] = label

    for lane in range(64):
        r, s = lane // LPT, lane % LPT
        for u in range(U):
            T = u >> 2 if D == 128 else r >> 2
            rho = 4 * r + (u & 3) if D == 128 else 4 * (r & 3) + u
            base = T * TILE + rho * ROW + ((s ^ (rho & (LPT - 1))) << 4)
            for e in range(8):
                put(base + 2 * e, ("K", token_of_load(u, r), 8 * s + e))
        for w in range(4):
            for e in range(2):
                d = 8 * s + 2 * w + e
                if D == 128:
                    base = VT + d * VROW + ((r ^ ((d >> 4) & 3)) << 4)
                    for u in range(8):  # bf16 element u of the 16 bytes
                        put(base + 2 * u, ("V", token_of_load(u, r), d))
                else:
                    base = VT + d * VROW + (((r & 3) ^ ((d >> 4) & 3)) << 4) + 8 * (r >> 2)
                    for u in range(4):
                        put(base + 2 * u, ("V", token_of_load(u, r), d))
    return mem, LPT, ROW, TILE, VROW, VT


@pytest.mark.parametrize("D", [128, 64])
def test_matrix_core_chunk_layout_agrees(D):
    mem, LPT, ROW, TILE, VROW, VT = mf_layout(D)

    def score_token(T, g, c):  # the token the kernel masks for (tile, group, register)
        return 16 * T + 4 * c + g if D == 128 else 8 * c + 4 * T + g

    seen_tokens = set()
    for T in range(2):
        row_token = {}
        for j in range(D // 32):
            for lane in range(64):
                g, i = lane >> 4, lane & 15
                base = T * TILE + i * ROW + (((4 * j + g) ^ (i & (LPT - 1))) << 4)
                labels = [mem[base + 2 * e] for e in range(8)]
                toks = {lab[1] for lab in labels}
                assert len(toks) == 1 and labels[0][0] == "K"
                assert [lab[2] for lab in labels] == [32 * j + 8 * g + e for e in range(8)]
                tok = toks.pop()
                assert row_token.setdefault(i, tok) == tok  # row i is one token throughout
        # the S^T accumulator: lane (g, i), register c holds tile row 4g + c
        for g in range(4):
            for c in range(4):
                assert row_token[4 * g + c] == score_token(T, g, c)
                seen_tokens.add(score_token(T, g, c))
    assert seen_tokens == set(range(32))
    # V^T operand of tile mt: lane (g, i) reads d = 16 mt + i, k-index 8 g + q,
    # which must be V[token][d] for the token P^T holds there (q = 4 T + c)
    for mt in range(D // 16):
        for lane in range(64):
            g, i = lane >> 4, lane & 15
            d = 16 * mt + i
            base = VT + d * VROW + ((g ^ (mt & 3)) << 4)
            for q in range(8):
                T, c = q >> 2, q & 3
                assert mem[base + 2 * q] == ("V", score_token(T, g, c), d)


# ---------------------------------------------------------- dispatch order

def split_parts(n, P, max_parts):
    nn = min(n, max_parts * P)
    return nn, (nn + P - 1) // P


def len_bucket(length, P, buckets=32):
    return 1 + ((length - 1) * buckets) // P


def dispatch_slot(r, rnd, max_items):
    k = r // rnd
    start = k * rnd
    ln = min(rnd, max_items - start)
    return start + ln - 1 - (r - start) if k & 1 else r


def emulate_order(lens, P, max_parts, rnd, rng):
    """The rank assignment with the threads' atomics taken in a random order."""
    max_items = len(lens) * max_parts
    NB = 33
    items = {}
    for s, n in enumerate(lens):
        if n == 0:
            items[s] = (0, 0, 0)
            continue
        nn, k = split_parts(n, P, max_parts)
        items[s] = (k - 1, 32, len_bucket(nn - (k - 1) * P, P))
    counts = [0] * NB
    for s in rng.permutation(len(lens)):
        bulk, kb, kl = items[s]
        if bulk:
            counts[kb] += bulk
        counts[kl] += 1
    nxt, run = [0] * NB, 0
    for k in range(NB - 1, -1, -1):
        nxt[k], run = run, run + counts[k]
    total = run
    order = [None] * max_items
    for s in rng.permutation(len(lens)):  # a random interleaving of the atomics
        bulk, kb, kl = items[s]
        if bulk:
            pos = nxt[kb]
            nxt[kb] += bulk
            for j in range(bulk):
                slot = dispatch_slot(pos + j, rnd, max_items)
                assert 0 <= slot < max_items and order[slot] is None
                order[slot] = (j, s)
        pos = nxt[kl]
        nxt[kl] += 1
        slot = dispatch_slot(pos, rnd, max_items)
        assert 0 <= slot < max_items and order[slot] is None
        order[slot] = (bulk, s)
    for r in range(total, max_items):
        slot = dispatch_slot(r, rnd, max_items)
        assert order[slot] is None
        order[slot] = -1
    return order, items, total


@pytest.mark.parametrize("seed", range(12))
def test_dispatch_order_is_a_permutation(seed):
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 600))
    lens = rng.integers(0, 9000, size=n)
    lens[rng.random(n) < 0.1] = 0
    P = 256 * int(rng.choice([1, 2, 4, 8, 16]))
    max_parts = max(1, -(-int(lens.max()) // P))
    rnd = int(rng.choice([64, 128, 256]))
    order, items, total = emulate_order(lens, P, max_parts, rnd, rng)
    assert None not in order
    want = set()
    for s, n_ in enumerate(lens):
        k = split_parts(int(n_), P, max_parts)[1] if n_ else 1
        want.update((j, s) for j in range(k))
    got = [e for e in order if e != -1]
    assert len(got) == len(want) == total and set(got) == want
    # longest first: ranks in bucket order (full partitions, then by length)
    ranks = {}
    for r in range(total):
        ranks[order[dispatch_slot(r, rnd, max_items=len(order))]] = r
    by_rank = sorted(want, key=lambda e: ranks[e])
    buckets = []
    for j, s in by_rank:
        bulk, kb, kl = items[s]
        buckets.append(kb if j < bulk else kl)
    assert buckets == sorted(buckets, reverse=True)


# ---- stream grid (decode_stream_kernel, stream_locate)

def stream_schedule(units, slots, chunk, min_piece_tokens=256):
    """stream_locate's schedule restated: units C, W equal grabs; lo(j) and
    grab_of(x) as Sched computes them."""
    C = int(sum(units))
    W = max(1, min(slots, C // max(1, min_piece_tokens // chunk)))
    return C, W, (lambda j: j * C // W), (lambda x: ((x + 1) * W - 1) // C)


def find_sequence(units, x):
    """stream_locate's search restated: 64 lengths per step, a scan, then
    the first lane whose sequence ends past x."""
    ns = len(units)
    S = 0
    for base in range(0, ns, 64):
        u = np.zeros(64, dtype=np.int64)
        m = min(64, ns - base)
        u[:m] = units[base:base + m]
        incl = np.cumsum(u)
        past = np.nonzero(S + incl > x)[0]
        if past.size:
            l = int(past[0])
            return base + l, S + int(incl[l] - u[l])
        S += int(incl[-1])
    raise AssertionError("x past the last unit")


PIECE_COST = 2  # kPieceCost: units of fixed cost placed before each sequence's units


def stream_walk(lengths, slots, chunk, piece_cost=PIECE_COST):
    """Every grab's pieces as its wave visits them: (grab, sequence, token
    start, token end, direct, partial row, first, last). Grabs split the
    batch's cost (each sequence: piece_cost, then its units); a grab's
    piece of a sequence is its share of that sequence's units, none if the
    grab holds only the sequence's fixed cost."""
    units = [1 if n <= 0 else -(-n // chunk) for n in lengths]
    cost = [u + piece_cost for u in units]
    C, W, lo, grab_of = stream_schedule(cost, slots, chunk)
    pieces = []
    for j in range(W):
        lo_j, hi_j = lo(j), lo(j + 1)
        assert lo_j < hi_j, "an empty grab"
        b, S = find_sequence(cost, lo_j)
        u = lo_j
        while u < hi_j and b < len(lengths):
            n, c = lengths[b], units[b]
            f = S + piece_cost
            u1 = min(hi_j, f + c)
            p0 = max(u, f)
            if p0 < u1:
                first, last = grab_of(f), grab_of(f + c - 1)
                pieces.append((j, b, (p0 - f) * chunk, min((u1 - f) * chunk, n),
                               first == last, j + b, first, last))
            u = u1
            S = f + c
            b += 1
    return pieces, W, units


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("chunk", [16, 32])
def test_stream_grabs_cover_every_token_once(seed, chunk):
    rng = np.random.default_rng(seed)
    kind = seed % 5
    ns = [1, 7, 64, 300, 700][kind]
    if kind == 0:
        lengths = [int(rng.integers(0, 40000))]
    elif seed % 2:
        lengths = [int(x) for x in rng.integers(0, 5000, size=ns)]
    else:  # one long sequence among short ones, some empty rows
        lengths = [int(x) for x in rng.integers(0, 120, size=ns)]
        lengths[int(rng.integers(0, ns))] = 8192
    slots = int(rng.choice([1, 3, 64, 256, 1024]))
    pieces, W, units = stream_walk(lengths, slots, chunk)
    covered = {}
    rows = set()
    per_seq = {}
    for (j, b, s, e, direct, row, first, last) in pieces:
        assert first <= j <= last < W
        assert s % chunk == 0  # a piece starts on a chunk boundary
        for t in range(s, e):
            assert (b, t) not in covered, "token read twice"
            covered[(b, t)] = j
        per_seq.setdefault(b, []).append((j, direct, row, first, last))
        if not direct:
            assert row not in rows, "two pieces share a partial row"
            rows.add(row)
            assert 0 <= row < slots + len(lengths) - 1  # the workspace's rows
    assert len(covered) == sum(lengths)
    for b, n in enumerate(lengths):
        ps = sorted(per_seq[b])
        first, last = ps[0][3], ps[0][4]
        assert [p[0] for p in ps] == list(range(first, last + 1))  # one piece per grab
        assert all(p[1] == (first == last) for p in ps)
        if n == 0:
            assert len(ps) == 1 and ps[0][1]  # an empty row: one direct piece (its zeros)


def test_stream_last_arriver_merges_once_in_any_arrival_order():
    """The counter protocol: pieces of a split sequence arrive in any order;
    exactly the arrival that sees count == pieces - 1 merges, and it leaves
    the counter at zero; only a grab's first or last piece can complete a
    sequence."""
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(1, 9000, size=40)]
    pieces, W, _ = stream_walk(lengths, 256, 16)
    by_grab = {}
    for p in pieces:
        by_grab.setdefault(p[0], []).append(p)
    for ps in by_grab.values():
        for p in ps[1:-1]:
            assert p[4], "a middle piece of a grab is a whole sequence"
    split = {}
    for p in pieces:
        if not p[4]:
            split.setdefault(p[1], []).append(p)
    assert split
    for b, ps in split.items():
        for trial in range(5):
            order = rng.permutation(len(ps))
            cnt, merges = 0, 0
            for i in order:
                first, last = ps[i][6], ps[i][7]
                before, cnt = cnt, cnt + 1
                if before == last - first:
                    merges += 1
                    cnt = 0
            assert merges == 1 and cnt == 0


@pytest.mark.parametrize("tpi,u_loads", [(2, 8), (4, 8), (8, 4), (1, 8), (4, 4)])
def test_fused_store_lanes_hold_the_newest_token(tpi, u_loads):
    """decode_piece's tail with the fused store: load u of lane row r reads
    tail token min(u * TPI + r, e) (e = the newest token's index in the
    tail), and the lanes of row max(0, e - (U-1) * TPI) write the newest
    token from their last load: that load must hold token e, for every e
    the tail can end on."""
    chunk = tpi * u_loads
    for e in range(chunk):
        r = max(0, e - (u_loads - 1) * tpi)
        assert 0 <= r < tpi
        assert min((u_loads - 1) * tpi + r, e) == e
        # and the newest token is the one the tail masks last: every load
        # of a valid token index reads it at most once per row
        seen = {min(u * tpi + row, e) for u in range(u_loads) for row in range(tpi)}
        assert seen == set(range(e + 1))
