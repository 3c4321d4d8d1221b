"""Replays the block-manager trace fixture against any allocator exposing the
oracle's interface (can_allocate, allocate, deallocate, can_append,
may_append, hash_blocks, state) over the oracle's Seq objects."""

import json
import os

import numpy as np

from oracle.block_manager import Seq, chained_hash

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_manager_trace.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def tokens(rng, n):
    return rng.integers(0, 150000, size=n).tolist()


def index_of(seqs, entries):
    """The expected prefix index as {chained hash: block id}."""
    out = {}
    for name, i, bid in entries:
        seq = seqs[name]
        h = None
        for j in range(i + 1):
            h = chained_hash(seq.block(j), h)
        out[h] = bid
    return out


def run_op(bm, seqs, op, rng):
    kind, name = op[0], op[1]
    seq = seqs[name]
    if kind == "prefill":
        n = op[2]
        if not seq.block_table:
            k = bm.can_allocate(seq)
            assert k >= 0, (name, k)
            bm.allocate(seq, k)
        bm.hash_blocks(seq, n)
        seq.num_cached_tokens += n
        if seq.num_cached_tokens == len(seq):
            seq.token_ids.append(tokens(rng, 1)[0])
    elif kind in ("decode", "decode_preempting"):
        if kind == "decode_preempting":
            victim = seqs[op[2]]
            while not bm.can_append(seq):
                bm.deallocate(victim)
        assert bm.can_append(seq), name
        bm.may_append(seq)
        bm.hash_blocks(seq, 1)
        seq.num_cached_tokens += 1
        seq.token_ids.append(tokens(rng, 1)[0])
    elif kind == "can_allocate":
        assert bm.can_allocate(seq) == op[2], (name, op[2])
    else:
        raise ValueError(kind)


def replay_trace(make_bm, seed=0, stop_after=None):
    """Runs the trace; checks every printed state. Returns (bm, seqs)."""
    g = load()["trace"]
    rng = np.random.default_rng(seed)
    bm = make_bm(g["num_blocks"], g["block_size"])
    seqs = {n: Seq(tokens(rng, L), g["block_size"]) for n, L in g["prompts"].items()}
    for rd in g["rounds"]:
        for op in rd["ops"]:
            run_op(bm, seqs, op, rng)
        st = bm.state()
        assert st["free"] == rd["free"], ("round", rd["round"], st["free"])
        for name, table in rd.get("tables", {}).items():
            assert seqs[name].block_table == table, ("round", rd["round"], name)
        if "index" in rd:
            assert st["index"] == index_of(seqs, rd["index"]), ("round", rd["round"])
        assert set(st["used"]) == {b for b, c in enumerate(st["ref_count"]) if c > 0}
        if stop_after == rd["round"]:
            break
    return bm, seqs


def check_prefix_hit(make_bm, seed=0):
    g = load()["prefix_hit"]
    bm, seqs = replay_trace(make_bm, seed, stop_after=g["after_round"])
    rng = np.random.default_rng(seed + 1)
    src = seqs[g["shares_first_tokens_with"]]
    r7 = Seq(src.token_ids[:g["shared_tokens"]] + tokens(rng, g["length"] - g["shared_tokens"]),
             src.block_size)
    assert bm.can_allocate(r7) == g["can_allocate"]
    bm.allocate(r7, g["can_allocate"])
    assert r7.block_table == g["table"]
    assert bm.state()["ref_count"][0] == g["ref_count_block0"]
    assert r7.num_cached_tokens == g["num_cached_tokens"]


def check_shared_blocks(make_bm, seed=0):
    g = load()["shared_blocks"]
    rng = np.random.default_rng(seed)
    bs = g["block_size"]
    a = Seq(tokens(rng, g["A_blocks"] * bs), bs)
    b = Seq(a.token_ids[:g["B_shared_blocks"] * bs] +
            tokens(rng, (g["B_blocks"] - g["B_shared_blocks"]) * bs), bs)
    bm = make_bm(g["num_blocks"], bs)
    for s in (a, b):
        k = bm.can_allocate(s)
        bm.allocate(s, k)
        bm.hash_blocks(s, len(s) - s.num_cached_tokens)
        s.num_cached_tokens = len(s)
    st = bm.state()
    assert a.block_table == g["tables"]["A"] and b.block_table == g["tables"]["B"]
    assert st["free"] == g["free"] and st["ref_count"] == g["ref_count"]
    assert st["index"] == index_of({"A": a, "B": b}, g["index"])


def check_remainder_after_hit(bm_cls):
    """A 500-token prompt whose first 256 tokens were hashed by an earlier
    prompt: one cached block, so 500 - 256 = 244 tokens are left to prefill
    ("12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.9 Scheduler,
    the num_tokens example)."""
    rng = np.random.default_rng(5)
    first = tokens(rng, 256)
    bm = bm_cls(8, 256)
    a = Seq(first + tokens(rng, 44), 256)
    bm.allocate(a, bm.can_allocate(a))
    bm.hash_blocks(a, len(a))
    a.num_cached_tokens = len(a)
    b = Seq(first + tokens(rng, 244), 256)
    hits = bm.can_allocate(b)
    assert hits == 1
    bm.allocate(b, hits)
    assert b.num_cached_tokens == 256 and len(b) - b.num_cached_tokens == 244
    assert b.block_table[0] == a.block_table[0] and len(b.block_table) == 2
