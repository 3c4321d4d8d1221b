"""Helpers shared by the GPU parity tests (host <-> device bf16 bits,
error metrics, NaN poisoning of unused pool rows)."""

import numpy as np

import oracle

MAX_ABS = 1e-2   # attention tolerance vs the fp64 oracle (bf16 in, fp32 accumulate)
MEAN_ABS = 1e-3

NAN_BF16 = np.uint16(0x7FC1)


def dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def dev_i32(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    return oracle.bf16_bits_to_f64(host_bits(t))


def err_stats(got: np.ndarray, ref: np.ndarray):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())


def assert_close(got, ref, what=""):
    mx, mean = err_stats(got, ref)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, "%s: max abs %.3g, mean abs %.3g" % (what, mx, mean)
    return mx, mean


def poison_unused(k_cache, v_cache, block_tables, n_tokens, block_size):
    """Copies of the caches with every row outside tokens 0..n_tokens[b]-1 of
    the sequences set to NaN (results must not depend on those rows)."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    used = oracle.used_rows(block_tables, n_tokens, block_size)
    mask = np.ones(kc.shape[0] * kc.shape[1], dtype=bool)
    mask[used] = False
    kc.reshape(-1, *kc.shape[2:])[mask] = NAN_BF16
    vc.reshape(-1, *vc.shape[2:])[mask] = NAN_BF16
    return kc, vc


def check_whole_output(kind: str, case_name: str, out, block_size: int = 256):
    """Compare every row of a named workload's GPU output (a bf16 tensor, or
    its values as float64) with the oracle,
    computed by tests/oracle_ref.py in a child process (a fresh interpreter
    without a GPU context, with a pool of worker processes). Returns the
    error statistics; asserts the attention tolerance."""
    import json
    import os
    import subprocess
    import sys
    import tempfile
    if isinstance(out, np.ndarray):  # float64 values read back from bf16 (exact)
        u = out.astype(np.float32).view(np.uint32)
        bits = (u >> np.uint32(16)).astype(np.uint16)
        assert np.array_equal(oracle.bf16_bits_to_f64(bits), out, equal_nan=True)
    else:
        bits = host_bits(out)
    here = os.path.dirname(os.path.abspath(__file__))
    with tempfile.TemporaryDirectory(prefix="pa_ref_") as tmp:
        src = os.path.join(tmp, "gpu.npy")
        dst = os.path.join(tmp, "stats.json")
        np.save(src, bits)
        print("  whole-output oracle: %s %s (block %d), %d rows" % (
            kind, case_name, block_size, bits.shape[0]), flush=True)
        r = subprocess.run([sys.executable, os.path.join(here, "oracle_ref.py"), kind, case_name,
                            src, dst, "--block-size", str(block_size)],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                           timeout=900)
        if r.returncode != 0:
            raise AssertionError("oracle_ref failed (%d):\n%s" % (r.returncode, r.stdout[-3000:]))
        with open(dst) as f:
            rec = json.load(f)
    print("  parity %s %s (every row, %d elements, oracle %.1f s on %d workers): max abs %.3g "
          "mean abs %.3g (max |ref| %.3g)" % (kind, case_name, rec["elements"], rec["seconds"],
                                              rec["workers"], rec["max_abs"], rec["mean_abs"],
                                              rec["max_abs_ref"]), flush=True)
    assert rec["finite"], "non-finite output: %s" % rec
    assert rec["max_abs"] <= MAX_ABS and rec["mean_abs"] <= MEAN_ABS, (
        "%s %s: max abs %.3g at %s (got %.6g, ref %.6g), mean abs %.3g" % (
            kind, case_name, rec["max_abs"], rec["argmax"], rec["got_at_max"], rec["ref_at_max"],
            rec["mean_abs"]))
    return rec
