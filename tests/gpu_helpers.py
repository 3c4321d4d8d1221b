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
