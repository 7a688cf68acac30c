"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing kernel outputs with the oracle at the stated tolerances."""

from __future__ import annotations

import numpy as np
import torch

from workloads import bf16_bits_to_f32

# Acceptance bars (elementwise over O; LSE over all rows)
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5
LSE_MAX_ABS = 1e-3


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> bf16 tensor on cuda:0 (bit-identical)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")


def dev_i32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")


def host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device tensor (bf16 or fp32)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def assert_close_bf16(got: np.ndarray, want: np.ndarray, what: str = "O") -> dict:
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in kernel output"
    err = np.abs(got - want)
    stats = {"max_abs": float(err.max(initial=0.0)), "mean_abs": float(err.mean()) if err.size else 0.0}
    assert stats["max_abs"] <= BF16_MAX_ABS, f"{what}: max |err| {stats['max_abs']:.3e} > {BF16_MAX_ABS}"
    assert stats["mean_abs"] <= BF16_MEAN_ABS, f"{what}: mean |err| {stats['mean_abs']:.3e} > {BF16_MEAN_ABS}"
    return stats


def assert_close_f32(got: np.ndarray, want: np.ndarray, what: str = "O") -> dict:
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in kernel output"
    err = float(np.abs(got - want).max(initial=0.0))
    assert err <= F32_MAX_ABS, f"{what}: max |err| {err:.3e} > {F32_MAX_ABS}"
    return {"max_abs": err}


def assert_close_lse(got: np.ndarray, want: np.ndarray) -> dict:
    both_inf = np.isneginf(got) & np.isneginf(want)
    g, w = got[~both_inf], want[~both_inf]
    assert np.all(np.isfinite(g)), "LSE: non-finite values where the oracle is finite"
    err = float(np.abs(g - w).max(initial=0.0))
    assert err <= LSE_MAX_ABS, f"LSE: max |err| {err:.3e} > {LSE_MAX_ABS}"
    return {"lse_max_abs": err}


def sample_rows(B, H, N, n_random, seed, tile=64):
    """Rows (b, h, i) to check at full size: sequence ends, tile edges and seeded random picks."""
    rng = np.random.default_rng(seed)
    edges = sorted({0, 1, tile - 1, tile, 2 * tile - 1, 2 * tile, N // 2, N - tile, N - 2, N - 1} & set(range(N)))
    rows = [(b, h, i) for b in {0, B - 1} for h in {0, H - 1, H // 2} for i in edges]
    rows += [(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))) for _ in range(n_random)]
    return sorted(set(rows))


def zero_query_expected(v, H, causal, window=0, n_global=0):
    """Closed form of masked attention (softmax of the scaled scores plus the mask, times V: "Fast Attention
    Kernels and Operator Fusion", "FlashAttention-Style Kernels") when Q = 0: every visible key scores 0, so
    its weight is one over the number n_i of keys row i sees, O_i is the mean of those V rows and
    LSE_i = ln n_i.  v: float64 [B, Hkv, N, d] (the V the kernel reads); returns O [B, H, N, d] and LSE
    [B, H, N], query head h reading KV head h // (H / Hkv).  The mask is causal (optionally a sliding
    window of width ``window`` plus ``n_global`` leading keys) or none."""
    B, Hkv, N, d = v.shape
    pre = np.concatenate([np.zeros((B, Hkv, 1, d)), np.cumsum(v, axis=2)], axis=2)  # pre[k] = sum of rows < k
    i = np.arange(N)
    if not causal:
        tot = np.broadcast_to(pre[:, :, N:N + 1], (B, Hkv, N, d))
        cnt = np.full(N, float(N))
    elif window <= 0:
        tot = pre[:, :, 1:]
        cnt = (i + 1).astype(np.float64)
    else:
        lo = np.maximum(0, i - window + 1)             # the window: keys lo .. i
        gl = np.minimum(n_global, lo)                  # global tokens left of the window: keys 0 .. gl - 1
        tot = pre[:, :, i + 1] - pre[:, :, lo] + pre[:, :, gl]
        cnt = (i + 1 - lo + gl).astype(np.float64)
    o = tot / cnt[None, None, :, None]
    o = np.repeat(o, H // Hkv, axis=1)                  # query head h reads KV head h // (H / Hkv)
    lse = np.broadcast_to(np.log(cnt), (B, H, N))
    return o, lse



def decode_zero_query_expected(v_rows_f64, v_cache, block_table, seq_lens, H):
    """Closed form of paged decode (one query per sequence over its cached keys, gathered through the
    block table: "Fast Attention Kernels and Operator Fusion", "Paged Attention Kernels") when q = 0:
    every cached key scores 0, so each head's output is the mean of its KV head's V rows over the
    sequence's L tokens and LSE = ln L (an empty sequence gives O = 0 and LSE = -inf).  v_cache is
    the raw pool [num_pages, page_size, Hkv, d]; v_rows_f64 turns gathered raw rows into float64
    values.  Returns O [S, H, d] and LSE [S, H]."""
    num_pages, page_size, Hkv, d = v_cache.shape
    S = len(seq_lens)
    o = np.zeros((S, H, d))
    lse = np.full((S, H), -np.inf)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        pages = np.asarray(block_table[s][: -(-L // page_size)])
        rows = v_rows_f64(v_cache[pages]).reshape(-1, Hkv, d)[:L]  # token t at page t // page_size
        o[s] = np.repeat(rows.mean(axis=0), H // Hkv, axis=0)      # query head h reads KV head h // group
        lse[s] = np.log(L)
    return o, lse
