"""Seeded synthetic input recipes (no attention arithmetic lives here).

Recipe shared by every workload:
  * one ``numpy.random.Generator(PCG64(seed))`` per workload, seed 0 unless
    given, draws in a fixed order (stated per function below);
  * values are float32 standard normals; bfloat16 inputs are those float32
    values rounded to nearest-even and carried as uint16 bit patterns, so the
    GPU and the oracle read bit-identical numbers;
  * the scale is float32(1 / sqrt(d)).

The pages measure on no public dataset or benchmark, so these synthetic draws
are the workloads themselves.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


E4M3_MAX = 448.0


def _e4m3_table():
    """Finite non-negative OCP E4M3 values and their codes, ascending (bias 7, 3 mantissa bits,
    exponent field 0 for subnormals, S.1111.111 reserved for NaN)."""
    vals, codes = [], []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
            codes.append((e << 3) | m)
    return np.array(vals), np.array(codes, dtype=np.uint8)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to the even code), saturating at +-448; returns bytes."""
    vals, codes = _e4m3_table()
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
    lo = hi - 1
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return np.where(np.signbit(x), out | np.uint8(0x80), out).astype(np.uint8)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor scaled E4M3: returns (bytes, scale) with x ~ scale * value(bytes), max |x| at 448."""
    amax = float(np.abs(x).max()) if x.size else 0.0
    scale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
    return f32_to_e4m3_bits(np.asarray(x, dtype=np.float64) / float(scale)), float(scale)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """float32 value of bfloat16 bit patterns (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str = "bf16"          # "bf16" (bf16 in/out, fp32 accumulate) or "f32"
    q_mult: float = 1.0          # power of two, so it commutes with bf16 rounding
    k_outlier_frac: float = 0.0  # fraction of K rows per (b, kv head) scaled up
    k_outlier_mult: float = 8.0
    window: int = 0              # causal sliding window width (0: none)
    n_global: int = 0            # leading keys every later query sees (with a window)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def visible_pairs(self) -> int:
        """Query-key pairs the mask leaves visible, per (b, h)."""
        if self.window:
            i = np.arange(self.N)
            in_window = np.minimum(i + 1, self.window)
            extra_global = np.clip(np.minimum(self.n_global, i - self.window + 1), 0, None)
            return int(in_window.sum() + extra_global.sum())
        return self.N * (self.N + 1) // 2 if self.causal else self.N * self.N


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    num_seqs: int
    H: int
    Hkv: int
    d: int
    L_lo: int
    L_hi: int
    page_size: int = 16
    num_pages: int = 40000

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def max_pages_per_seq(self) -> int:
        return -(-self.L_hi // self.page_size)


@dataclass(frozen=True)
class ChunkedPrefillWorkload:
    """A batch of sequences, each with ctx tokens cached in pages and a chunk of q_len new tokens."""
    name: str
    num_seqs: int
    H: int
    Hkv: int
    d: int
    ctx_lo: int
    ctx_hi: int
    q_len: int
    page_size: int = 16
    num_pages: int = 40000

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def max_pages_per_seq(self) -> int:
        return -(-(self.ctx_hi + self.q_len) // self.page_size)


WORKLOADS = {
    w.name: w
    for w in [
        PrefillWorkload("tiny_f32_b1h2n128d64", 1, 2, 2, 128, 64, causal=False, dtype="f32"),
        PrefillWorkload("causal_b4h16n1024d64", 4, 16, 16, 1024, 64, causal=True),
        PrefillWorkload("causal_gqa_b2h32kv8n4096d128", 2, 32, 8, 4096, 128, causal=True),
        PrefillWorkload("causal_gqa_long_b1h32kv8n16384d128", 1, 32, 8, 16384, 128, causal=True,
                        q_mult=4.0, k_outlier_frac=0.01, k_outlier_mult=8.0),
        DecodeWorkload("paged_decode_s64h32kv8d128", 64, 32, 8, 128, 512, 8192, 16, 40000),
        DecodeWorkload("paged_decode_s4h32kv8d128_short", 4, 32, 8, 128, 256, 1024, 16, 512),
        ChunkedPrefillWorkload("chunked_prefill_s16h32kv8d128_ctx0to4096_q512", 16, 32, 8, 128, 0, 4096, 512,
                               num_pages=6000),
        PrefillWorkload("fp8_causal_gqa_b2h32kv8n4096d128", 2, 32, 8, 4096, 128, causal=True, dtype="fp8"),
        PrefillWorkload("fp8_causal_gqa_long_b1h32kv8n16384d128", 1, 32, 8, 16384, 128, causal=True, dtype="fp8",
                        q_mult=4.0, k_outlier_frac=0.01, k_outlier_mult=8.0),
        PrefillWorkload("window_gqa_b1h32kv8n16384d128_w4096_g64", 1, 32, 8, 16384, 128, causal=True,
                        window=4096, n_global=64),
    ]
}


def prefill_inputs(w: PrefillWorkload, seed: int = 0):
    """Q [B,H,N,d], K, V [B,Hkv,N,d]; draw order Q, K, V, then outlier rows.

    Q is multiplied by ``q_mult``.  For each (b, kv head) in order,
    round(k_outlier_frac * N) distinct K rows chosen by the generator are
    multiplied by ``k_outlier_mult``.  Returns a dict with the arrays (uint16
    bfloat16 bits or float32) and the outlier row indices.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.N, w.d), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.N, w.d), dtype=np.float32)
    if w.q_mult != 1.0:
        q *= np.float32(w.q_mult)
    outliers = np.zeros((w.B, w.Hkv, 0), dtype=np.int64)
    n_out = int(round(w.k_outlier_frac * w.N))
    if n_out:
        outliers = np.zeros((w.B, w.Hkv, n_out), dtype=np.int64)
        for b in range(w.B):
            for g in range(w.Hkv):
                rows = rng.choice(w.N, size=n_out, replace=False)
                outliers[b, g] = rows
                k[b, g, rows] *= np.float32(w.k_outlier_mult)
    if w.dtype == "fp8":
        # per-tensor scaled E4M3; V is handed over transposed, [B, Hkv, d, N]
        q8, qs = quantize_e4m3(q)
        k8, ks = quantize_e4m3(k)
        v8, vs = quantize_e4m3(v)
        return {"q8": q8, "k8": k8, "vt8": np.ascontiguousarray(np.swapaxes(v8, -1, -2)), "q_scale": qs,
                "k_scale": ks, "v_scale": vs, "outliers": outliers, "scale": w.scale}
    if w.dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype}")
    return {"q": q, "k": k, "v": v, "outliers": outliers, "scale": w.scale}


def decode_inputs(w: DecodeWorkload, seed: int = 0, poison: bool = True, seq_lens=None,
                  block_table=None):
    """Paged-decode inputs.

    Draw order: sequence lengths (uniform integers in [L_lo, L_hi]), one
    permutation of the ``num_pages`` physical page ids, Q [S, H, d], then per
    sequence K [L, Hkv, d] followed by V [L, Hkv, d].  Sequence s takes the
    next ceil(L_s / page_size) ids of the permutation as its block table, so
    pages are distinct across all sequences; unused table entries are -1.
    Token t of sequence s is stored at page block_table[s, t // page_size],
    slot t % page_size of the [num_pages, page_size, Hkv, d] pools.  With
    ``poison`` every slot no token occupies (unreferenced pages and the tail
    of each last page) holds bfloat16 NaN.

    ``seq_lens`` / ``block_table`` may be given to override the drawn ones
    (then the corresponding draws are still made, to keep the order).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S, ps = w.num_seqs, w.page_size
    drawn = rng.integers(w.L_lo, w.L_hi, endpoint=True, size=S)
    lens = np.asarray(drawn if seq_lens is None else seq_lens, dtype=np.int32)
    perm = rng.permutation(w.num_pages)
    max_pages = w.max_pages_per_seq
    if block_table is None:
        need = -(-lens.astype(np.int64) // ps)
        if int(need.sum()) > w.num_pages:
            raise ValueError("page pool too small for the drawn lengths")
        bt = np.full((S, max_pages), -1, dtype=np.int32)
        cursor = 0
        for s in range(S):
            n = int(need[s])
            bt[s, :n] = perm[cursor:cursor + n]
            cursor += n
    else:
        bt = np.asarray(block_table, dtype=np.int32)
    q = f32_to_bf16_bits(rng.standard_normal((S, w.H, w.d), dtype=np.float32))
    fill = BF16_NAN if poison else np.uint16(0)
    k_pool = np.full((w.num_pages, ps, w.Hkv, w.d), fill, dtype=np.uint16)
    v_pool = np.full((w.num_pages, ps, w.Hkv, w.d), fill, dtype=np.uint16)
    for s in range(S):
        L = int(lens[s])
        kk = f32_to_bf16_bits(rng.standard_normal((L, w.Hkv, w.d), dtype=np.float32))
        vv = f32_to_bf16_bits(rng.standard_normal((L, w.Hkv, w.d), dtype=np.float32))
        t = np.arange(L)
        pages = bt[s, t // ps]
        k_pool[pages, t % ps] = kk
        v_pool[pages, t % ps] = vv
    return {"q": q, "k_cache": k_pool, "v_cache": v_pool, "block_table": bt,
            "seq_lens": lens, "scale": w.scale, "max_pages_per_seq": max_pages}


E4M3_NAN = np.uint8(0x7F)  # S.1111.111: the E4M3 ("fn") NaN pattern


def decode_inputs_fp8(w: DecodeWorkload, seed: int = 0, poison: bool = True, seq_lens=None, block_table=None):
    """FP8 (E4M3) paged-decode inputs: the draws of :func:`decode_inputs` (same order, same values),
    with the K and V pools quantized per tensor (scale = max |x| over the stored tokens / 448, each
    value rounded to the nearest E4M3 code, ties to even).  With ``poison`` every slot no token
    occupies holds the E4M3 NaN code.  Q stays bfloat16; adds ``k_scale`` and ``v_scale``."""
    a = decode_inputs(w, seed, poison=True, seq_lens=seq_lens, block_table=block_table)
    out = dict(a)
    for name, sname in (("k_cache", "k_scale"), ("v_cache", "v_scale")):
        x = bf16_bits_to_f32(a[name])
        used = ~np.isnan(x)  # drawn tokens are finite; every other slot was poisoned
        codes, scale = quantize_e4m3(np.where(used, x, np.float32(0)))
        codes[~used] = E4M3_NAN if poison else np.uint8(0)
        out[name], out[sname] = codes, scale
    return out


def chunked_prefill_inputs(w: ChunkedPrefillWorkload, seed: int = 0, poison: bool = True, ctx_lens=None,
                           q_lens=None):
    """Chunked-prefill inputs.

    Draw order: context lengths (uniform integers in [ctx_lo, ctx_hi]), one permutation of the
    ``num_pages`` physical page ids, then per sequence the context K [ctx, Hkv, d] and V, then the
    chunks' Q [T, H, d], K [T, Hkv, d] and V [T, Hkv, d] (T = the sum of the chunk lengths, each
    ``q_len`` unless ``q_lens`` is given).  Sequence s takes the next ceil((ctx_s + q_len_s) /
    page_size) ids of the permutation as its block table (room for the chunk to be appended);
    unused table entries are -1.  With ``poison`` every slot no context token occupies holds
    bfloat16 NaN, including the slots the chunk will be appended to.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S, ps = w.num_seqs, w.page_size
    drawn = rng.integers(w.ctx_lo, w.ctx_hi, endpoint=True, size=S)
    ctx = np.asarray(drawn if ctx_lens is None else ctx_lens, dtype=np.int32)
    ql = np.full(S, w.q_len, dtype=np.int32) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    perm = rng.permutation(w.num_pages)
    need = -(-(ctx.astype(np.int64) + ql) // ps)
    max_pages = max(1, int(need.max()) if S else 1)
    if int(need.sum()) > w.num_pages:
        raise ValueError("page pool too small for the drawn lengths")
    bt = np.full((S, max_pages), -1, dtype=np.int32)
    cursor = 0
    for s in range(S):
        n = int(need[s])
        bt[s, :n] = perm[cursor:cursor + n]
        cursor += n
    fill = BF16_NAN if poison else np.uint16(0)
    k_pool = np.full((w.num_pages, ps, w.Hkv, w.d), fill, dtype=np.uint16)
    v_pool = np.full((w.num_pages, ps, w.Hkv, w.d), fill, dtype=np.uint16)
    for s in range(S):
        L = int(ctx[s])
        kk = f32_to_bf16_bits(rng.standard_normal((L, w.Hkv, w.d), dtype=np.float32))
        vv = f32_to_bf16_bits(rng.standard_normal((L, w.Hkv, w.d), dtype=np.float32))
        t = np.arange(L)
        k_pool[bt[s, t // ps], t % ps] = kk
        v_pool[bt[s, t // ps], t % ps] = vv
    T = int(ql.sum())
    q = f32_to_bf16_bits(rng.standard_normal((T, w.H, w.d), dtype=np.float32))
    k_new = f32_to_bf16_bits(rng.standard_normal((T, w.Hkv, w.d), dtype=np.float32))
    v_new = f32_to_bf16_bits(rng.standard_normal((T, w.Hkv, w.d), dtype=np.float32))
    q_start = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    return {"q": q, "k_new": k_new, "v_new": v_new, "k_cache": k_pool, "v_cache": v_pool, "block_table": bt,
            "ctx_lens": ctx, "q_start": q_start, "scale": w.scale, "max_q_len": int(ql.max()) if S else 0}
