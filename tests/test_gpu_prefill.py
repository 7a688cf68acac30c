"""GPU parity of attn_fwd / attn_fwd_f32 (through the C ABI) against the float64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_attention_attn_amd as paa
import oracle_pool
from gpu_util import (assert_close_bf16, assert_close_f32, assert_close_lse, dev_bf16, dev_f32, host_f64,
                      zero_query_expected)
from workloads import WORKLOADS, PrefillWorkload, f32_to_bf16_bits, prefill_inputs

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _run_bf16(a, w):
    q, k, v = dev_bf16(a["q"]), dev_bf16(a["k"]), dev_bf16(a["v"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    o, _ = paa.attn_fwd(q, k, v, w.causal, a["scale"], lse=lse)
    torch.cuda.synchronize()
    return host_f64(o), lse.cpu().numpy().astype(np.float64)


# Small shapes: the oracle computes every output.  They span several 64-key
# tiles and 128-row query tiles, ragged ends, every head-grouping branch and
# both head dims.
SMALL = [
    (2, 4, 2, 300, 64, True), (2, 4, 2, 300, 64, False),
    (1, 8, 2, 257, 128, True), (1, 8, 2, 257, 128, False),
    (1, 4, 4, 200, 128, True), (1, 6, 2, 131, 64, True),   # group 3 -> one head per workgroup
    (1, 8, 1, 190, 128, True),                               # group 8 -> two head subgroups
    (1, 2, 1, 1, 64, True), (1, 2, 2, 17, 128, False), (1, 2, 2, 64, 64, True), (3, 2, 1, 129, 128, True),
    # d = 128 small grids take the split-key kernel: one key tile (group B idle), an even and an odd
    # number of key tiles, a row block ending exactly on a tile edge, no mask
    (1, 4, 4, 1, 128, True), (1, 4, 1, 63, 128, True), (2, 4, 2, 128, 128, True), (1, 4, 2, 192, 128, True),
    (1, 8, 2, 511, 128, False), (1, 3, 3, 96, 128, True),
    # d = 64 short sequences: keys only in the first half of the one tile, one and a half tiles,
    # group 4, no mask
    (1, 2, 2, 20, 64, True), (1, 2, 2, 20, 64, False), (1, 4, 4, 96, 64, True), (2, 8, 2, 160, 64, True),
    (1, 4, 1, 65, 64, False),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", SMALL)
def test_bf16_small_full_parity(B, H, Hkv, N, d, causal):
    w = PrefillWorkload("small", B, H, Hkv, N, d, causal)
    _announce(f"attn_fwd bf16 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    a = prefill_inputs(w, seed=N + d)
    o, lse = _run_bf16(a, w)
    ro, rl = oracle.attention(a["q"], a["k"], a["v"], causal, a["scale"])
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_bf16_peaked_scores_small():
    """Scores with a large range (Q x4, 1% of K rows x8) at a size the oracle covers fully."""
    w = PrefillWorkload("peaked", 1, 8, 2, 520, 128, True, q_mult=4.0, k_outlier_frac=0.01)
    _announce("attn_fwd bf16 peaked N520")
    a = prefill_inputs(w, seed=5)
    o, lse = _run_bf16(a, w)
    ro, rl = oracle.attention(a["q"], a["k"], a["v"], True, a["scale"])
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


@pytest.mark.parametrize("N,d", [(1500, 128), (700, 64)])
def test_bf16_rising_scores_and_deep_keys(N, d):
    """Scores that keep rising along the sequence (each key a little larger than the one before, so every
    row's maximum keeps moving and the kernels' reference must move many times), keys far below the
    row's maximum (whose weights underflow), and a row-block whose first tile holds only such keys:
    every element against the oracle, both kernels (d=128 ping-pong grid shape too small, so the
    split-key kernel; d=64 the lock-step kernel)."""
    rng = np.random.default_rng(80 + d)
    B, H, Hkv = 1, 4, 1
    q = 4.0 * rng.standard_normal((B, H, N, d))
    growth = np.linspace(1.0, 12.0, N)[:, None]
    k = rng.standard_normal((B, Hkv, N, d)) * growth
    k[0, 0, 10:40] *= -20.0  # very low scores for rows whose q aligns with the bulk
    v = rng.standard_normal((B, Hkv, N, d))
    a = {"q": f32_to_bf16_bits(q.astype(np.float32)), "k": f32_to_bf16_bits(k.astype(np.float32)),
         "v": f32_to_bf16_bits(v.astype(np.float32)), "scale": float(np.float32(1.0 / np.sqrt(d)))}
    w = PrefillWorkload("rising", B, H, Hkv, N, d, True)
    _announce(f"attn_fwd rising scores N{N} d{d}")
    o, lse = _run_bf16(a, w)
    ro, rl = oracle.attention(a["q"], a["k"], a["v"], True, a["scale"])
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_bf16_causal_mha_b4h16n1024d64_full():
    """Causal self-attention B=4, H=16, N=1024, d=64: every output element against the oracle."""
    w = WORKLOADS["causal_b4h16n1024d64"]
    _announce(w.name)
    a = prefill_inputs(w, seed=0)
    o, lse = _run_bf16(a, w)
    ro, rl = oracle.attention(a["q"], a["k"], a["v"], True, a["scale"])
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["causal_gqa_b2h32kv8n4096d128", "causal_gqa_long_b1h32kv8n16384d128"])
def test_bf16_full_size_whole(name):
    """Full-size causal GQA prefill: every element of O and LSE against the oracle (one oracle call per
    (batch entry, head), run in a thread pool)."""
    w = WORKLOADS[name]
    _announce(name)
    a = prefill_inputs(w, seed=0)
    o, lse = _run_bf16(a, w)
    ro, rl = oracle_pool.attention(a["q"], a["k"], a["v"], True, a["scale"])
    st = assert_close_bf16(o, ro)
    st.update(assert_close_lse(lse, rl))
    _announce(f"{name}: {st}")


def test_bf16_deterministic_and_linear_memory():
    """Two runs are bitwise equal; the call allocates nothing (peak memory = inputs + outputs)."""
    w = PrefillWorkload("det", 1, 8, 2, 2048, 128, True)
    a = prefill_inputs(w, seed=2)
    q, k, v = dev_bf16(a["q"]), dev_bf16(a["k"]), dev_bf16(a["v"])
    o1, lse1 = torch.empty_like(q), torch.empty((1, 8, 2048), dtype=torch.float32, device="cuda:0")
    o2, lse2 = torch.empty_like(q), torch.empty_like(lse1)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    paa.attn_fwd(q, k, v, True, a["scale"], out=o1, lse=lse1)
    paa.attn_fwd(q, k, v, True, a["scale"], out=o2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_f32_tiny_workload_parity():
    """fp32 path, B=1, H=2, N=128, d=64, non-causal, seed 0: max |err| <= 1e-5."""
    w = WORKLOADS["tiny_f32_b1h2n128d64"]
    a = prefill_inputs(w, seed=0)
    q, k, v = dev_f32(a["q"]), dev_f32(a["k"]), dev_f32(a["v"])
    lse = torch.empty((1, 2, 128), dtype=torch.float32, device="cuda:0")
    o, _ = paa.attn_fwd_f32(q, k, v, False, a["scale"], lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(a["q"], a["k"], a["v"], False, a["scale"])
    assert_close_f32(host_f64(o), ro)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [(1, 2, 2, 128, 64, True), (2, 4, 2, 100, 128, True),
                                                 (1, 3, 1, 70, 64, False), (1, 2, 1, 1, 128, True)])
def test_f32_small_parity(B, H, Hkv, N, d, causal):
    w = PrefillWorkload("f32", B, H, Hkv, N, d, causal, dtype="f32")
    a = prefill_inputs(w, seed=7)
    q, k, v = dev_f32(a["q"]), dev_f32(a["k"]), dev_f32(a["v"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o, _ = paa.attn_fwd_f32(q, k, v, causal, a["scale"], lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(a["q"], a["k"], a["v"], causal, a["scale"])
    assert_close_f32(host_f64(o), ro)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)


def test_empty_and_argument_errors():
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda:0")
    o, _ = paa.attn_fwd(q, q[:, :1], q[:, :1], True)  # B = 0: valid, nothing launched
    assert o.shape == q.shape
    x = torch.zeros((1, 2, 16, 96), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError, match="head dimension"):
        paa.attn_fwd(x, x, x, True)
    y = torch.zeros((1, 2, 16, 64), dtype=torch.float16, device="cuda:0")
    with pytest.raises(TypeError):
        paa.attn_fwd(y, y, y, True)
    z = torch.zeros((1, 2, 64, 16), dtype=torch.bfloat16, device="cuda:0").transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        paa.attn_fwd(z, z, z, True)
    k3 = torch.zeros((1, 3, 16, 64), dtype=torch.bfloat16, device="cuda:0")
    q4 = torch.zeros((1, 4, 16, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(RuntimeError, match="invalid shape"):
        paa.attn_fwd(q4, k3, k3, True)


# ---- sliding window + global tokens (attn_fwd_window) ----

def _run_window(a, w, window, n_global):
    q, k, v = dev_bf16(a["q"]), dev_bf16(a["k"]), dev_bf16(a["v"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    o, _ = paa.attn_fwd_window(q, k, v, window, n_global, a["scale"], lse=lse)
    torch.cuda.synchronize()
    return host_f64(o), lse.cpu().numpy().astype(np.float64)


# window below one key tile, across tiles, with and without global tokens, window 1, window >= N
WINDOW_SMALL = [
    (1, 4, 2, 300, 64, 16, 0), (1, 4, 2, 300, 64, 16, 5), (2, 8, 2, 333, 128, 100, 0),
    (1, 8, 2, 333, 128, 100, 70), (1, 4, 4, 257, 128, 1, 0), (1, 6, 2, 129, 64, 1, 1),
    (1, 8, 1, 200, 128, 64, 64), (1, 2, 2, 90, 64, 500, 3), (1, 4, 1, 520, 128, 130, 2),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,window,n_global", WINDOW_SMALL)
def test_window_small_full_parity(B, H, Hkv, N, d, window, n_global):
    w = PrefillWorkload("win", B, H, Hkv, N, d, True)
    _announce(f"attn_fwd_window B{B} H{H} Hkv{Hkv} N{N} d{d} window={window} n_global={n_global}")
    a = prefill_inputs(w, seed=N + window)
    o, lse = _run_window(a, w, window, n_global)
    ro, rl = oracle.attention_window(a["q"], a["k"], a["v"], window, n_global, a["scale"])
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_window_covering_everything_equals_causal():
    """window >= N is the plain causal mask: bitwise the same output as attn_fwd."""
    w = PrefillWorkload("wc", 1, 8, 2, 640, 128, True)
    a = prefill_inputs(w, seed=31)
    q, k, v = dev_bf16(a["q"]), dev_bf16(a["k"]), dev_bf16(a["v"])
    o1, _ = paa.attn_fwd(q, k, v, True, a["scale"])
    o2, _ = paa.attn_fwd_window(q, k, v, 640, 0, a["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.timeout(600)
def test_window_full_size_whole():
    """B=1, H=32, Hkv=8, N=16384, d=128, window 4096, 64 global tokens: every element against the oracle."""
    w = WORKLOADS["window_gqa_b1h32kv8n16384d128_w4096_g64"]
    _announce(w.name)
    a = prefill_inputs(w, seed=0)
    o, lse = _run_window(a, w, w.window, w.n_global)
    ro, rl = oracle_pool.attention_window(a["q"], a["k"], a["v"], w.window, w.n_global, a["scale"])
    st = assert_close_bf16(o, ro)
    st.update(assert_close_lse(lse, rl))
    _announce(f"{w.name}: {st}")


# Grids large enough (at least 1024 eight-wave units) for the d=128 ping-pong kernel (the kernel the
# full-size GQA workloads run), with a ragged sequence end and every head-grouping branch; every output
# element is compared.
PINGPONG = [(4, 32, 8, 2000, True, 0, 0), (4, 32, 8, 2000, False, 0, 0), (8, 16, 8, 1999, True, 0, 0),
            (32, 8, 8, 1000, True, 0, 0), (4, 32, 8, 2000, True, 300, 17)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B,H,Hkv,N,causal,window,n_global", PINGPONG)
def test_bf16_pingpong_grids_whole(B, H, Hkv, N, causal, window, n_global):
    w = PrefillWorkload("pingpong", B, H, Hkv, N, 128, causal)
    _announce(f"pingpong B{B} H{H} Hkv{Hkv} N{N} causal{causal} window{window} g{n_global}")
    a = prefill_inputs(w, seed=N + H)
    if window:
        o, lse = _run_window(a, w, window, n_global)
        ro, rl = oracle_pool.attention_window(a["q"], a["k"], a["v"], window, n_global, a["scale"])
    else:
        o, lse = _run_bf16(a, w)
        ro, rl = oracle_pool.attention(a["q"], a["k"], a["v"], causal, a["scale"])
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


# the long GQA shape (ping-pong kernel), the d=64 causal shape (four-wave kernel), a d=64 grid large
# enough for the eight-wave kernel, a non-causal ping-pong grid, and the windowed workload's mask
ZERO_Q = [(1, 32, 8, 16384, 128, True, 0, 0), (4, 16, 16, 1024, 64, True, 0, 0), (2, 32, 8, 4096, 64, True, 0, 0),
          (2, 32, 8, 2000, 128, False, 0, 0), (1, 32, 8, 16384, 128, True, 4096, 64)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B,H,Hkv,N,d,causal,window,n_global", ZERO_Q)
def test_bf16_zero_query_closed_form(B, H, Hkv, N, d, causal, window, n_global):
    """Q = 0 at full size: O and LSE against the closed form (no oracle), every element."""
    _announce(f"attn_fwd{'_window' if window else ''} bf16 Q=0 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    a = prefill_inputs(PrefillWorkload("zq", B, H, Hkv, N, d, causal), seed=N + d + 7)
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda:0")
    k, v = dev_bf16(a["k"]), dev_bf16(a["v"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    if window:
        o, _ = paa.attn_fwd_window(q, k, v, window, n_global, a["scale"], lse=lse)
    else:
        o, _ = paa.attn_fwd(q, k, v, causal, a["scale"], lse=lse)
    torch.cuda.synchronize()
    vf = host_f64(v)
    ro, rl = zero_query_expected(vf, H, causal, window, n_global)
    assert_close_bf16(host_f64(o), ro)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_mha_with_repeated_kv(causal):
    """GQA (32 query heads over 8 KV heads) against the same call with each KV head repeated for its 4
    query heads (32 KV heads): every row walks the same key tiles in the same order whichever heads share
    its workgroup, so O and LSE agree bit for bit (B=2, N=4096, d=128: 1024 eight-wave units either way)."""
    w = PrefillWorkload("gqa_mha", 2, 32, 8, 4096, 128, causal)
    _announce(f"attn_fwd GQA vs MHA repeated, causal={causal}")
    a = prefill_inputs(w, seed=77)
    q, k, v = dev_bf16(a["q"]), dev_bf16(a["k"]), dev_bf16(a["v"])
    lse_g = torch.empty((2, 32, 4096), dtype=torch.float32, device="cuda:0")
    lse_m = torch.empty_like(lse_g)
    o_g, _ = paa.attn_fwd(q, k, v, causal, a["scale"], lse=lse_g)
    k4, v4 = k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous()
    o_m, _ = paa.attn_fwd(q, k4, v4, causal, a["scale"], lse=lse_m)
    torch.cuda.synchronize()
    assert torch.equal(o_g.view(torch.int16), o_m.view(torch.int16))
    assert torch.equal(lse_g, lse_m)
