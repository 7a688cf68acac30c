"""GPU parity of attn_fwd_fp8 (through the C ABI) against the float64 oracle.

Tolerance.  The kernel rounds each probability to E4M3 before the product with V (relative error
at most 2^-4 for probabilities in the normal range) and keeps everything else in fp32, whose
errors are far smaller.  Hence |O - O_exact| <= 2^-4 * max|V~| elementwise (V~ = v_scale * V, the
dequantized values), the bar used for the maximum.  Those rounding errors are zero-mean and
largely cancel over a row; the mean bar, 2^-8 * max|V~|, sits about four times above the mean
error of an emulation of this rounding at these shapes.

The 8-bit matrix instruction does not accumulate its 64 products in full fp32: on gfx950 its
error reaches 2^-13.6 of the sum of the products' magnitudes (measured with random E4M3
operands against the exact sums), where fp32 would give 2^-24.  A score then carries an error up
to 2^-13 * scale * sum_d |q~_d k~_d|, and the LSE, which follows the row's largest scores, the
same: its bar is the bf16 path's 1e-3 plus that bound for the row's largest such sum.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_attention_attn_amd as paa
from gpu_util import host_f64, sample_rows
from workloads import WORKLOADS, PrefillWorkload, prefill_inputs

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _dev8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _run(a, w):
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    o, _ = paa.attn_fwd_fp8(_dev8(a["q8"]), _dev8(a["k8"]), _dev8(a["vt8"]), w.causal, a["scale"],
                            a["q_scale"], a["k_scale"], a["v_scale"], lse=lse)
    torch.cuda.synchronize()
    return host_f64(o), lse.cpu().numpy().astype(np.float64)


def _assert_close_lse_fp8(got, want, a, rows, causal):
    """|dLSE| <= 1e-3 + 2^-13 * scale * max over visible keys j of sum_d |q~_id k~_jd| for each row (b, h, i)."""
    q = np.abs(oracle.e4m3_bits_to_f64(a["q8"])) * a["q_scale"]
    k = np.abs(oracle.e4m3_bits_to_f64(a["k8"])) * a["k_scale"]
    H, Hkv = q.shape[1], k.shape[1]
    bound = np.empty(len(rows))
    for n, (b, h, i) in enumerate(rows):
        sums = k[b, h // (H // Hkv), : (i + 1 if causal else None)] @ q[b, h, i]
        bound[n] = 1e-3 + 2.0 ** -13 * a["scale"] * sums.max()
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), "LSE: non-finite values"
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"LSE: |err| {err[worst]:.3e} > bound {bound[worst]:.3e} at row {rows[worst]}"


def _assert_close_fp8(got, want, a):
    vmax = float(np.abs(oracle.e4m3_bits_to_f64(a["vt8"])).max()) * a["v_scale"]
    assert np.all(np.isfinite(got)), "non-finite values in kernel output"
    err = np.abs(got - want)
    assert err.max() <= 2.0 ** -4 * vmax, f"max |err| {err.max():.3e} > 2^-4 * max|V| = {2.0 ** -4 * vmax:.3e}"
    assert err.mean() <= 2.0 ** -8 * vmax, f"mean |err| {err.mean():.3e} > 2^-8 * max|V| = {2.0 ** -8 * vmax:.3e}"


# several tiles and query tiles, ragged ends (N a multiple of 16 but not of 64), every head grouping,
# both head dims, causal and not
SMALL = [(1, 4, 2, 1024, 64, True), (2, 8, 2, 512, 128, False), (1, 8, 8, 1008, 128, True),
         (1, 16, 4, 400, 64, False), (2, 6, 3, 272, 128, True), (1, 2, 1, 16, 64, True)]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", SMALL)
def test_fp8_small_full_parity(B, H, Hkv, N, d, causal):
    w = PrefillWorkload("fp8", B, H, Hkv, N, d, causal, dtype="fp8")
    _announce(f"fp8 B{B} H{H} Hkv{Hkv} N{N} d{d} causal{causal}")
    a = prefill_inputs(w, seed=N + d)
    o, lse = _run(a, w)
    ro, rl = oracle.attention_fp8(a["q8"], a["k8"], a["vt8"], causal, a["scale"], a["q_scale"], a["k_scale"],
                                  a["v_scale"])
    _assert_close_fp8(o, ro, a)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(N)]
    _assert_close_lse_fp8(lse.reshape(-1), rl.reshape(-1), a, rows, causal)


@pytest.mark.parametrize("name", ["fp8_causal_gqa_b2h32kv8n4096d128", "fp8_causal_gqa_long_b1h32kv8n16384d128"])
def test_fp8_full_size_sampled(name):
    w = WORKLOADS[name]
    _announce(name)
    a = prefill_inputs(w, seed=0)
    o, lse = _run(a, w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = sample_rows(w.B, w.H, w.N, 160, seed=4)
    rows += [(0, h, i) for h in (0, w.H - 1) for i in (0, 63, 64, w.N - 1)]
    rows = sorted(set(rows))
    ro, rl = oracle.attention_fp8_rows(a["q8"], a["k8"], a["vt8"], True, a["scale"], a["q_scale"], a["k_scale"],
                                       a["v_scale"], rows)
    idx = tuple(np.array(rows).T)
    _assert_close_fp8(o[idx], ro, a)
    _assert_close_lse_fp8(lse[idx], rl, a, rows, True)


def test_fp8_scales_and_determinism():
    """The tensor scales enter as the definition says (doubling v_scale doubles O up to bf16 rounding); two
    calls give identical bits."""
    w = PrefillWorkload("fp8", 1, 4, 2, 256, 128, True, dtype="fp8")
    a = prefill_inputs(w, seed=7)
    o1, l1 = _run(a, w)
    o1b, l1b = _run(a, w)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    b = dict(a, v_scale=2 * a["v_scale"])
    o2, l2 = _run(b, w)
    assert np.array_equal(l1, l2) and np.allclose(o2, 2 * o1, rtol=2.0 ** -7, atol=0)
