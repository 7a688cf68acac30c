"""GPU parity of attn_fwd_fp8 (through the C ABI) against the float64 oracle, every output element.

What the kernel computes.  Each probability is taken relative to a reference maximum m_ref of its
row (at most 2^4 below the row's true maximum, in log2 units), scaled by C = 2^4 * 2^(m - m_ref)
(so 16 <= C <= 256) and rounded to E4M3: a value in the normal range (>= 2^-6) moves by at most
2^-4 of itself, a smaller one (subnormal or flushed) by at most FLUSH_ERR absolutely.  O is the sum
of rounded probabilities times V over the sum of the same rounded probabilities (both from 8-bit
MFMAs); LSE uses the fp32 sum of the unrounded ones.  The 8-bit MFMA does not sum its 64 products in
full fp32: its error reaches 2^-13.6 of the sum of the products' magnitudes (measured with random
E4M3 operands against the exact sums), so a score carries an error up to E_i = 2^-13 * scale *
max_j sum_d |q~_id k~_jd| for row i.

Per-element bound on O.  With w_ij the oracle's weights, O* the oracle's output, A_id = sum_j w_ij
|v~_jd| (the oracle over |V~|), delta = (1 + 2^-4) e^(E_i) - 1, l_i = exp(LSE_i - m_i) (m_i the row's
largest scaled score) and n_i visible keys with S_id = sum_j |v~_jd| over them:
    num = delta * (A_id + |O*_id|) + 2^-4 * FLUSH_ERR * (S_id + n_i |O*_id|) / l_i
    |O - O*| <= num * l_i / ((1 - delta) * max(1, l_i - n_i * 2^-6 * e^(E_i) / 16))
              + 2^-12 (A_id + |O*_id|) + 2^-9 (|O*_id| + that bound)
The first line is the rounding of the weights (relative, then absolute for the small ones: a key is
small only if C p_j e^(e_j) < 2^-6); the denominator bounds the sum of the rounded probabilities
from below by the normal keys' share; the last terms are the two MFMA sums and the bf16 output.
Mean bar: rounding to nearest with 3 mantissa bits leaves a relative error of variance at most
2^-8 / 3; taking the errors as independent and zero-mean, the error of O_id has standard deviation
at most 2^-4 / sqrt(3) * sqrt(max_j w_ij * sum_j w_ij (v~_jd - O*_id)^2), with max_j w_ij = 1 / l_i
and sum_j w_ij (v~_jd - O*_id)^2 = A2_id - O*_id^2 (A2 the oracle over V~^2); that bounds its mean
absolute value.  The mean bar is the mean of that plus the systematic terms (score error and bf16
rounding).

LSE: its bar is the bf16 path's 1e-3 plus E_i.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_attention_attn_amd as paa
import oracle_pool
from gpu_util import assert_close_bf16, assert_close_lse, host_f64, zero_query_expected
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


# Absolute error of rounding a probability below e4m3's normal range (2^-6): subnormals are kept and
# rounded to nearest (spacing 2^-9), values under 2^-10 become 0.  Measured on gfx950 with the packed
# conversion the kernel uses, and the 8-bit MFMA multiplies subnormal codes at their value.
FLUSH_ERR = 2.0 ** -10


def _dequant(a):
    q = oracle.e4m3_bits_to_f64(a["q8"]) * a["q_scale"]
    k = oracle.e4m3_bits_to_f64(a["k8"]) * a["k_scale"]
    v = np.swapaxes(oracle.e4m3_bits_to_f64(a["vt8"]), -1, -2) * a["v_scale"]
    return q, k, v


def _reference(a, causal):
    """Per (b, h), in a thread pool: O* and A (one oracle call over the values [V, |V|], |V| being the
    codes with their sign bit cleared), LSE*, and for the bounds m_i, E_i, n_i and S_id."""
    B, H, N, d = a["q8"].shape
    Hkv = a["k8"].shape[1]
    group = H // Hkv
    vt_cat = np.concatenate([a["vt8"], a["vt8"] & np.uint8(0x7F)], axis=2)
    q, k, v = _dequant(a)
    vabs = np.abs(v)
    vsq = v * v
    out = {n: np.empty((B, H, N, d)) for n in ("o", "A", "A2", "S")}
    out.update({n: np.empty((B, H, N)) for n in ("lse", "m", "E", "n")})

    def run(bh):
        b, h = bh
        g = h // group
        ro, rl = oracle.attention_fp8(a["q8"][b:b + 1, h:h + 1], a["k8"][b:b + 1, g:g + 1], vt_cat[b:b + 1, g:g + 1],
                                      causal, a["scale"], a["q_scale"], a["k_scale"], a["v_scale"])
        out["o"][b, h], out["A"][b, h], out["lse"][b, h] = ro[0, 0, :, :d], ro[0, 0, :, d:], rl[0, 0]
        out["A2"][b, h] = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], vsq[b:b + 1, g:g + 1], causal,
                                           a["scale"])[0][0, 0]
        csum = np.cumsum(vabs[b, g], axis=0)
        for r0 in range(0, N, 512):
            r1 = min(N, r0 + 512)
            nk = r1 if causal else N
            s = a["scale"] * (q[b, h, r0:r1] @ k[b, g, :nk].T)
            t = np.abs(q[b, h, r0:r1]) @ np.abs(k[b, g, :nk]).T
            if causal:
                hidden = np.arange(nk)[None, :] > np.arange(r0, r1)[:, None]
                s[hidden] = -np.inf
                t[hidden] = 0.0
            out["m"][b, h, r0:r1] = s.max(axis=1)
            out["E"][b, h, r0:r1] = 2.0 ** -13 * a["scale"] * t.max(axis=1)
            rows = np.arange(r0, r1)
            out["n"][b, h, r0:r1] = rows + 1 if causal else N
            out["S"][b, h, r0:r1] = csum[rows] if causal else csum[-1]

    oracle_pool._pool(run, [(b, h) for b in range(B) for h in range(H)])
    return out


def _assert_close_fp8(got_o, got_lse, ref):
    assert np.all(np.isfinite(got_o)), "non-finite values in kernel output"
    assert np.all(np.isfinite(got_lse)), "LSE: non-finite values"
    o, A, S = ref["o"], ref["A"], ref["S"]
    E = ref["E"][..., None]
    n = ref["n"][..., None]
    l = np.exp(ref["lse"] - ref["m"])[..., None]
    delta = (1 + 2.0 ** -4) * np.exp(E) - 1
    ao = np.abs(o)
    num = delta * (A + ao) + 2.0 ** -4 * FLUSH_ERR * (S + n * ao) / l
    l_normal = np.maximum(1.0, l - n * 2.0 ** -6 * np.exp(E) / 16)
    bound = num * l / ((1 - delta) * l_normal) + 2.0 ** -12 * (A + ao)
    bound = bound + 2.0 ** -9 * (ao + bound)
    err = np.abs(got_o - o)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert np.all(err <= bound), \
        f"|dO| {err[worst]:.3e} > bound {bound[worst]:.3e} at {tuple(int(x) for x in worst)}"
    sd = 2.0 ** -4 / np.sqrt(3.0) * np.sqrt(np.maximum(ref["A2"] - o * o, 0.0) / l)
    mean_bar = float(np.mean(sd + (delta - 2.0 ** -4) * (A + ao) + 2.0 ** -9 * ao))
    assert err.mean() <= mean_bar, f"mean |dO| {err.mean():.3e} > {mean_bar:.3e}"
    lse_bound = 1e-3 + ref["E"]
    lerr = np.abs(got_lse - ref["lse"])
    lw = np.unravel_index(int(np.argmax(lerr - lse_bound)), lerr.shape)
    assert np.all(lerr <= lse_bound), f"LSE |err| {lerr[lw]:.3e} > {lse_bound[lw]:.3e} at {lw}"
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "mean_bar": mean_bar,
            "max_err_over_bound": float((err / bound).max()), "lse_max_abs": float(lerr.max())}


def _check(a, w):
    o, lse = _run(a, w)
    ref = _reference(a, w.causal)
    return _assert_close_fp8(o, lse, ref)


# several tiles and query tiles, ragged ends (N a multiple of 16 but not of 64), every head grouping,
# both head dims, causal and not
SMALL = [(1, 4, 2, 1024, 64, True), (2, 8, 2, 512, 128, False), (1, 8, 8, 1008, 128, True),
         (1, 16, 4, 400, 64, False), (2, 6, 3, 272, 128, True), (1, 2, 1, 16, 64, True)]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", SMALL)
def test_fp8_small_full_parity(B, H, Hkv, N, d, causal):
    w = PrefillWorkload("fp8", B, H, Hkv, N, d, causal, dtype="fp8")
    _announce(f"fp8 B{B} H{H} Hkv{Hkv} N{N} d{d} causal{causal}")
    a = prefill_inputs(w, seed=N + d)
    _check(a, w)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["fp8_causal_gqa_b2h32kv8n4096d128", "fp8_causal_gqa_long_b1h32kv8n16384d128"])
def test_fp8_full_size_whole(name):
    """The full-size FP8 workloads: every element of O and LSE within its derived bound."""
    w = WORKLOADS[name]
    _announce(name)
    a = prefill_inputs(w, seed=0)
    st = _check(a, w)
    _announce(f"{name}: {st}")


def _quantized(x):
    from workloads import quantize_e4m3
    return quantize_e4m3(x)


def test_fp8_dominant_key_with_many_small_ones():
    """One key far above the rest and thousands of keys whose probabilities sit below e4m3's normal
    range, with identical V rows: O must return that row (the normalisation uses the same rounded
    probabilities as the numerator), and everything stays within the bounds."""
    B, H, Hkv, N, d = 1, 4, 1, 4096, 128
    rng = np.random.default_rng(70)
    q = np.zeros((B, H, N, d))
    q[..., 0] = 1.0
    k = np.zeros((B, Hkv, N, d))
    k[..., 0] = 0.375
    k[0, 0, 0, 0] = 8.0  # key 0 dominates every row that sees it
    v = np.tile(rng.standard_normal(d), (B, Hkv, N, 1))  # identical rows
    q8, qs = _quantized(q)
    k8, ks = _quantized(k)
    v8, vs = _quantized(v)
    a = dict(q8=q8, k8=k8, vt8=np.ascontiguousarray(np.swapaxes(v8, -1, -2)), q_scale=qs, k_scale=ks, v_scale=vs,
             scale=float(np.float32(1.0)))
    w = PrefillWorkload("fp8_dominant", B, H, Hkv, N, d, True, dtype="fp8")
    o, lse = _run(a, w)
    row = oracle.e4m3_bits_to_f64(v8[0, 0, 0]) * vs
    # with scale 1 the dominant key's score is 8 against about 0.36 for the others (0.375 after e4m3
    # rounding of the key): their probabilities are about 2^-11 of its own, which e4m3 would flush to 0
    # without the shift by 2^4 (and 4095 of them carry two thirds of the mass); with it they are
    # subnormals near 2^-7, kept
    assert np.allclose(o, np.broadcast_to(row, o.shape), rtol=2.0 ** -8, atol=2.0 ** -12)
    ref = _reference(a, True)
    _assert_close_fp8(o, lse, ref)


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


@pytest.mark.timeout(300)
@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [(1, 32, 8, 16384, 128, True), (2, 8, 2, 2000, 128, False)])
def test_fp8_zero_query_closed_form(B, H, Hkv, N, d, causal):
    """Q = 0 (all-zero E4M3 codes) at full size: every probability is the same power of two, which E4M3
    holds exactly, so O is the mean of the dequantized V rows a query sees and LSE = ln(count); O and LSE
    against that closed form (no oracle), every element, at the bf16 bars."""
    w = PrefillWorkload("fp8_zq", B, H, Hkv, N, d, causal, dtype="fp8")
    _announce(f"attn_fwd_fp8 Q=0 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    a = prefill_inputs(w, seed=N + 3)
    a["q8"] = np.zeros_like(a["q8"])
    o, lse = _run(a, w)
    _, _, v = _dequant(a)
    ro, rl = zero_query_expected(v, H, causal)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_fp8_gqa_equals_mha_with_repeated_kv():
    """FP8 prefill with 32 query heads over 8 KV heads against the same call with each KV head repeated
    for its 4 query heads: O and LSE agree bit for bit (B=2, N=2048, causal)."""
    w = PrefillWorkload("fp8_gqa_mha", 2, 32, 8, 2048, 128, True, dtype="fp8")
    _announce("attn_fwd_fp8 GQA vs MHA repeated")
    a = prefill_inputs(w, seed=79)
    o_g, l_g = _run(a, w)
    b = dict(a, k8=np.repeat(a["k8"], 4, axis=1), vt8=np.repeat(a["vt8"], 4, axis=1))
    o_m, l_m = _run(b, PrefillWorkload("fp8_gqa_mha", 2, 32, 32, 2048, 128, True, dtype="fp8"))
    assert np.array_equal(o_g, o_m) and np.array_equal(l_g, l_m)
