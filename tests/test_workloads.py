"""CPU tests of the seeded input generators (layout and rounding, no attention math)."""

import numpy as np

from workloads import (WORKLOADS, DecodeWorkload, PrefillWorkload, BF16_NAN, bf16_bits_to_f32,
                       decode_inputs, f32_to_bf16_bits, prefill_inputs)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -3.5, 0.0, np.inf, np.nan],
                 dtype=np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7: goes to the even pattern (1.0);
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: goes to 1+2^-6 (even mantissa)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -3.5, 0.0, np.inf], dtype=np.float32)
    got = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(got[:-1]), want)
    assert got[-1] == BF16_NAN


def test_prefill_inputs_shapes_and_outliers():
    w = PrefillWorkload("t", 1, 4, 2, 300, 64, causal=True, q_mult=4.0, k_outlier_frac=0.01)
    a = prefill_inputs(w, seed=3)
    assert a["q"].shape == (1, 4, 300, 64) and a["k"].shape == (1, 2, 300, 64)
    assert a["q"].dtype == np.uint16
    assert a["outliers"].shape == (1, 2, 3)
    for g in range(2):
        assert len(set(a["outliers"][0, g])) == 3
    b = prefill_inputs(w, seed=3)
    assert np.array_equal(a["k"], b["k"])  # seeded


def test_named_workloads():
    assert WORKLOADS["causal_gqa_long_b1h32kv8n16384d128"].q_mult == 4.0
    assert WORKLOADS["tiny_f32_b1h2n128d64"].scale == 0.125
    assert WORKLOADS["paged_decode_s64h32kv8d128"].max_pages_per_seq == 512


def test_decode_layout_and_poison():
    w = DecodeWorkload("t", 5, 4, 2, 16, 1, 70, page_size=16, num_pages=40)
    a = decode_inputs(w, seed=1)
    lens, bt, kc = a["seq_lens"], a["block_table"], a["k_cache"]
    assert np.all((lens >= 1) & (lens <= 70))
    used = []
    for s in range(5):
        n = -(-int(lens[s]) // 16)
        assert np.all(bt[s, :n] >= 0) and np.all(bt[s, n:] == -1)
        used += list(bt[s, :n])
        # every slot past the last token of the last page is poisoned
        last = bt[s, n - 1]
        tail = int(lens[s]) - 16 * (n - 1)
        assert np.all(kc[last, tail:] == BF16_NAN)
        assert not np.any(kc[last, :tail] == BF16_NAN)
    assert len(used) == len(set(used))  # distinct physical pages
    unused = sorted(set(range(40)) - set(used))
    assert np.all(kc[unused] == BF16_NAN)


def test_window_visible_pairs_by_counting():
    """Visible-pair count of a windowed workload equals a direct count of the rule on a small case."""
    w = PrefillWorkload("t", 1, 1, 1, 37, 8, causal=True, window=5, n_global=3)
    want = sum(1 for i in range(37) for j in range(i + 1) if i - j < 5 or j < 3)
    assert w.visible_pairs() == want
    assert PrefillWorkload("c", 1, 1, 1, 37, 8, causal=True).visible_pairs() == 37 * 38 // 2


def test_e4m3_encoder_matches_torch_rounding():
    """The input quantizer rounds like torch's float8_e4m3fn cast (nearest, ties to even) within +-448."""
    import torch
    from workloads import f32_to_e4m3_bits, quantize_e4m3
    x = np.random.default_rng(3).standard_normal(50000).astype(np.float32) * 40
    x[:6] = [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 3 * 2.0 ** -10]  # zero, extremes, a subnormal, a tie
    want = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = f32_to_e4m3_bits(x)
    assert np.array_equal(got, want)
    q, s = quantize_e4m3(x)
    assert abs(s * 448.0 - np.abs(x).max()) <= 1e-6 * np.abs(x).max()


def test_fp8_workload_layout():
    from workloads import PrefillWorkload, prefill_inputs
    w = PrefillWorkload("t", 1, 4, 2, 48, 64, True, dtype="fp8")
    a = prefill_inputs(w, seed=1)
    assert a["q8"].shape == (1, 4, 48, 64) and a["k8"].shape == (1, 2, 48, 64) and a["vt8"].shape == (1, 2, 64, 48)
    assert a["q8"].dtype == np.uint8 and a["vt8"].flags["C_CONTIGUOUS"]


def test_fp8_decode_inputs_quantize_the_bf16_draws():
    """FP8 decode inputs hold the bf16 draws quantized per tensor (max |x| -> 448), with the E4M3 NaN code
    in exactly the slots no token occupies."""
    from workloads import DecodeWorkload, decode_inputs, decode_inputs_fp8, quantize_e4m3
    w = DecodeWorkload("fp8dec", 4, 8, 2, 64, 1, 90, 16, 40)
    a = decode_inputs(w, seed=7)
    b = decode_inputs_fp8(w, seed=7)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["block_table"], b["block_table"])
    for name, sname in (("k_cache", "k_scale"), ("v_cache", "v_scale")):
        x = bf16_bits_to_f32(a[name])
        used = ~np.isnan(x)
        assert np.array_equal(b[name][~used], np.full((~used).sum(), 0x7F, np.uint8))
        codes, scale = quantize_e4m3(x[used])
        assert b[sname] == scale and abs(scale * 448.0 - np.abs(x[used]).max()) <= 1e-6 * scale * 448.0
        assert np.array_equal(b[name][used], codes)
