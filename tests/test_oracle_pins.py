"""CPU tests: the oracle against its pins, and planted mistakes against the pins."""

import numpy as np
import pytest

import oracle
from oracle import exact as A
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _mut_softmax_no_shift(s):
    e = np.exp(s)
    l = e.sum(axis=1)
    return e / l[:, None], np.zeros(s.shape[0]), l


def _mut_softmax_unnormalised(s):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return e, m, e.sum(axis=1)


def _mut_softmax_lse_without_max(s):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], np.zeros_like(m), l


def _mut_causal_strict(s, row_pos):
    cols = np.arange(s.shape[1])
    s[cols[None, :] >= row_pos[:, None]] = -np.inf


def _mut_causal_flipped(s, row_pos):
    cols = np.arange(s.shape[1])
    s[cols[None, :] < row_pos[:, None]] = -np.inf


def _mut_window_inclusive(row_pos, n_keys, window, n_global):
    j = np.arange(n_keys)[None, :]
    i = row_pos[:, None]
    return ~((j <= i) & ((i - j <= window) | (j < n_global)))


def _mut_window_global_inclusive(row_pos, n_keys, window, n_global):
    j = np.arange(n_keys)[None, :]
    i = row_pos[:, None]
    return ~((j <= i) & ((i - j < window) | (j <= n_global)))


def _mut_window_not_causal(row_pos, n_keys, window, n_global):
    j = np.arange(n_keys)[None, :]
    i = row_pos[:, None]
    return ~((np.abs(i - j) < window) | (j < n_global))


def _mut_e4m3_bias8(x):
    b = np.asarray(x, dtype=np.uint8).astype(np.int64)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    return np.where(b >> 7, -mag, mag)


def _mut_dequant_no_transpose(q8, k8, vt8, q_scale, k_scale, v_scale):
    return (A.e4m3_bits_to_f64(q8) * q_scale, A.e4m3_bits_to_f64(k8) * k_scale,
            A.e4m3_bits_to_f64(vt8) * v_scale)


# Each entry: (helper name in oracle.exact, planted replacement)
MUTANTS = {
    "gqa_modulo_mapping": ("_kv_head", lambda h, H, Hkv: h % Hkv),
    "gqa_off_by_one": ("_kv_head", lambda h, H, Hkv: min(Hkv - 1, (h + 1) // (H // Hkv))),
    "scale_dropped": ("_scores", lambda q, k, scale: q @ k.T),
    "scale_squared": ("_scores", lambda q, k, scale: scale * scale * (q @ k.T)),
    "sign_flipped": ("_scores", lambda q, k, scale: -scale * (q @ k.T)),
    "key_dims_reversed": ("_scores", lambda q, k, scale: scale * (q @ k[:, ::-1].T)),
    "causal_masks_diagonal": ("_apply_causal", _mut_causal_strict),
    "causal_mask_flipped": ("_apply_causal", _mut_causal_flipped),
    "softmax_no_max_shift": ("_softmax", _mut_softmax_no_shift),
    "softmax_unnormalised": ("_softmax", _mut_softmax_unnormalised),
    "lse_without_max": ("_softmax", _mut_softmax_lse_without_max),
    "page_block_slot_swapped": ("_page_slot", lambda t, ps: (t % ps, t // ps)),
    "page_off_by_one_token": ("_page_slot", lambda t, ps: ((t + 1) // ps, (t + 1) % ps)),
    "window_off_by_one": ("_window_mask", _mut_window_inclusive),
    "window_global_off_by_one": ("_window_mask", _mut_window_global_inclusive),
    "window_not_causal": ("_window_mask", _mut_window_not_causal),
    "chunk_aligned_at_start": ("_chunk_positions", lambda ctx, n: np.arange(n)),
    "chunk_positions_off_by_one": ("_chunk_positions", lambda ctx, n: ctx + 1 + np.arange(n)),
    "chunk_positions_reversed": ("_chunk_positions", lambda ctx, n: ctx + np.arange(n)[::-1]),
    "fp8_exponent_bias_8": ("e4m3_bits_to_f64", _mut_e4m3_bias8),
    "fp8_v_not_transposed": ("_dequant_fp8", _mut_dequant_no_transpose),
    "seqs_subset_ignored": ("_selected", lambda n, seqs: range(n)),
    "seqs_subset_reordered": ("_selected", lambda n, seqs: range(n) if seqs is None else sorted(set(seqs))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(A, attr, repl)
    caught = []
    with np.errstate(all="ignore"):
        for pin in P.ALL_PINS:
            try:
                pin()
            except (AssertionError, IndexError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
    assert caught, f"planted mistake {name} escaped every pin"


def test_bf16_bits_to_f64_exact():
    # 1.0, -2.0, 0.15625 (exactly representable), largest finite bf16, smallest normal
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x7F7F, 0x0080], dtype=np.uint16)
    want = np.array([1.0, -2.0, 0.15625, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -126])
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), want)


@pytest.mark.parametrize("causal,window,n_global", [(False, 0, 0), (True, 0, 0), (True, 5, 0), (True, 5, 3),
                                                    (True, 40, 2)])
def test_zero_query_closed_form(causal, window, n_global):
    """With Q = 0 every visible score is 0: the oracle gives each row the mean of the V rows it sees and
    LSE = ln(count).  This pins the oracle's masks and weights, and the closed form the full-size GPU
    tests compare against."""
    from gpu_util import zero_query_expected
    rng = np.random.default_rng(7)
    B, H, Hkv, N, d = 2, 4, 2, 37, 8
    q = np.zeros((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    if window:
        o, lse = oracle.attention_window(q, k, v, window, n_global, 0.3)
    else:
        o, lse = oracle.attention(q, k, v, causal, 0.3)
    ro, rl = zero_query_expected(v, H, causal, window, n_global)
    # brute force on one row: the visible set written out from the mask's definition
    i, vis = 20, [j for j in range(N) if (not causal) or (j <= 20 and (not window or 20 - j < window or j < n_global))]
    np.testing.assert_allclose(ro[1, 3, i], v[1, 1, vis].mean(axis=0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_decode_zero_query_closed_form():
    """q = 0 in decode: the oracle returns each head the mean of its KV head's V rows over the sequence
    (gathered through the block table) and LSE = ln L; this pins the oracle's decode gather and the
    closed form the full-size GPU tests compare against."""
    from gpu_util import decode_zero_query_expected
    from workloads import DecodeWorkload, decode_inputs
    lens = [1, 15, 16, 17, 40, 0, 100]
    w = DecodeWorkload("zq", len(lens), 8, 2, 16, 1, 128, 16, 64)
    a = decode_inputs(w, seed=5, seq_lens=lens)
    a["q"] = np.zeros_like(a["q"])
    o, lse = oracle.paged_decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], a["scale"])
    ro, rl = decode_zero_query_expected(oracle.bf16_bits_to_f64, a["v_cache"], a["block_table"], a["seq_lens"], 8)
    # brute force for sequence 4, head 5 (KV head 1): token t from page bt[4][t // 16], slot t % 16
    v = oracle.bf16_bits_to_f64(a["v_cache"])
    rows = [v[a["block_table"][4][t // 16], t % 16, 1] for t in range(40)]
    np.testing.assert_allclose(ro[4, 5], np.mean(rows, axis=0), rtol=0, atol=1e-12)
    live = np.asarray(lens) > 0
    np.testing.assert_allclose(o[live], ro[live], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[live], rl[live], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(rl[~live])) and np.all(ro[~live] == 0)
