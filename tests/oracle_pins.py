"""Pins for the float64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle breaks the fact
it checks.  ``test_oracle_pins.py`` runs them against the oracle as it stands,
and against copies of it with one planted mistake each (every planted mistake
must be caught by at least one pin).  Nothing here re-types the oracle's
formula: the expected values come from closed forms, invariants, a brute-force
``math.fsum`` loop, ``numpy.repeat`` and the CPU float64
``torch.nn.functional.scaled_dot_product_attention`` library routine.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


# ---------------------------------------------------------------- prefill pins

def pin_softmax_rows_sum_to_one():
    """Every probability row sums to 1, entries are in [0, 1], masked entries are exactly 0."""
    q, k = _rand((1, 2, 37, 8), 1), _rand((1, 2, 37, 8), 2)
    for causal in (False, True):
        for h in range(2):
            p = oracle.softmax_probs(q, k, causal, 0.3, 0, h)
            assert np.all(np.abs(p.sum(axis=1) - 1.0) < 1e-12)
            assert np.all(p >= 0) and np.all(p <= 1)
            if causal:
                assert np.all(p[np.triu_indices(37, 1)] == 0.0)
                assert np.all(np.diag(p) > 0)


def pin_zero_query_gives_mean_of_visible_values():
    """Q = 0 makes all visible scores equal: O_i is the mean of the visible V rows, LSE_i = ln(count)."""
    B, H, N, d = 2, 4, 23, 6
    v = _rand((B, 2, N, d), 3)
    k = _rand((B, 2, N, d), 4)
    q = np.zeros((B, H, N, d))
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.7)
        for b in range(B):
            for h in range(H):
                g = h // 2
                for i in range(N):
                    n = i + 1 if causal else N
                    assert np.allclose(o[b, h, i], v[b, g, :n].mean(axis=0), rtol=0, atol=1e-13)
                    assert abs(lse[b, h, i] - math.log(n)) < 1e-13


def pin_identical_value_rows():
    """If every V row is the same vector c, every output row is c."""
    c = _rand((5,), 5)
    v = np.broadcast_to(c, (1, 1, 19, 5)).copy()
    q, k = _rand((1, 3, 19, 5), 6, 3.0), _rand((1, 1, 19, 5), 7, 3.0)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 0.5)
        assert np.allclose(o, c, rtol=0, atol=1e-13)


def pin_causal_first_row():
    """With the causal mask, query 0 sees only key 0: O_0 = V_0 and LSE_0 = scale * q_0 . k_0."""
    q, k, v = _rand((2, 2, 11, 7), 8), _rand((2, 1, 11, 7), 9), _rand((2, 1, 11, 7), 10)
    scale = 0.37
    o, lse = oracle.attention(q, k, v, True, scale)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(o[b, h, 0], v[b, 0, 0])
            assert abs(lse[b, h, 0] - scale * math.fsum(q[b, h, 0] * k[b, 0, 0])) < 1e-13


def _brute(q, k, v, causal, scale):
    """Attention from the definition with pure-Python loops and math.fsum (H == Hkv)."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if (not causal) or j <= i]
                s = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, h, j, c]) for c in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(w[n] * float(v[b, h, j, c]) for n, j in enumerate(keys)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


def pin_brute_force_tiny():
    """Agreement with a brute-force fsum implementation on tiny shapes (to 1e-12)."""
    for N, d, causal, seed in [(1, 1, False, 0), (3, 2, True, 1), (5, 4, False, 2), (8, 4, True, 3),
                               (7, 3, True, 4)]:
        q, k, v = _rand((1, 2, N, d), seed), _rand((1, 2, N, d), seed + 10), _rand((1, 2, N, d), seed + 20)
        o, lse = oracle.attention(q, k, v, causal, 0.61)
        ob, lb = _brute(q, k, v, causal, 0.61)
        assert np.allclose(o, ob, rtol=0, atol=1e-12)
        assert np.allclose(lse, lb, rtol=0, atol=1e-12)


def pin_torch_sdpa_float64():
    """Agreement with torch's CPU float64 scaled_dot_product_attention (GQA via enable_gqa)."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, N, d, causal) in [(2, 4, 2, 33, 16, True), (1, 6, 3, 29, 8, False),
                                      (1, 8, 2, 64, 32, True), (2, 2, 2, 17, 64, False)]:
        q, k, v = _rand((B, H, N, d), N), _rand((B, Hkv, N, d), N + 1), _rand((B, Hkv, N, d), N + 2)
        scale = 1.0 / math.sqrt(d)
        o, _ = oracle.attention(q, k, v, causal, scale)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             is_causal=causal, scale=scale, enable_gqa=True).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-10)


def pin_gqa_equals_mha_with_repeated_kv():
    """Grouped heads equal plain multi-head attention on K/V repeated per group (numpy.repeat)."""
    q = _rand((1, 8, 21, 4), 11)
    k, v = _rand((1, 2, 21, 4), 12), _rand((1, 2, 21, 4), 13)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal, 0.9)
        o2, l2 = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), causal, 0.9)
        assert np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-14)


def pin_key_permutation_invariance():
    """Without a mask, permuting keys and values together leaves O and LSE unchanged."""
    q, k, v = _rand((1, 2, 30, 5), 14), _rand((1, 2, 30, 5), 15), _rand((1, 2, 30, 5), 16)
    perm = np.random.default_rng(17).permutation(30)
    o1, l1 = oracle.attention(q, k, v, False, 0.8)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.8)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)


def pin_peaked_scores_stay_finite():
    """Scores in the thousands: the max-shifted softmax stays finite and picks the dominant key.

    Key 3 is q's own direction times 40, every other key is orthogonal to q, so
    row 0's scores are 1600*|q|^2*scale for key 3 and 0 elsewhere: O_0 = V_3 to
    within exp(-1000), LSE_0 = that score to within 1e-12 relative.
    """
    d = 4
    qv = np.array([1.0, 2.0, -1.0, 0.5])
    k = np.zeros((1, 1, 6, d))
    k[0, 0, 3] = 40.0 * qv
    k[0, 0, [0, 1, 2, 4, 5]] = np.array([2.0, -1.0, 0.0, 0.0]) * np.arange(1, 6)[:, None]  # orthogonal to qv
    q = np.zeros((1, 1, 6, d))
    q[0, 0, :] = 40.0 * qv
    v = _rand((1, 1, 6, d), 18)
    o, lse = oracle.attention(q, k, v, False, 0.5)
    top = 0.5 * 1600.0 * float(qv @ qv)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.allclose(o[0, 0, 0], v[0, 0, 3], rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - top) < 1e-12 * top


def pin_rows_equal_full():
    """attention_rows returns exactly the selected rows of attention."""
    q, k, v = _rand((2, 4, 40, 8), 19), _rand((2, 2, 40, 8), 20), _rand((2, 2, 40, 8), 21)
    rows = [(0, 0, 0), (1, 3, 39), (0, 2, 17), (1, 1, 5)]
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.4)
        ro, rl = oracle.attention_rows(q, k, v, causal, 0.4, rows)
        for n, (b, h, i) in enumerate(rows):
            assert np.allclose(ro[n], o[b, h, i], rtol=0, atol=1e-14)
            assert abs(rl[n] - lse[b, h, i]) < 1e-14


# ----------------------------------------------------------------- the tiled online algorithm

def _online_attention(q, k, v, causal, scale, br, bc):
    """The tile-by-tile algorithm with a running max, a running sum and a rescaled accumulator ("Kernel
    Fusion and Custom Kernels", section 3, FlashAttention v1/v2), written independently of the oracle:
    query blocks of br rows, key tiles of bc keys, causal tiles wholly above a block's last row skipped.
    Query head h reads KV head h // (H // Hkv)."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            kh, vh = k[b, h // (H // Hkv)], v[b, h // (H // Hkv)]
            for r0 in range(0, N, br):
                rows = np.arange(r0, min(r0 + br, N))
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), d))
                for c0 in range(0, N, bc):
                    if causal and c0 > rows[-1]:
                        break  # this tile and every later one lie above the diagonal
                    cols = np.arange(c0, min(c0 + bc, N))
                    s = scale * (q[b, h, rows] @ kh[cols].T)
                    if causal:
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_new = np.maximum(m, s.max(axis=1))
                    # a row with no visible key yet keeps m = -inf; its factors are taken as 0
                    alpha = np.where(np.isneginf(m_new), 0.0, np.exp(np.where(np.isneginf(m), -np.inf, m - m_new)))
                    p = np.where(np.isneginf(s), 0.0, np.exp(s - np.where(np.isneginf(m_new), 0.0, m_new)[:, None]))
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ vh[cols]
                    m = m_new
                o[b, h, rows] = acc / l[:, None]
                lse[b, h, rows] = m + np.log(l)
    return o, lse


def _merge_splits(parts):
    """Merge per-split (O_c, LSE_c) of the same rows: weights exp(LSE_c - max), splits with LSE = -inf weigh 0."""
    lses = np.stack([p[1] for p in parts])
    top = lses.max(axis=0)
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - top))
    tot = w.sum(axis=0)
    o = sum(w[c][..., None] * parts[c][0] for c in range(len(parts))) / tot[..., None]
    return o, top + np.log(tot)


def pin_online_tiles_equal_plain():
    """The online algorithm reaches the plain softmax result for any tiling ("Kernel Fusion and Custom
    Kernels", section 3: exact, not approximate), causal and not, with grouped KV heads."""
    q, k, v = _rand((2, 4, 37, 8), 40, 2.0), _rand((2, 2, 37, 8), 41), _rand((2, 2, 37, 8), 42)
    for causal in (False, True):
        ro, rl = oracle.attention(q, k, v, causal, 0.3)
        for br, bc in ((1, 1), (3, 5), (16, 8), (8, 64), (37, 37)):
            o, lse = _online_attention(q, k, v, causal, 0.3, br, bc)
            assert np.allclose(o, ro, rtol=0, atol=1e-12), (causal, br, bc)
            assert np.allclose(lse, rl, rtol=0, atol=1e-12), (causal, br, bc)


def pin_split_key_merge_equals_plain():
    """Cutting a sequence's pages into consecutive ranges, decoding each range on its own and merging the
    partial (O_c, LSE_c) by weights exp(LSE_c - max) (the rescaling identity of "Kernel Fusion and Custom
    Kernels", section 3, as the decode's reduce applies it) gives the decode over all the pages."""
    H, Hkv, d, L = 4, 2, 8, 77  # 5 pages of 16, the last one partly used
    n_pages = -(-L // 16)
    q = _rand((1, H, d), 46)
    kc, vc = _rand((n_pages, 16, Hkv, d), 47), _rand((n_pages, 16, Hkv, d), 48)
    table = np.array([[3, 0, 4, 1, 2]])
    full_o, full_lse = oracle.paged_decode(q, kc, vc, table, np.array([L]), 0.4)
    for cuts in ((0, 5), (0, 1, 5), (0, 2, 3, 5), (0, 1, 2, 3, 4, 5)):
        parts = []
        for p0, p1 in zip(cuts[:-1], cuts[1:]):
            n = min(L, 16 * p1) - 16 * p0  # tokens of the range
            parts.append(oracle.paged_decode(q, kc, vc, table[:, p0:p1], np.array([n]), 0.4))
        o, lse = _merge_splits(parts)
        assert np.allclose(o, full_o, rtol=0, atol=1e-12), cuts
        assert np.allclose(lse, full_lse, rtol=0, atol=1e-12), cuts
    # a range with no visible key (LSE = -inf, output 0) weighs nothing
    empty = (np.zeros_like(full_o), np.full_like(full_lse, -np.inf))
    o, lse = _merge_splits([empty, (full_o, full_lse)])
    assert np.allclose(o, full_o, rtol=0, atol=1e-15) and np.allclose(lse, full_lse, rtol=0, atol=1e-15)


# ----------------------------------------------------------------- sliding window + global tokens

def _brute_window(q, k, v, window, n_global, scale):
    """Windowed causal attention straight from the rule, with pure-Python loops and math.fsum."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = []
                for j in range(N):
                    if j > i:
                        continue
                    if i - j < window or j < n_global:
                        keys.append(j)
                s = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, h, j, c]) for c in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(w[n] * float(v[b, h, j, c]) for n, j in enumerate(keys)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


def pin_window_brute_force_tiny():
    """Sliding window + global tokens against the brute-force rule on tiny shapes (to 1e-12)."""
    for N, d, window, n_global, seed in [(9, 3, 2, 0, 40), (9, 3, 3, 2, 41), (12, 4, 4, 1, 42), (6, 2, 1, 0, 43),
                                         (10, 2, 20, 0, 44), (11, 3, 5, 11, 45)]:
        q, k, v = _rand((1, 2, N, d), seed), _rand((1, 2, N, d), seed + 10), _rand((1, 2, N, d), seed + 20)
        o, lse = oracle.attention_window(q, k, v, window, n_global, 0.7)
        ob, lb = _brute_window(q, k, v, window, n_global, 0.7)
        assert np.allclose(o, ob, rtol=0, atol=1e-12)
        assert np.allclose(lse, lb, rtol=0, atol=1e-12)


def pin_window_torch_sdpa_boolean_mask():
    """Agreement with torch's CPU float64 SDPA given the window mask as a boolean matrix built by loops."""
    import torch
    import torch.nn.functional as F
    for (N, d, window, n_global) in [(40, 8, 7, 3), (33, 16, 1, 0), (50, 8, 64, 0), (37, 4, 5, 37)]:
        q, k, v = _rand((1, 2, N, d), N), _rand((1, 2, N, d), N + 1), _rand((1, 2, N, d), N + 2)
        allowed = torch.zeros((N, N), dtype=torch.bool)
        for i in range(N):
            for j in range(i + 1):
                allowed[i, j] = (i - j < window) or (j < n_global)
        o, _ = oracle.attention_window(q, k, v, window, n_global, 0.3)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             attn_mask=allowed, scale=0.3).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-10)


def pin_window_one_is_identity():
    """window = 1 with no global token: each query sees only its own key, O_i = V_i, LSE_i = scale q_i.k_i."""
    q, k, v = _rand((1, 1, 13, 5), 46), _rand((1, 1, 13, 5), 47), _rand((1, 1, 13, 5), 48)
    o, lse = oracle.attention_window(q, k, v, 1, 0, 0.45)
    assert np.array_equal(o, v)
    for i in range(13):
        assert abs(lse[0, 0, i] - 0.45 * math.fsum(q[0, 0, i] * k[0, 0, i])) < 1e-13


def pin_window_one_with_one_global_token():
    """window = 1, one global token: query i >= 1 sees keys {0, i}, a two-term softmax in closed form."""
    q, k, v = _rand((1, 1, 10, 4), 49), _rand((1, 1, 10, 4), 50), _rand((1, 1, 10, 4), 51)
    o, lse = oracle.attention_window(q, k, v, 1, 1, 0.6)
    for i in range(1, 10):
        s0 = 0.6 * math.fsum(q[0, 0, i] * k[0, 0, 0])
        si = 0.6 * math.fsum(q[0, 0, i] * k[0, 0, i])
        mx = max(s0, si)
        w0, wi = math.exp(s0 - mx), math.exp(si - mx)
        assert np.allclose(o[0, 0, i], (w0 * v[0, 0, 0] + wi * v[0, 0, i]) / (w0 + wi), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - (mx + math.log(w0 + wi))) < 1e-13
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])


def pin_window_rows_equal_full():
    """attention_window_rows returns exactly the selected rows of attention_window."""
    q, k, v = _rand((1, 4, 70, 8), 52), _rand((1, 2, 70, 8), 53), _rand((1, 2, 70, 8), 54)
    o, lse = oracle.attention_window(q, k, v, 9, 3, 0.4)
    rows = [(0, 0, 0), (0, 3, 69), (0, 1, 8), (0, 2, 9), (0, 2, 40)]
    ro, rl = oracle.attention_window_rows(q, k, v, 9, 3, 0.4, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.allclose(ro[n], o[b, h, i], rtol=0, atol=1e-14)
        assert abs(rl[n] - lse[b, h, i]) < 1e-14


# ----------------------------------------------------------------- decode pins

def _golden_example():
    with open(os.path.join(GOLDEN, "block_table_example.json")) as f:
        return json.load(f)


def _pool_from_table(table, L, Hkv, d, num_pages, page_size, seed):
    """A pool holding L logical tokens placed by hand from the golden locations rule; NaN elsewhere."""
    rng = np.random.default_rng(seed)
    kk, vv = rng.standard_normal((L, Hkv, d)), rng.standard_normal((L, Hkv, d))
    kc = np.full((num_pages, page_size, Hkv, d), np.nan)
    vc = np.full((num_pages, page_size, Hkv, d), np.nan)
    for t in range(L):
        kc[table[t // page_size], t % page_size] = kk[t]
        vc[table[t // page_size], t % page_size] = vv[t]
    return kk, vv, kc, vc


def pin_block_table_worked_example():
    """The pages' table [17, 4, 29, 8]: gathering through it returns the logical tokens in order,
    and decode over the pages equals attention over the contiguous logical sequence."""
    ex = _golden_example()
    table, ps = ex["physical_blocks"], ex["page_size"]
    Hkv, H, d, L = 2, 4, 8, 57  # the last page is partly filled (57 = 3 * 16 + 9)
    kk, vv, kc, vc = _pool_from_table(table, L, Hkv, d, 32, ps, 22)
    for t, page, slot in ex["token_locations"]:
        if t < L:
            assert np.array_equal(kc[page, slot], kk[t])
    gk, gv = oracle.paged_gather(kc, vc, np.array(table), L)
    assert np.array_equal(gk, kk) and np.array_equal(gv, vv)
    q = _rand((1, H, d), 23)
    bt = np.array([table + [-1] * 4], dtype=np.int32)
    o, lse = oracle.paged_decode(q, kc, vc, bt, np.array([L]), 0.35)
    # contiguous reference: the same logical tokens as a [1, Hkv, L, d] prefill, non-causal, one query row
    qp = np.zeros((1, H, L, d))
    qp[0, :, L - 1] = q[0]
    o2, l2 = oracle.attention_rows(qp, kk.transpose(1, 0, 2)[None], vv.transpose(1, 0, 2)[None], False, 0.35,
                                   [(0, h, L - 1) for h in range(H)])
    assert np.all(np.isfinite(o))
    assert np.allclose(o[0], o2, rtol=0, atol=1e-14) and np.allclose(lse[0], l2, rtol=0, atol=1e-14)


def pin_decode_equals_causal_prefill_last_row():
    """Decode for a sequence equals the last row of causal prefill over the same L tokens."""
    H, Hkv, d, L, ps = 4, 2, 8, 45, 16
    table = [5, 0, 3]
    kk, vv, kc, vc = _pool_from_table(table, L, Hkv, d, 6, ps, 24)
    qfull = _rand((1, H, L, d), 25)
    o, lse = oracle.paged_decode(qfull[:, :, L - 1], kc, vc, np.array([table], dtype=np.int32), [L], 0.5)
    op, lp = oracle.attention(qfull, kk.transpose(1, 0, 2)[None], vv.transpose(1, 0, 2)[None], True, 0.5)
    assert np.allclose(o[0], op[0, :, L - 1], rtol=0, atol=1e-13)
    assert np.allclose(lse[0], lp[0, :, L - 1], rtol=0, atol=1e-13)


def pin_decode_single_token():
    """L = 1: O is the one V row at (block_table[0], slot 0); LSE = scale * q . k."""
    H, Hkv, d = 2, 1, 6
    kk, vv, kc, vc = _pool_from_table([3], 1, Hkv, d, 4, 16, 26)
    q = _rand((1, H, d), 27)
    o, lse = oracle.paged_decode(q, kc, vc, np.array([[3, -1]], dtype=np.int32), [1], 0.25)
    for h in range(H):
        assert np.array_equal(o[0, h], vc[3, 0, 0])
        assert abs(lse[0, h] - 0.25 * math.fsum(q[0, h] * kc[3, 0, 0])) < 1e-14


def pin_decode_empty_sequence():
    """L = 0: the empty sum, O = 0 and LSE = -inf."""
    kc = np.full((2, 16, 1, 4), np.nan)
    o, lse = oracle.paged_decode(_rand((1, 2, 4), 28), kc, kc, np.array([[-1]], dtype=np.int32), [0], 1.0)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def pin_decode_page_permutation_invariance():
    """Moving the same logical tokens to other physical pages changes nothing."""
    H, Hkv, d, L = 4, 2, 8, 70
    q = _rand((1, H, d), 29)
    t1, t2 = [9, 2, 7, 0, 4], [1, 8, 3, 6, 5]
    _, _, kc1, vc1 = _pool_from_table(t1, L, Hkv, d, 10, 16, 30)
    _, _, kc2, vc2 = _pool_from_table(t2, L, Hkv, d, 10, 16, 30)
    o1, l1 = oracle.paged_decode(q, kc1, vc1, np.array([t1]), [L], 0.3)
    o2, l2 = oracle.paged_decode(q, kc2, vc2, np.array([t2]), [L], 0.3)
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------- chunked paged prefill pins

def _chunked_case(ctxs, qlens, H, Hkv, d, num_pages, seed, ps=16):
    """Sequences with ctx tokens placed by hand in shuffled pages (NaN elsewhere) and chunks of new tokens."""
    rng = np.random.default_rng(seed)
    S = len(ctxs)
    max_pages = max((c + n + ps - 1) // ps for c, n in zip(ctxs, qlens))
    perm = rng.permutation(num_pages)
    bt = np.full((S, max_pages), -1, dtype=np.int32)
    kc = np.full((num_pages, ps, Hkv, d), np.nan)
    vc = np.full((num_pages, ps, Hkv, d), np.nan)
    ctx_k, ctx_v, used = [], [], 0
    for s, (c, n) in enumerate(zip(ctxs, qlens)):
        npg = (c + n + ps - 1) // ps
        bt[s, :npg] = perm[used:used + npg]
        used += npg
        kk, vv = rng.standard_normal((c, Hkv, d)), rng.standard_normal((c, Hkv, d))
        for t in range(c):
            kc[bt[s, t // ps], t % ps] = kk[t]
            vc[bt[s, t // ps], t % ps] = vv[t]
        ctx_k.append(kk)
        ctx_v.append(vv)
    T = sum(qlens)
    q_start = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = rng.standard_normal((T, H, d))
    k_new, v_new = rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hkv, d))
    return dict(q=q, k_new=k_new, v_new=v_new, kc=kc, vc=vc, bt=bt, ctx=np.array(ctxs, dtype=np.int32),
                q_start=q_start, ctx_k=ctx_k, ctx_v=ctx_v)


def _run_chunked(c, scale):
    return oracle.paged_prefill(c["q"], c["k_new"], c["v_new"], c["kc"], c["vc"], c["bt"], c["ctx"], c["q_start"],
                                scale)


def pin_chunked_prefill_torch_sdpa():
    """Each sequence against torch's CPU float64 SDPA over its context followed by its chunk (joined by
    plain concatenation), with the end-aligned causal mask built by loops as a boolean matrix."""
    import torch
    import torch.nn.functional as F
    for ctxs, qlens, H, Hkv, d, seed in [([0, 20, 37], [5, 16, 1], 4, 2, 8, 40), ([70, 3], [33, 64], 6, 3, 16, 41),
                                         ([16], [17], 2, 2, 4, 42)]:
        c = _chunked_case(ctxs, qlens, H, Hkv, d, 40, seed)
        o, lse, _, _ = _run_chunked(c, 0.37)
        for s, (ctx, n) in enumerate(zip(ctxs, qlens)):
            lo = int(c["q_start"][s])
            kfull = np.concatenate([c["ctx_k"][s], c["k_new"][lo:lo + n]])  # [ctx + n, Hkv, d]
            vfull = np.concatenate([c["ctx_v"][s], c["v_new"][lo:lo + n]])
            allowed = torch.zeros((n, ctx + n), dtype=torch.bool)
            for i in range(n):
                for j in range(ctx + i + 1):
                    allowed[i, j] = True
            qt = torch.from_numpy(c["q"][lo:lo + n].transpose(1, 0, 2)[None].copy())
            kt = torch.from_numpy(kfull.transpose(1, 0, 2)[None].copy())
            vt = torch.from_numpy(vfull.transpose(1, 0, 2)[None].copy())
            ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=0.37, enable_gqa=True)
            ref = ref[0].numpy().transpose(1, 0, 2)
            assert np.allclose(o[lo:lo + n], ref, rtol=0, atol=1e-10)
            assert np.all(np.isfinite(lse[lo:lo + n]))


def pin_append_block_table_worked_example():
    """The pages' table [17, 4, 29, 8] with 40 tokens cached and a chunk of 9: the chunk lands at the hand-derived
    locations (token 47 at block 29 slot 15, token 48 at block 8 slot 0), and nothing else changes."""
    ex = _golden_example()
    table, ps = ex["physical_blocks"], ex["page_size"]
    Hkv, d, ctx, n = 2, 4, 40, 9
    kk, vv, kc, vc = _pool_from_table(table, ctx, Hkv, d, 32, ps, 43)
    k_new, v_new = _rand((n, Hkv, d), 44), _rand((n, Hkv, d), 45)
    bt = np.array([table], dtype=np.int32)
    kc2, vc2 = oracle.paged_append(kc, vc, k_new, v_new, bt, np.array([ctx]), np.array([0, n]))
    where = {t: (page, slot) for t, page, slot in ex["token_locations"]}
    for t in (47, 48):
        page, slot = where[t]
        assert np.array_equal(kc2[page, slot], k_new[t - ctx]) and np.array_equal(vc2[page, slot], v_new[t - ctx])
    changed = ~((kc2 == kc) | (np.isnan(kc2) & np.isnan(kc)))
    assert changed.sum() == n * Hkv * d
    assert np.array_equal(kc2[29, 8:16], k_new[:8]) and np.array_equal(kc2[8, 0], k_new[8])
    assert np.array_equal(kc2[17], kc[17], equal_nan=True) and np.array_equal(kc2[4], kc[4], equal_nan=True)
    assert np.array_equal(kc, _pool_from_table(table, ctx, Hkv, d, 32, ps, 43)[2], equal_nan=True)  # input untouched


def pin_chunk_of_one_token_is_decode():
    """A chunk of one token is a decode step: it equals decode over the appended cache with L = ctx + 1."""
    ctxs = [0, 15, 16, 33]
    c = _chunked_case(ctxs, [1] * 4, 4, 2, 8, 20, 46)
    o, lse, kc2, vc2 = _run_chunked(c, 0.41)
    od, ld = oracle.paged_decode(c["q"], kc2, vc2, c["bt"], c["ctx"] + 1, 0.41)
    assert np.allclose(o, od, rtol=0, atol=1e-14) and np.allclose(lse, ld, rtol=0, atol=1e-14)


def pin_chunk_without_context_is_causal_prefill():
    """With nothing cached, a chunk is causal prefill over its own tokens."""
    c = _chunked_case([0], [29], 4, 2, 8, 8, 47)
    o, lse, _, _ = _run_chunked(c, 0.3)
    op, lp = oracle.attention(c["q"].transpose(1, 0, 2)[None], c["k_new"].transpose(1, 0, 2)[None],
                              c["v_new"].transpose(1, 0, 2)[None], True, 0.3)
    assert np.allclose(o, op[0].transpose(1, 0, 2), rtol=0, atol=1e-13)
    assert np.allclose(lse, lp[0].T, rtol=0, atol=1e-13)


def pin_chunking_does_not_change_results():
    """A sequence prefilled as one chunk, or as two chunks where the second sees the first through the cache,
    gives the same outputs for the second chunk's tokens and the same cache."""
    H, Hkv, d, n1, n2 = 4, 2, 8, 23, 27
    c = _chunked_case([0], [n1 + n2], H, Hkv, d, 10, 48)
    o, lse, kc_a, vc_a = _run_chunked(c, 0.5)
    # first chunk alone, then the second with ctx = n1
    o1, _, kc1, vc1 = oracle.paged_prefill(c["q"][:n1], c["k_new"][:n1], c["v_new"][:n1], c["kc"], c["vc"], c["bt"],
                                           np.array([0]), np.array([0, n1]), 0.5)
    o2, l2, kc2, vc2 = oracle.paged_prefill(c["q"][n1:], c["k_new"][n1:], c["v_new"][n1:], kc1, vc1, c["bt"],
                                            np.array([n1]), np.array([0, n2]), 0.5)
    assert np.allclose(o2, o[n1:], rtol=0, atol=1e-13) and np.allclose(l2, lse[n1:], rtol=0, atol=1e-13)
    assert np.allclose(o1, o[:n1], rtol=0, atol=1e-13)
    assert np.array_equal(kc2, kc_a, equal_nan=True) and np.array_equal(vc2, vc_a, equal_nan=True)


def pin_chunked_prefill_brute_force_tiny():
    """Agreement with an fsum loop that walks the block table token by token (to 1e-12)."""
    ps = 16
    for ctxs, qlens, seed in [([3], [2], 49), ([16, 0], [1, 3], 50), ([31], [4], 51)]:
        H, Hkv, d = 2, 1, 3
        c = _chunked_case(ctxs, qlens, H, Hkv, d, 6, seed)
        o, lse, _, _ = _run_chunked(c, 0.7)
        for s, (ctx, n) in enumerate(zip(ctxs, qlens)):
            lo = int(c["q_start"][s])
            for i in range(n):
                for h in range(H):
                    def key(t):
                        if t < ctx:
                            return c["kc"][c["bt"][s, t // ps], t % ps, 0], c["vc"][c["bt"][s, t // ps], t % ps, 0]
                        return c["k_new"][lo + t - ctx, 0], c["v_new"][lo + t - ctx, 0]
                    sc = [0.7 * math.fsum(c["q"][lo + i, h] * key(t)[0]) for t in range(ctx + i + 1)]
                    m = max(sc)
                    w = [math.exp(x - m) for x in sc]
                    l = math.fsum(w)
                    want = [math.fsum(w[t] * key(t)[1][e] for t in range(ctx + i + 1)) / l for e in range(d)]
                    assert np.allclose(o[lo + i, h], want, rtol=0, atol=1e-12)
                    assert abs(lse[lo + i, h] - (m + math.log(l))) < 1e-12


# ------------------------------------------------------------------------------ fp8 pins

def pin_e4m3_decode_matches_torch():
    """All 256 E4M3 codes decode to torch's float8_e4m3fn values (NaN codes to NaN)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.e4m3_bits_to_f64(codes), want, equal_nan=True)


def pin_e4m3_decode_closed_forms():
    """Hand-decoded E4M3 codes: 1, 448 (largest), 2^-6 (smallest normal), 2^-9 and 7 * 2^-9 (subnormals),
    -2, signed zero and NaN."""
    codes = np.array([0x38, 0x7E, 0x08, 0x01, 0x07, 0xC0, 0x00, 0x80, 0x7F, 0xFF], dtype=np.uint8)
    got = oracle.e4m3_bits_to_f64(codes)
    want = [1.0, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, -2.0, 0.0, -0.0]
    assert np.array_equal(got[:8], want) and np.signbit(got[7]) and np.all(np.isnan(got[8:]))


def _fp8_case(B, H, Hkv, N, d, seed):
    from workloads import quantize_e4m3
    rng = np.random.default_rng(seed)
    q8, qs = quantize_e4m3(rng.standard_normal((B, H, N, d)))
    k8, ks = quantize_e4m3(rng.standard_normal((B, Hkv, N, d)))
    v8, vs = quantize_e4m3(rng.standard_normal((B, Hkv, N, d)))
    return q8, k8, np.ascontiguousarray(np.swapaxes(v8, -1, -2)), qs, ks, vs


def pin_fp8_attention_torch_sdpa():
    """FP8 attention equals torch's CPU float64 SDPA over the inputs decoded by torch (float8_e4m3fn), scaled, with
    V taken back from its transpose by torch."""
    import torch
    import torch.nn.functional as F
    for (B, H, Hkv, N, d, causal, seed) in [(1, 4, 2, 16, 16, True, 60), (2, 2, 2, 24, 8, False, 61),
                                            (1, 6, 3, 33, 16, True, 62)]:
        q8, k8, vt8, qs, ks, vs = _fp8_case(B, H, Hkv, N, d, seed)
        o, _ = oracle.attention_fp8(q8, k8, vt8, causal, 0.3, qs, ks, vs)

        def dec(x):
            return torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.float64)
        ref = F.scaled_dot_product_attention(dec(q8) * qs, dec(k8) * ks, dec(vt8).transpose(-1, -2) * vs,
                                             is_causal=causal, scale=0.3, enable_gqa=True).numpy()
        assert np.allclose(o, ref, rtol=0, atol=1e-10)


def pin_fp8_scales_enter_linearly():
    """Doubling q_scale equals doubling the softmax scale; doubling v_scale doubles O and leaves LSE alone."""
    q8, k8, vt8, qs, ks, vs = _fp8_case(1, 2, 1, 20, 8, 63)
    o, lse = oracle.attention_fp8(q8, k8, vt8, True, 0.2, qs, ks, vs)
    o2, lse2 = oracle.attention_fp8(q8, k8, vt8, True, 0.4, qs, ks, vs)
    o3, lse3 = oracle.attention_fp8(q8, k8, vt8, True, 0.2, 2 * qs, ks, vs)
    o4, lse4 = oracle.attention_fp8(q8, k8, vt8, True, 0.2, qs, ks, 2 * vs)
    assert np.allclose(o2, o3, rtol=0, atol=1e-13) and np.allclose(lse2, lse3, rtol=0, atol=1e-13)
    assert np.allclose(o4, 2 * o, rtol=0, atol=1e-13) and np.array_equal(lse4, lse)


def _fp8_decode_case(seed):
    """A small FP8 paged cache: 3 sequences (one empty-tailed page each), 2 KV heads, 5 of 9 pages used."""
    rng = np.random.default_rng(seed)
    lens = np.array([21, 1, 30])
    table = np.array([[4, 7], [0, -1], [8, 2]], dtype=np.int32)
    k8 = rng.integers(0, 256, size=(9, 16, 2, 8), dtype=np.uint8)
    v8 = rng.integers(0, 256, size=(9, 16, 2, 8), dtype=np.uint8)
    for x in (k8, v8):  # NaN codes only where no token sits
        x[(x & 0x7F) == 0x7F] = 0x3C
        for s, L in enumerate(lens):
            for t in range(L, 32):
                if t // 16 < 2 and table[s, t // 16] >= 0:
                    x[table[s, t // 16], t % 16] = 0x7F
    q = _rand((3, 4, 8), seed + 1)
    return q, k8, v8, table, lens


def pin_fp8_decode_is_decode_of_the_values():
    """With unit scales, FP8 decode is the bfloat16 decode of the same numbers, decoded here by torch's
    float8_e4m3fn (every finite E4M3 value is a bfloat16); NaN codes in unused slots are never read."""
    import torch
    q, k8, v8, table, lens = _fp8_decode_case(50)
    o8, l8 = oracle.paged_decode_fp8(q, k8, v8, 1.0, 1.0, table, lens, 0.7)
    as_bf16 = lambda x: torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
    o, l = oracle.paged_decode(q, as_bf16(k8), as_bf16(v8), table, lens, 0.7)
    assert np.all(np.isfinite(o8)) and np.all(np.isfinite(l8))
    assert np.allclose(o8, o, rtol=0, atol=1e-13) and np.allclose(l8, l, rtol=0, atol=1e-13)


def pin_fp8_decode_scales_enter_linearly():
    """k_scale multiplies every score (the same as multiplying the softmax scale); v_scale multiplies the
    output and leaves the LSE alone."""
    q, k8, v8, table, lens = _fp8_decode_case(51)
    base_o, base_l = oracle.paged_decode_fp8(q, k8, v8, 1.0, 1.0, table, lens, 0.6)
    o, l = oracle.paged_decode_fp8(q, k8, v8, 1.0, 4.0, table, lens, 0.6)
    assert np.allclose(o, 4.0 * base_o, rtol=0, atol=1e-12) and np.allclose(l, base_l, rtol=0, atol=0)
    o, l = oracle.paged_decode_fp8(q, k8, v8, 0.25, 1.0, table, lens, 0.6)
    o2, l2 = oracle.paged_decode_fp8(q, k8, v8, 1.0, 1.0, table, lens, 0.15)
    assert np.allclose(o, o2, rtol=0, atol=1e-13) and np.allclose(l, l2, rtol=0, atol=1e-13)



def pin_fp8_rows_equal_full():
    """attention_fp8_rows returns exactly the selected rows of attention_fp8 (the same dequantisation,
    V taken back from its transpose the same way), causal and not, with grouped KV heads."""
    q8, k8, vt8, qs, ks, vs = _fp8_case(2, 6, 2, 48, 16, 64)
    rows = [(0, 0, 0), (1, 5, 47), (0, 3, 16), (1, 2, 31), (0, 4, 1), (1, 0, 46)]
    for causal in (False, True):
        o, lse = oracle.attention_fp8(q8, k8, vt8, causal, 0.3, qs, ks, vs)
        ro, rl = oracle.attention_fp8_rows(q8, k8, vt8, causal, 0.3, qs, ks, vs, rows)
        for n, (b, h, i) in enumerate(rows):
            assert np.allclose(ro[n], o[b, h, i], rtol=0, atol=1e-14)
            assert abs(rl[n] - lse[b, h, i]) < 1e-14


def pin_decode_seqs_subset_equals_full():
    """paged_decode and paged_decode_fp8 with seqs= return the full call's rows of those sequences, in the
    order asked for (repeats included)."""
    H, Hkv, d = 4, 2, 8
    tables = [[5, 0, 3], [1, 7, -1], [6, 2, 4]]
    lens = [45, 20, 33]
    rng = np.random.default_rng(31)
    kc, vc = rng.standard_normal((8, 16, Hkv, d)), rng.standard_normal((8, 16, Hkv, d))
    q = _rand((3, H, d), 32)
    bt = np.array(tables, dtype=np.int32)
    o, lse = oracle.paged_decode(q, kc, vc, bt, lens, 0.4)
    for seqs in ([2, 0], [1], [2, 2, 1, 0]):
        so, sl = oracle.paged_decode(q, kc, vc, bt, lens, 0.4, seqs=seqs)
        assert so.shape == (len(seqs), H, d)
        assert np.array_equal(so, o[seqs]) and np.array_equal(sl, lse[seqs])
    q, k8, v8, table, lens8 = _fp8_decode_case(52)
    o, lse = oracle.paged_decode_fp8(q, k8, v8, 0.5, 2.0, table, lens8, 0.7)
    for seqs in ([2, 0], [1, 1]):
        so, sl = oracle.paged_decode_fp8(q, k8, v8, 0.5, 2.0, table, lens8, 0.7, seqs=seqs)
        assert np.array_equal(so, o[seqs]) and np.array_equal(sl, lse[seqs])


def pin_chunked_seqs_subset_equals_full():
    """paged_prefill with seqs= returns the full call's chunk rows of those sequences, concatenated in the
    order asked for, and the same appended caches."""
    c = _chunked_case([40, 0, 17], [9, 21, 16], 4, 2, 8, 12, 33)
    o, lse, kc, vc = _run_chunked(c, 0.45)
    qs = c["q_start"]
    for seqs in ([2, 0], [1], [0, 2, 1]):
        so, sl, skc, svc = oracle.paged_prefill(c["q"], c["k_new"], c["v_new"], c["kc"], c["vc"], c["bt"], c["ctx"],
                                                qs, 0.45, seqs=seqs)
        want = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs])
        assert np.array_equal(so, o[want]) and np.array_equal(sl, lse[want])
        assert np.array_equal(skc, kc, equal_nan=True) and np.array_equal(svc, vc, equal_nan=True)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
