"""Plain float64 attention oracle (test infrastructure only; see the package docstring).

Sources (the pages this follows; cited by page title and section):

* "Fast Attention Kernels and Operator Fusion", section "FlashAttention-Style
  Kernels": attention with an additive mask M is softmax(Q K^T / sqrt(d) + M) V.
  The scale is passed in (it is 1/sqrt(d) in every workload used here).  The
  causal mask is the M whose entries are 0 where key j <= query i and -inf
  elsewhere (the ``is_causal=True`` call shown in the same section).
* "Kernel Fusion and Custom Kernels", section "3. FlashAttention: The Milestone
  of Fusion", v1: the softmax is the numerically stable one (shift each row by
  its maximum before exponentiating).
* "Fast Attention Kernels and Operator Fusion", section "Paged Attention
  Kernels": a sequence's KV cache lives in fixed-size physical blocks; logical
  block b of a sequence is stored in physical block ``block_table[b]``, and a
  kernel must translate each logical token position through that table.  The
  block size in the pages' serving example is 16 tokens.

Readings taken where the pages are silent:

* LSE is the natural log of the sum of exp over the scaled, masked scores of
  a row: LSE_i = m_i + ln(l_i), with m_i the row max and l_i the shifted sum.
* Layout: Q, O are [B, H, N, d]; K, V are [B, Hkv, N, d]; LSE is [B, H, N].
* Grouped heads: query head h reads KV head floor(h / (H / Hkv)); H % Hkv == 0.
* Causal alignment: query and key lengths are equal, key j is visible to
  query i iff j <= i.
* Decode: one query per sequence at the last position; it sees all L keys.
  K/V caches are [num_pages, page_size, Hkv, d]; token t of sequence s lives
  at page ``block_table[s, t // page_size]``, slot ``t % page_size``; slots at
  t >= L are never read.
* An empty key set (L = 0) gives O = 0 and LSE = -inf (the empty sum).
* Chunked prefill over a paged cache: a sequence holds ctx tokens in its pages
  and brings a chunk of new tokens (queries, keys, values).  The chunk's keys and
  values are appended at positions ctx, ctx + 1, ...; chunk query i sits at
  position ctx + i and sees positions 0 .. ctx + i (the causal mask aligned at
  the end, so that a chunk of one token is a decode step and a chunk with no
  context is causal prefill).  Chunk tokens are packed [T, heads, d] with
  sequence s owning rows q_start[s] .. q_start[s+1]-1.
* Sliding window with global tokens ("Kernel Fusion and Custom Kernels",
  section "4. FlashInfer", block-sparse masks: the Longformer pattern of a
  sliding window plus global tokens), read under the causal mask: key j is
  visible to query i iff j <= i and (i - j < window or j < n_global).  A
  global token's own row is causal anyway, so "global tokens see everything"
  adds nothing once the causal mask applies.

The helpers ``_kv_head``, ``_scores``, ``_apply_causal``, ``_window_mask``, ``_softmax``,
``_page_slot``, ``_chunk_positions`` and ``_selected`` are looked up at call time, so tests can plant a mistake in
one of them (on the CPU) and check that a pin catches it.
"""

from __future__ import annotations

import numpy as np

ROW_BLOCK = 512  # rows of one (b, h) computed at once; only bounds memory


def bf16_bits_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 numbers stored as their 16-bit patterns.

    bfloat16 is the upper half of an IEEE binary32, so the value is the
    binary32 whose upper 16 bits are the pattern and whose lower 16 are zero.
    """
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def _as_f64(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:  # bfloat16 bit patterns
        return bf16_bits_to_f64(x)
    return x.astype(np.float64, copy=False)


def _kv_head(h: int, H: int, Hkv: int) -> int:
    """KV head read by query head h: consecutive groups of H/Hkv query heads."""
    return h // (H // Hkv)


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for a block of query rows [r, d] against keys [n, d]."""
    return scale * (q_rows @ k.T)


def _window_mask(row_pos: np.ndarray, n_keys: int, window: int, n_global: int) -> np.ndarray:
    """True where key j is hidden from query row_pos[r]: causal, then outside the window unless global."""
    j = np.arange(n_keys)[None, :]
    i = row_pos[:, None]
    visible = (j <= i) & ((i - j < window) | (j < n_global))
    return ~visible


def _apply_causal(s: np.ndarray, row_pos: np.ndarray) -> None:
    """Additive causal mask in place: S[r, j] = -inf where key j > query position."""
    cols = np.arange(s.shape[1])
    s[cols[None, :] > row_pos[:, None]] = -np.inf


def _softmax(s: np.ndarray):
    """Row softmax shifted by the row max. Returns (P, m, l) with l = sum exp(S - m)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def _attend(q_rows, k, v, scale, row_pos=None):
    """O and LSE for query rows [r, d] over keys/values [n, d] (float64)."""
    r, d = q_rows.shape
    if k.shape[0] == 0:  # no visible key: empty sum
        return np.zeros((r, v.shape[1])), np.full(r, -np.inf)
    s = _scores(q_rows, k, scale)
    if row_pos is not None:
        _apply_causal(s, row_pos)
    p, m, l = _softmax(s)
    return p @ v, m + np.log(l)


def _check_heads(H: int, Hkv: int) -> None:
    if H <= 0 or Hkv <= 0 or H % Hkv != 0:
        raise ValueError(f"query heads {H} must be a positive multiple of KV heads {Hkv}")


def softmax_probs(q, k, causal: bool, scale: float, b: int = 0, h: int = 0):
    """The full probability matrix P [N, N] of one (batch, head); small N only."""
    q64, k64 = _as_f64(q), _as_f64(k)
    H, Hkv, N = q64.shape[1], k64.shape[1], q64.shape[2]
    _check_heads(H, Hkv)
    s = _scores(q64[b, h], k64[b, _kv_head(h, H, Hkv)], scale)
    if causal:
        _apply_causal(s, np.arange(N))
    return _softmax(s)[0]


def attention(q, k, v, causal: bool, scale: float):
    """Exact attention over [B, H, N, d] queries; returns (O [B,H,N,d], LSE [B,H,N]) in float64.

    Rows are processed ROW_BLOCK at a time; each row still sees its whole key
    range at once.  For causal rows the keys after the block's last row are
    left out: every one of them is masked (-inf) for every row of the block,
    so it would contribute exp(-inf) = 0.
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q64.shape
    Hkv = k64.shape[1]
    _check_heads(H, Hkv)
    o = np.zeros((B, H, N, v64.shape[3]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            for r0 in range(0, N, ROW_BLOCK):
                r1 = min(N, r0 + ROW_BLOCK)
                n_keys = r1 if causal else N
                pos = np.arange(r0, r1) if causal else None
                o[b, h, r0:r1], lse[b, h, r0:r1] = _attend(
                    q64[b, h, r0:r1], k64[b, g, :n_keys], v64[b, g, :n_keys], scale, pos)
    return o, lse


def attention_window(q, k, v, window: int, n_global: int, scale: float):
    """Causal attention with a sliding window and global tokens; (O, LSE) in float64.

    Key j is visible to query i iff j <= i and (i - j < window or j < n_global).
    Every row sees at least its own key (window >= 1).
    """
    if window < 1 or n_global < 0:
        raise ValueError("window must be >= 1 and n_global >= 0")
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q64.shape
    Hkv = k64.shape[1]
    _check_heads(H, Hkv)
    o = np.zeros((B, H, N, v64.shape[3]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            for r0 in range(0, N, ROW_BLOCK):
                r1 = min(N, r0 + ROW_BLOCK)
                pos = np.arange(r0, r1)
                s = _scores(q64[b, h, r0:r1], k64[b, g, :r1], scale)
                s[_window_mask(pos, r1, window, n_global)] = -np.inf
                p, m, l = _softmax(s)
                o[b, h, r0:r1], lse[b, h, r0:r1] = p @ v64[b, g, :r1], m + np.log(l)
    return o, lse


def attention_window_rows(q, k, v, window: int, n_global: int, scale: float, rows):
    """O and LSE of selected query rows ``(b, h, i)`` of :func:`attention_window`, one row at a time."""
    if window < 1 or n_global < 0:
        raise ValueError("window must be >= 1 and n_global >= 0")
    q_, k_, v_ = np.asarray(q), np.asarray(k), np.asarray(v)
    H, Hkv = q_.shape[1], k_.shape[1]
    _check_heads(H, Hkv)
    out_o, out_l = [], []
    for b, h, i in rows:
        g = _kv_head(int(h), H, Hkv)
        i = int(i)
        s = _scores(_as_f64(q_[b, h, i])[None, :], _as_f64(k_[b, g, :i + 1]), scale)
        s[_window_mask(np.array([i]), i + 1, window, n_global)] = -np.inf
        p, m, l = _softmax(s)
        out_o.append((p @ _as_f64(v_[b, g, :i + 1]))[0])
        out_l.append((m + np.log(l))[0])
    return np.array(out_o), np.array(out_l)


def attention_rows(q, k, v, causal: bool, scale: float, rows):
    """O and LSE of selected query rows only; ``rows`` is a sequence of (b, h, i).

    The same definition as :func:`attention`, one row at a time, for sampled
    checks at sizes where the full output would take too long.
    """
    q_, k_, v_ = np.asarray(q), np.asarray(k), np.asarray(v)
    H, Hkv = q_.shape[1], k_.shape[1]
    _check_heads(H, Hkv)
    out_o, out_l = [], []
    for b, h, i in rows:
        g = _kv_head(int(h), H, Hkv)
        n_keys = int(i) + 1 if causal else k_.shape[2]
        pos = np.array([int(i)]) if causal else None
        o, l = _attend(_as_f64(q_[b, h, i])[None, :], _as_f64(k_[b, g, :n_keys]),
                       _as_f64(v_[b, g, :n_keys]), scale, pos)
        out_o.append(o[0])
        out_l.append(l[0])
    return np.array(out_o), np.array(out_l)


def _page_slot(t: np.ndarray, page_size: int):
    """Logical token positions -> (logical block index, slot within the block)."""
    return t // page_size, t % page_size


def paged_gather(k_cache, v_cache, block_table_row, L: int):
    """Logical K, V [L, Hkv, d] of one sequence, read through its block table."""
    page_size = np.asarray(k_cache).shape[1]
    t = np.arange(int(L))
    blk, slot = _page_slot(t, page_size)
    pages = np.asarray(block_table_row)[blk]
    return _as_f64(np.asarray(k_cache)[pages, slot]), _as_f64(np.asarray(v_cache)[pages, slot])


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale: float, seqs=None):
    """Single-query decode over a paged KV cache.

    q [S, H, d]; k_cache, v_cache [num_pages, page_size, Hkv, d];
    block_table [S, max_pages]; seq_lens [S].  Returns (O [S,H,d], LSE [S,H])
    in float64 for the sequences in ``seqs`` (default: all), in that order.
    The query of sequence s sits at position L_s - 1 and sees all L_s keys.
    """
    return _decode_rows(q, np.asarray(k_cache).shape[2], np.asarray(v_cache).shape[3],
                        lambda s, L: paged_gather(k_cache, v_cache, np.asarray(block_table)[s], L),
                        seq_lens, scale, seqs)


def paged_decode_fp8(q, k8, v8, k_scale: float, v_scale: float, block_table, seq_lens, scale: float, seqs=None):
    """Single-query decode over an FP8 (E4M3) paged KV cache with per-tensor scales.

    k8, v8 [num_pages, page_size, Hkv, d] are e4m3 bytes; the cache holds their values times k_scale and
    v_scale (the FP8 inputs of "Kernel Fusion and Custom Kernels", section "3. FlashAttention: The
    Milestone of Fusion", v3, stored in the paged cache of "Fast Attention Kernels and Operator Fusion",
    section "Paged Attention Kernels").  The result is :func:`paged_decode` over those values, in float64;
    q stays bfloat16.  Only the tokens a sequence holds are decoded.
    """
    def gather(s, L):
        t = np.arange(int(L))
        blk, slot = _page_slot(t, np.asarray(k8).shape[1])
        pages = np.asarray(block_table)[s][blk]
        return (e4m3_bits_to_f64(np.asarray(k8)[pages, slot]) * float(k_scale),
                e4m3_bits_to_f64(np.asarray(v8)[pages, slot]) * float(v_scale))
    return _decode_rows(q, np.asarray(k8).shape[2], np.asarray(v8).shape[3], gather, seq_lens, scale, seqs)


def _selected(n_seqs: int, seqs):
    """The sequences a call covers, in the order asked for: all of them when seqs is None."""
    return range(n_seqs) if seqs is None else list(seqs)


def _decode_rows(q, Hkv: int, d_v: int, gather, seq_lens, scale: float, seqs):
    """One query row per sequence attending over the L_s keys/values gather(s, L_s) returns."""
    q64 = _as_f64(q)
    S, H, d = q64.shape
    _check_heads(H, Hkv)
    seqs = _selected(S, seqs)
    o = np.zeros((len(seqs), H, d_v))
    lse = np.zeros((len(seqs), H))
    for n, s in enumerate(seqs):
        L = int(seq_lens[s])
        kk, vv = gather(s, L)
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            o_h, l_h = _attend(q64[s, h][None, :], kk[:, g], vv[:, g], scale, None)
            o[n, h], lse[n, h] = o_h[0], l_h[0]
    return o, lse


def _chunk_positions(ctx: int, n: int) -> np.ndarray:
    """Logical positions of a chunk's n tokens in a sequence that already holds ctx tokens."""
    return ctx + np.arange(n)


def paged_append(k_cache, v_cache, k_new, v_new, block_table, ctx_lens, q_start):
    """The caches after each sequence's chunk of new tokens has been appended.

    Sequence s already holds ctx_lens[s] tokens; its chunk is rows q_start[s] ..
    q_start[s+1]-1 of k_new / v_new ([T, Hkv, d]).  Chunk token i goes to logical
    position ctx_lens[s] + i, which lives at page block_table[s, pos // page_size],
    slot pos % page_size (the block-table translation of "Fast Attention Kernels and
    Operator Fusion", section "Paged Attention Kernels"; appending to a cache is one of
    the features listed in "Kernel Fusion and Custom Kernels", section "4. FlashInfer").
    Returns new arrays of the caches' dtype; the inputs are left unchanged.
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    page_size = kc.shape[1]
    k_new, v_new = np.asarray(k_new), np.asarray(v_new)
    for s in range(len(ctx_lens)):
        lo, hi = int(q_start[s]), int(q_start[s + 1])
        pos = _chunk_positions(int(ctx_lens[s]), hi - lo)
        blk, slot = _page_slot(pos, page_size)
        pages = np.asarray(block_table)[s][blk]
        kc[pages, slot] = k_new[lo:hi]
        vc[pages, slot] = v_new[lo:hi]
    return kc, vc


def paged_prefill(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, q_start, scale: float, seqs=None):
    """Chunked prefill over a paged KV cache, with the chunk's keys/values appended.

    q [T, H, d] holds the chunks' queries, sequence s owning rows q_start[s] ..
    q_start[s+1]-1 (q_start has S + 1 entries); k_new, v_new [T, Hkv, d] are the same
    tokens' keys and values.  After :func:`paged_append`, chunk query i of sequence s
    sits at position ctx_lens[s] + i and attends, causally, over positions 0 .. ctx_lens[s] + i
    of its sequence: the cached context, then the chunk's own keys up to itself.
    Returns (O [T, H, d], LSE [T, H], k_cache_after, v_cache_after); O and LSE are
    float64 and cover the rows of the sequences in ``seqs`` (default: all), in order.
    """
    q64 = _as_f64(q)
    T, H, d = q64.shape
    Hkv = np.asarray(k_cache).shape[2]
    _check_heads(H, Hkv)
    kc, vc = paged_append(k_cache, v_cache, k_new, v_new, block_table, ctx_lens, q_start)
    seqs = _selected(len(ctx_lens), seqs)
    o, lse = [], []
    for s in seqs:
        lo, hi = int(q_start[s]), int(q_start[s + 1])
        ctx = int(ctx_lens[s])
        kk, vv = paged_gather(kc, vc, np.asarray(block_table)[s], ctx + hi - lo)
        o_s = np.zeros((hi - lo, H, np.asarray(v_cache).shape[3]))
        l_s = np.zeros((hi - lo, H))
        pos = _chunk_positions(ctx, hi - lo)
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            o_s[:, h], l_s[:, h] = _attend(q64[lo:hi, h], kk[:, g], vv[:, g], scale, pos)
        o.append(o_s)
        lse.append(l_s)
    o = np.concatenate(o) if o else np.zeros((0, H, d))
    lse = np.concatenate(lse) if lse else np.zeros((0, H))
    return o, lse, kc, vc


def e4m3_bits_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of OCP FP8 E4M3 (the "fn" variant: no infinities) numbers given as bytes.

    Sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
    subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; the largest finite value
    is 1.75 * 2^8 = 448.
    """
    b = np.asarray(x, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def _dequant_fp8(q8, k8, vt8, q_scale, k_scale, v_scale):
    """Values of the fp8 inputs: Q [B,H,N,d], K [B,Hkv,N,d], V from its transpose [B,Hkv,d,N]."""
    q = e4m3_bits_to_f64(q8) * float(q_scale)
    k = e4m3_bits_to_f64(k8) * float(k_scale)
    v = np.swapaxes(e4m3_bits_to_f64(vt8), -1, -2) * float(v_scale)
    return q, k, v


def attention_fp8(q8, k8, vt8, causal: bool, scale: float, q_scale: float, k_scale: float, v_scale: float):
    """Exact attention of FP8 inputs with per-tensor scales (the FP8 variant named in "Kernel Fusion and
    Custom Kernels", section "3. FlashAttention: The Milestone of Fusion", v3).

    q8 [B,H,N,d], k8 [B,Hkv,N,d] and vt8 [B,Hkv,d,N] (V transposed) are e4m3 bytes; the inputs are
    their values times q_scale, k_scale and v_scale.  The result is :func:`attention` of those values
    in float64 (any rounding of intermediate values, such as of the probabilities, is the method's
    approximation, not part of this definition).
    """
    q, k, v = _dequant_fp8(q8, k8, vt8, q_scale, k_scale, v_scale)
    return attention(q, k, v, causal, scale)


def attention_fp8_rows(q8, k8, vt8, causal: bool, scale: float, q_scale: float, k_scale: float, v_scale: float,
                       rows):
    """O and LSE of selected rows (b, h, i) of :func:`attention_fp8`."""
    q, k, v = _dequant_fp8(q8, k8, vt8, q_scale, k_scale, v_scale)
    return attention_rows(q, k, v, causal, scale, rows)
