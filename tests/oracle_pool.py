"""Runs the float64 oracle over the independent slices of a large workload in a thread pool.

Test infrastructure only.  The oracle's arithmetic is untouched: every slice is one ordinary oracle
call on the inputs of one (batch entry, query head) with its KV head, or of one sequence, and the
results are written back in place.  NumPy's matrix products and elementwise loops release the
interpreter lock, so with BLAS held to one thread per call the slices run in parallel on the host
cores; this keeps whole-output checks of the largest workloads to tens of seconds.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool(fn, jobs):
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers()) as ex:
        for _ in ex.map(fn, jobs):
            pass


def _per_head(call, B, H, Hkv, N, d_v):
    """Runs call(b, h, g) -> (O [N, d_v], LSE [N]) for every (b, h) and gathers the results."""
    o = np.empty((B, H, N, d_v))
    lse = np.empty((B, H, N))
    group = H // Hkv

    def run(bh):
        b, h = bh
        o[b, h], lse[b, h] = call(b, h, h // group)

    _pool(run, [(b, h) for b in range(B) for h in range(H)])
    return o, lse


def attention(q, k, v, causal, scale):
    """oracle.attention, one (b, h) per call."""
    B, H, N, _ = q.shape
    Hkv = k.shape[1]

    def call(b, h, g):
        ro, rl = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], causal, scale)
        return ro[0, 0], rl[0, 0]
    return _per_head(call, B, H, Hkv, N, v.shape[3])


def attention_window(q, k, v, window, n_global, scale):
    """oracle.attention_window, one (b, h) per call."""
    B, H, N, _ = q.shape
    Hkv = k.shape[1]

    def call(b, h, g):
        ro, rl = oracle.attention_window(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], window,
                                         n_global, scale)
        return ro[0, 0], rl[0, 0]
    return _per_head(call, B, H, Hkv, N, v.shape[3])


def attention_fp8(q8, k8, vt8, causal, scale, q_scale, k_scale, v_scale):
    """oracle.attention_fp8, one (b, h) per call."""
    B, H, N, _ = q8.shape
    Hkv = k8.shape[1]

    def call(b, h, g):
        ro, rl = oracle.attention_fp8(q8[b:b + 1, h:h + 1], k8[b:b + 1, g:g + 1], vt8[b:b + 1, g:g + 1], causal,
                                      scale, q_scale, k_scale, v_scale)
        return ro[0, 0], rl[0, 0]
    return _per_head(call, B, H, Hkv, N, vt8.shape[2])


def _per_seq(call, S):
    parts = [None] * S
    _pool(lambda s: parts.__setitem__(s, call(s)), range(S))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale):
    """oracle.paged_decode, one sequence per call (its seqs= subset)."""
    return _per_seq(lambda s: oracle.paged_decode(q, k_cache, v_cache, block_table, seq_lens, scale, seqs=[s]),
                    len(seq_lens))


def paged_decode_fp8(q, k8, v8, k_scale, v_scale, block_table, seq_lens, scale):
    """oracle.paged_decode_fp8, one sequence per call (its seqs= subset)."""
    return _per_seq(lambda s: oracle.paged_decode_fp8(q, k8, v8, k_scale, v_scale, block_table, seq_lens, scale,
                                                      seqs=[s]), len(seq_lens))


def paged_prefill(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens, q_start, scale):
    """oracle.paged_prefill's O and LSE, one sequence per call (its seqs= subset), and the caches after the
    append (from one oracle.paged_append call)."""
    o, lse = _per_seq(lambda s: oracle.paged_prefill(q, k_new, v_new, k_cache, v_cache, block_table, ctx_lens,
                                                     q_start, scale, seqs=[s])[:2], len(ctx_lens))
    kc, vc = oracle.paged_append(k_cache, v_cache, k_new, v_new, block_table, ctx_lens, q_start)
    return o, lse, kc, vc
