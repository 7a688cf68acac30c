"""GPU parity of paged_prefill (chunked prefill over a paged cache with the chunk appended), through
the C ABI, against the float64 oracle; the caches after the call are compared bit for bit."""

from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import paged_attention_attn_amd as paa
from gpu_util import assert_close_bf16, assert_close_lse, dev_bf16, dev_i32, host_f64
from workloads import BF16_NAN, WORKLOADS, ChunkedPrefillWorkload, chunked_prefill_inputs, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _to_dev(a):
    return {"q": dev_bf16(a["q"]), "k_new": dev_bf16(a["k_new"]), "v_new": dev_bf16(a["v_new"]),
            "k_cache": dev_bf16(a["k_cache"]), "v_cache": dev_bf16(a["v_cache"]),
            "block_table": dev_i32(a["block_table"]), "ctx_lens": dev_i32(a["ctx_lens"]),
            "q_start": dev_i32(a["q_start"])}


def _run(a, max_q_len=None):
    t = _to_dev(a)
    H = a["q"].shape[1]
    lse = torch.empty((a["q"].shape[0], H), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_prefill(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["block_table"],
                             t["ctx_lens"], t["q_start"], max_q_len=max_q_len, scale=a["scale"], lse=lse)
    torch.cuda.synchronize()
    kc = t["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    vc = t["v_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    return host_f64(o), lse.cpu().numpy().astype(np.float64), kc, vc


def _oracle(a, seqs=None):
    return oracle.paged_prefill(a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["block_table"],
                                a["ctx_lens"], a["q_start"], a["scale"], seqs=seqs)


def _check_all(a, max_q_len=None):
    o, lse, kc, vc = _run(a, max_q_len)
    ro, rl, rkc, rvc = _oracle(a)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)
    # the append is a copy of bf16 bit patterns: the caches must match exactly (NaN slots included)
    assert np.array_equal(kc, rkc) and np.array_equal(vc, rvc)


# (ctx lengths, chunk lengths) per case: contexts and chunks on and off page (16) and tile (64)
# boundaries, empty contexts, one-token chunks, an empty chunk, a chunk longer than one query tile
SMALL = [
    ([0, 5, 16, 64, 100], [37, 1, 16, 64, 129], 8, 2, 128),
    ([33, 0, 200], [200, 0, 7], 4, 4, 64),
    ([511, 17], [1, 300], 16, 4, 128),
    ([1000], [65], 6, 2, 64),
    ([0, 0, 0, 0], [128, 127, 129, 1], 2, 1, 128),
    # more than 64 key tiles: the per-wave window of page ids is refilled mid-sequence
    ([4100, 1], [60, 2], 2, 1, 128),
    ([4200, 70], [40, 3], 4, 2, 64),
]


@pytest.mark.parametrize("ctxs,qlens,H,Hkv,d", SMALL)
def test_paged_prefill_small_full_parity(ctxs, qlens, H, Hkv, d):
    w = ChunkedPrefillWorkload("small", len(ctxs), H, Hkv, d, 0, 0, 1, num_pages=400)
    _announce(f"paged prefill ctx{ctxs} q{qlens} H{H} Hkv{Hkv} d{d}")
    a = chunked_prefill_inputs(w, seed=sum(ctxs) + d, ctx_lens=ctxs, q_lens=qlens)
    _check_all(a)


# Grids of at least 1024 eight-wave workgroups (d = 128 takes the ping-pong kernel there): one per
# head-sharing width (4, 2, 1 query heads per workgroup); the last three reach that size through a
# loose max_q_len, so most of their workgroups leave at once.
LARGE = [
    ([0, 1, 15, 16, 17, 63, 64, 65, 500, 1000, 2047, 3, 300, 0, 777, 129],
     [512, 1, 0, 100, 511, 64, 65, 300, 129, 17, 2, 512, 256, 16, 400, 33], 32, 8, 128, 512),
    ([5, 0, 64, 1500, 31, 200, 16, 999], [300, 129, 0, 64, 1, 250, 77, 16], 16, 8, 128, 2048),
    ([700, 0, 48, 1], [700, 0, 257, 1], 8, 8, 128, 8192),
    # d = 64 (eight-wave lock-step kernel) with contexts past 64 key tiles
    ([4200, 0, 70, 3000], [10, 100, 300, 1], 8, 8, 64, 8192),
    # ping-pong kernel past 128 key tiles: the per-wave window of page ids moves twice
    ([9000, 100, 0, 5000], [64, 300, 2048, 1], 32, 8, 128, 2048),
]


@pytest.mark.parametrize("ctxs,qlens,H,Hkv,d,max_q_len", LARGE)
def test_paged_prefill_large_grid_full_parity(ctxs, qlens, H, Hkv, d, max_q_len):
    pages = sum(-(-(c + q) // 16) for c, q in zip(ctxs, qlens))
    w = ChunkedPrefillWorkload("large", len(ctxs), H, Hkv, d, 0, 0, 1, num_pages=max(600, pages + 64))
    _announce(f"paged prefill ctx{ctxs} q{qlens} H{H} Hkv{Hkv} d{d} max_q_len {max_q_len}")
    a = chunked_prefill_inputs(w, seed=sum(ctxs) + H, ctx_lens=ctxs, q_lens=qlens)
    _check_all(a, max_q_len)


@pytest.mark.parametrize("num_seqs,H,Hkv,d", [(300, 8, 8, 128), (256, 16, 8, 128), (300, 8, 2, 64), (200, 8, 2, 64)])
def test_paged_prefill_many_sequences(num_seqs, H, Hkv, d):
    """Sequences are taken heaviest first when there are at most 256 of them, in the given order
    beyond that; both orders against the oracle, with short ragged contexts and chunks."""
    rng = np.random.default_rng(num_seqs + d)
    ctxs = [int(x) for x in rng.integers(0, 60, size=num_seqs)]
    qlens = [int(x) for x in rng.integers(0, 40, size=num_seqs)]
    w = ChunkedPrefillWorkload("many", num_seqs, H, Hkv, d, 0, 0, 1, num_pages=2000)
    _announce(f"paged prefill {num_seqs} sequences H{H} Hkv{Hkv} d{d}")
    a = chunked_prefill_inputs(w, seed=num_seqs + d, ctx_lens=ctxs, q_lens=qlens)
    _check_all(a, max_q_len=64)


def test_paged_prefill_loose_max_q_len():
    """A max_q_len far above every chunk only adds workgroups that leave at once."""
    w = ChunkedPrefillWorkload("loose", 3, 8, 2, 128, 0, 0, 1, num_pages=200)
    _announce("paged prefill, loose max_q_len")
    a = chunked_prefill_inputs(w, seed=5, ctx_lens=[40, 0, 300], q_lens=[9, 70, 3])
    _check_all(a, max_q_len=1000)


def test_paged_prefill_block_table_worked_example():
    """The pages' table [17, 4, 29, 8]: 40 cached tokens and a chunk of 9 land at block 29 slots 8-15 and block 8
    slot 0 (positions 40..48), and the chunk's outputs match the oracle."""
    with open(os.path.join(GOLDEN, "block_table_example.json")) as f:
        ex = json.load(f)
    table = ex["physical_blocks"]
    w = ChunkedPrefillWorkload("golden", 1, 8, 2, 128, 0, 0, 1, num_pages=32)
    _announce("paged prefill, golden block table")
    full = chunked_prefill_inputs(w, seed=9, ctx_lens=[0], q_lens=[49])  # 49 tokens' q, k, v
    ctx = 40
    k_pool = np.full_like(full["k_cache"], BF16_NAN)
    v_pool = k_pool.copy()
    for t in range(ctx):  # the context, placed through the table by hand
        k_pool[table[t // 16], t % 16] = full["k_new"][t]
        v_pool[table[t // 16], t % 16] = full["v_new"][t]
    b = {"q": full["q"][ctx:], "k_new": full["k_new"][ctx:], "v_new": full["v_new"][ctx:], "k_cache": k_pool,
         "v_cache": v_pool, "block_table": np.array([table], dtype=np.int32),
         "ctx_lens": np.array([ctx], dtype=np.int32), "q_start": np.array([0, 9], dtype=np.int32), "scale": w.scale}
    o, lse, kc, vc = _run(b)
    assert np.array_equal(kc[29, 8:16], full["k_new"][40:48]) and np.array_equal(kc[8, 0], full["k_new"][48])
    assert np.array_equal(vc[29, 8:16], full["v_new"][40:48]) and np.array_equal(vc[8, 0], full["v_new"][48])
    ro, rl, rkc, _ = _oracle(b)
    assert np.array_equal(kc, rkc)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_chunks_then_decode_match_one_pass():
    """A sequence prefilled in three chunks through the cache, then a decode step, against the oracle over the
    whole sequence: every chunk's rows equal causal prefill rows, and decode sees the appended cache."""
    H, Hkv, d, n = 8, 2, 128, 300
    w = ChunkedPrefillWorkload("chunks", 1, H, Hkv, d, 0, 0, 1, num_pages=64)
    a = chunked_prefill_inputs(w, seed=11, ctx_lens=[0], q_lens=[n])
    t = _to_dev(a)
    _announce("three chunks, then decode")
    bounds = [0, 70, 71, 300]
    outs = []
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        o, _ = paa.paged_prefill(t["q"][c0:c1], t["k_new"][c0:c1], t["v_new"][c0:c1], t["k_cache"], t["v_cache"],
                                 t["block_table"], dev_i32(np.array([c0])), dev_i32(np.array([0, c1 - c0])),
                                 scale=a["scale"])
        outs.append(o)
    torch.cuda.synchronize()
    ro, rl, rkc, rvc = _oracle(a)  # one chunk of n with no context
    got = np.concatenate([host_f64(o) for o in outs])
    assert_close_bf16(got, ro)
    kc = t["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(kc, rkc)
    # decode one more query over the n cached tokens
    qb = f32_to_bf16_bits(np.random.default_rng(12).standard_normal((1, H, d)).astype(np.float32))
    od, _ = paa.paged_attn_decode(dev_bf16(qb), t["k_cache"], t["v_cache"], t["block_table"],
                                  dev_i32(np.array([n])), a["scale"])
    torch.cuda.synchronize()
    rod, _ = oracle.paged_decode(qb, rkc, rvc, a["block_table"], [n], a["scale"])
    assert_close_bf16(host_f64(od), rod)


@pytest.mark.timeout(300)
def test_paged_prefill_full_workload_whole():
    """16 sequences, contexts U[0, 4096], chunks of 512, H=32, Hkv=8, d=128: every chunk row of every
    sequence against the oracle, and the whole cache against the oracle's append."""
    w = WORKLOADS["chunked_prefill_s16h32kv8d128_ctx0to4096_q512"]
    _announce(w.name)
    a = chunked_prefill_inputs(w, seed=0)
    o, lse, kc, vc = _run(a, a["max_q_len"])
    ro, rl, rkc, rvc = oracle_pool.paged_prefill(a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"],
                                                 a["block_table"], a["ctx_lens"], a["q_start"], a["scale"])
    st = assert_close_bf16(o, ro)
    st.update(assert_close_lse(lse, rl))
    assert np.array_equal(kc, rkc) and np.array_equal(vc, rvc)
    _announce(f"{w.name}: {st}")


def test_paged_prefill_repeat_is_bitwise_identical():
    """The full chunked workload twice on the same buffers: the second call appends the same rows again, so
    the caches are unchanged, and O and LSE repeat bit for bit (no atomics; fixed summation order)."""
    w = WORKLOADS["chunked_prefill_s16h32kv8d128_ctx0to4096_q512"]
    _announce(f"{w.name}: two calls")
    a = chunked_prefill_inputs(w, seed=4)
    t = _to_dev(a)
    H = a["q"].shape[1]
    outs = []
    for _ in range(2):
        lse = torch.empty((a["q"].shape[0], H), dtype=torch.float32, device="cuda:0")
        o, _ = paa.paged_prefill(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["block_table"],
                                 t["ctx_lens"], t["q_start"], max_q_len=a["max_q_len"], scale=a["scale"], lse=lse)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.cpu().numpy().view(np.uint32),
                     t["k_cache"].view(torch.int16).cpu().numpy(), t["v_cache"].view(torch.int16).cpu().numpy()))
    for x, y in zip(outs[0], outs[1]):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_paged_prefill_poisoned_slots_change_no_bit(d):
    """NaN in every cache slot no context token occupies (including the slots the chunk is appended to)
    against zeros there: O and LSE come out with the same bits, on a small grid (lock-step kernel, d=64)
    and the full workload's shape (ping-pong kernel, d=128)."""
    if d == 128:
        w = WORKLOADS["chunked_prefill_s16h32kv8d128_ctx0to4096_q512"]
    else:
        w = ChunkedPrefillWorkload("poison64", 6, 8, 2, 64, 0, 1500, 300, num_pages=1000)
    _announce(f"paged prefill d{d}: poisoned against zero-filled slots")
    o1, l1, _, _ = _run(chunked_prefill_inputs(w, seed=8, poison=True))
    o0, l0, _, _ = _run(chunked_prefill_inputs(w, seed=8, poison=False))
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, o0) and np.array_equal(l1, l0)


# (ctx lengths, chunk lengths, H, Hkv): a small grid (lock-step kernel) and one of 1024 eight-wave units
# (ping-pong kernel: 64 sequences x 8 KV heads x 2 query tiles)
OOB = [([37, 0, 300, 64], [50, 20, 129, 1], 8, 2),
       ([(37 * s) % 301 for s in range(64)], [128 if s % 3 else 65 for s in range(64)], 32, 8)]


@pytest.mark.parametrize("bad", [-1, "pool"])
@pytest.mark.parametrize("case", range(len(OOB)))
def test_paged_prefill_pages_outside_pool_are_not_written(case, bad):
    """Block-table entries of the chunk-only blocks set outside [0, num_pages) (no room reserved for the
    chunk): those rows are not appended and no other cache byte changes; rows that fall in the last
    context block (a valid page) are appended; O and LSE are unaffected, since no key position at or
    past the context length is read from the cache."""
    ctxs, qlens, H, Hkv = OOB[case]
    w = ChunkedPrefillWorkload("oob", len(ctxs), H, Hkv, 128, 0, 300, 0, num_pages=2048)
    a = chunked_prefill_inputs(w, seed=21 + case, ctx_lens=ctxs, q_lens=qlens)
    _announce(f"paged_prefill pages outside the pool: {len(ctxs)} sequences, H{H} Hkv{Hkv} ({bad})")
    ro, rl, _, _ = _oracle(a)
    bt = a["block_table"].copy()
    num_pages = a["k_cache"].shape[0]
    for s, c in enumerate(ctxs):
        first_chunk_only = -(-c // 16)  # blocks from here on hold no context token
        bt[s, first_chunk_only:] = -1 if bad == -1 else num_pages + 5 + s
    b = dict(a, block_table=bt)
    o, lse, kc, vc = _run(b)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)
    # expected caches: the inputs with only the rows whose page is valid appended
    ekc, evc = a["k_cache"].copy(), a["v_cache"].copy()
    for s, c in enumerate(ctxs):
        lo = int(a["q_start"][s])
        for i in range(qlens[s]):
            pos = c + i
            page = int(bt[s, pos // 16])
            if 0 <= page < num_pages:
                ekc[page, pos % 16] = a["k_new"][lo + i]
                evc[page, pos % 16] = a["v_new"][lo + i]
    assert np.array_equal(kc, ekc) and np.array_equal(vc, evc)
