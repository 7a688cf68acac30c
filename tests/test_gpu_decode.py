"""GPU parity of paged_attn_decode (through the C ABI) against the float64 oracle."""

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
from gpu_util import assert_close_bf16, assert_close_lse, decode_zero_query_expected, dev_bf16, dev_i32, host_f64
from workloads import WORKLOADS, DecodeWorkload, decode_inputs

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _run(a, H, num_pages=None):
    q = dev_bf16(a["q"])
    kc, vc = dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"])
    bt, lens = dev_i32(a["block_table"]), dev_i32(a["seq_lens"])
    lse = torch.empty((q.shape[0], H), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_attn_decode(q, kc, vc, bt, lens, a["scale"], num_pages=num_pages, lse=lse)
    torch.cuda.synchronize()
    return host_f64(o), lse.cpu().numpy().astype(np.float64), o


def _oracle(a, seqs=None):
    return oracle.paged_decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], a["scale"],
                               seqs=seqs)


def _partition_bound(a):
    """How far two page partitions of one decode may differ, elementwise, apart from terms in |O|: each
    range rounds its probabilities to bf16 (relative error up to 2^-8) against its own reference maximum,
    so a key's weight differs by up to 2^-7 of its value between partitions, and O by up to 2^-7 of
    (the softmax-weighted mean of |v| + |O|).  This returns the first part, from the oracle's decode over
    |V|; callers add 2^-6 |O| for the second part and the two outputs' own bf16 rounding."""
    abs_v = dict(a, v_cache=a["v_cache"] & np.uint16(0x7FFF))  # bf16 bits without the sign
    return 2.0 ** -7 * _oracle(abs_v)[0]


@pytest.mark.parametrize("d,H,Hkv", [(128, 32, 8), (64, 8, 8), (128, 16, 1), (64, 6, 2)])
def test_decode_small_ragged_lengths(d, H, Hkv):
    """Lengths around page and chunk edges, including 1 and 0; NaN in every unused slot."""
    lens = [1, 15, 16, 17, 31, 32, 33, 100, 257, 0, 700]
    w = DecodeWorkload("small", len(lens), H, Hkv, d, 1, 1024, 16, 200)
    _announce(f"decode d{d} H{H} Hkv{Hkv}")
    a = decode_inputs(w, seed=d + H, seq_lens=lens)
    o, lse, _ = _run(a, H)
    ro, rl = _oracle(a)
    assert np.all(o[9] == 0) and np.all(np.isneginf(lse[9]))  # L = 0
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_decode_block_table_worked_example():
    """The pages' block table [17, 4, 29, 8] with a partly filled last page."""
    with open(os.path.join(GOLDEN, "block_table_example.json")) as f:
        ex = json.load(f)
    w = DecodeWorkload("golden", 1, 8, 2, 128, 57, 57, ex["page_size"], 32)
    bt = np.array([ex["physical_blocks"]], dtype=np.int32)
    a = decode_inputs(w, seed=11, seq_lens=[57], block_table=bt)
    o, lse, _ = _run(a, 8)
    ro, rl = _oracle(a)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_decode_page_placement_is_invisible():
    """The same logical tokens in other physical pages give bitwise-equal outputs."""
    w = DecodeWorkload("perm", 3, 32, 8, 128, 200, 600, 16, 200)
    a = decode_inputs(w, seed=3)
    _, _, o1 = _run(a, 32)
    # move every used page to a new physical id via a permutation of the pool
    perm = np.random.default_rng(9).permutation(200)
    inv = np.argsort(perm)
    b = dict(a)
    b["k_cache"], b["v_cache"] = a["k_cache"][inv], a["v_cache"][inv]
    bt = a["block_table"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    b["block_table"] = bt
    _, _, o2 = _run(b, 32)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.timeout(300)
def test_decode_full_size_whole():
    """64 sequences, H=32, Hkv=8, d=128, lengths in [512, 8192], 40000-page pool: every sequence's O and LSE
    against the oracle."""
    w = WORKLOADS["paged_decode_s64h32kv8d128"]
    _announce(w.name)
    a = decode_inputs(w, seed=0)
    o, lse, _ = _run(a, w.H)
    ro, rl = oracle_pool.paged_decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"],
                                      a["scale"])
    st = assert_close_bf16(o, ro)
    st.update(assert_close_lse(lse, rl))
    _announce(f"{w.name}: {st}")


def test_decode_partition_does_not_change_results():
    """Unused block-table columns change how many equal page ranges the decode cuts the pages into
    (57, 120, then 256 here), so each sequence is split and merged differently; the result stays within
    the oracle's bars, and the partitions agree within the bound of _partition_bound (LSE: within fp32
    rounding)."""
    w = DecodeWorkload("split", 3, 32, 8, 128, 250, 300, 16, 80)
    a = decode_inputs(w, seed=23)
    assert a["block_table"].shape[1] == 19
    ro, rl = _oracle(a)
    outs = []
    for cols in (19, 40, 200):
        b = dict(a)
        bt = np.full((3, cols), -1, dtype=np.int32)
        bt[:, :19] = a["block_table"]
        b["block_table"] = bt
        o, lse, _ = _run(b, 32)
        assert_close_bf16(o, ro)
        assert_close_lse(lse, rl)
        outs.append((o, lse))
    bound = _partition_bound(a)
    for o, lse in outs[1:]:
        assert np.all(np.abs(o - outs[0][0]) <= bound + 2.0 ** -6 * np.maximum(np.abs(o), np.abs(outs[0][0])))
        assert np.max(np.abs(lse - outs[0][1])) <= 1e-5


def test_decode_out_of_range_page_id_is_not_read():
    """A page id past num_pages is never dereferenced; its tokens count as absent."""
    w = DecodeWorkload("oob", 1, 4, 1, 64, 48, 48, 16, 8)
    bt = np.array([[2, 5, 7]], dtype=np.int32)
    a = decode_inputs(w, seed=5, seq_lens=[48], block_table=bt)
    a["block_table"] = np.array([[2, 1000000, 7]], dtype=np.int32)
    o, lse, _ = _run(a, 4)
    # expected: attention over tokens 0..15 and 32..47 only
    keep = np.r_[0:16, 32:48]
    kk = oracle.bf16_bits_to_f64(np.concatenate([a["k_cache"][2], a["k_cache"][7]]))  # [32, 1, 64]
    vv = oracle.bf16_bits_to_f64(np.concatenate([a["v_cache"][2], a["v_cache"][7]]))
    assert len(keep) == kk.shape[0]
    q = oracle.bf16_bits_to_f64(a["q"])[0]  # [H, d]
    for h in range(4):
        ro, rl = oracle.attention_rows(q[None, h:h + 1, None, :], kk[None, :, 0][:, None], vv[None, :, 0][:, None],
                                       False, a["scale"], [(0, 0, 0)])
        assert_close_bf16(o[0, h][None], ro)
        assert_close_lse(lse[0, h:h + 1], rl)


def test_decode_argument_errors():
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device="cuda:0")
    kc = torch.zeros((4, 8, 1, 128), dtype=torch.bfloat16, device="cuda:0")  # page size 8
    bt = torch.zeros((2, 2), dtype=torch.int32, device="cuda:0")
    lens = torch.ones((2,), dtype=torch.int32, device="cuda:0")
    with pytest.raises(RuntimeError, match="page size"):
        paa.paged_attn_decode(q, kc, kc, bt, lens)
    kc16 = torch.zeros((4, 16, 1, 128), dtype=torch.bfloat16, device="cuda:0")
    ws = torch.zeros((8,), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(RuntimeError, match="workspace"):
        paa.paged_attn_decode(q, kc16, kc16, bt, lens, workspace=ws)
    with pytest.raises(TypeError):
        paa.paged_attn_decode(q, kc16, kc16, bt.long(), lens)


def test_decode_one_long_sequence_many_ranges():
    """One 8000-token sequence: its pages are cut across many workgroup ranges (more than 64 partials)."""
    w = DecodeWorkload("long1", 1, 32, 8, 128, 8000, 8000, 16, 600)
    _announce("decode one long sequence")
    a = decode_inputs(w, seed=12)
    o, lse, _ = _run(a, 32)
    ro, rl = _oracle(a)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


# Page lists of at least 8 pages per workgroup range (ranges = 2048 / Hkv) at three head layouts;
# lengths around page edges, an empty and a one-token sequence, ranges that straddle sequences.
LONG_LISTS = [
    (128, 32, 32, [3100, 1, 0, 2500, 17, 2600]),
    (64, 16, 16, [5000, 33, 7000, 0, 4600, 16]),
    (128, 32, 8, [9000, 8000, 1, 7000, 6600, 2000, 511]),
]


@pytest.mark.parametrize("d,H,Hkv,lens", LONG_LISTS)
def test_decode_long_lists_full_parity(d, H, Hkv, lens):
    w = DecodeWorkload("long", len(lens), H, Hkv, d, 0, max(lens), 16, sum(-(-n // 16) for n in lens) + 8)
    _announce(f"decode long page list d{d} H{H} Hkv{Hkv} lens {lens}")
    a = decode_inputs(w, seed=len(lens) + d, seq_lens=lens)
    o, lse, _ = _run(a, H)
    ro, rl = _oracle(a)
    empty = np.asarray(lens) == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_decode_garbage_workspace_and_repeats():
    """Whatever the workspace held before (here random bytes), repeated calls on it and a call on a
    fresh workspace give the same output and LSE, bit for bit."""
    d, H, Hkv, lens = LONG_LISTS[0]
    w = DecodeWorkload("long", len(lens), H, Hkv, d, 0, max(lens), 16, sum(-(-n // 16) for n in lens) + 8)
    _announce("decode garbage workspace and repeats")
    a = decode_inputs(w, seed=99, seq_lens=lens)
    q, kc, vc = dev_bf16(a["q"]), dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"])
    bt, sl = dev_i32(a["block_table"]), dev_i32(a["seq_lens"])
    need = paa.paged_attn_decode_workspace_size(len(lens), H, d, 16, a["block_table"].shape[1])
    gen = torch.Generator(device="cpu").manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=gen).to("cuda:0")
    outs = []
    for _ in range(4):
        lse = torch.empty((len(lens), H), dtype=torch.float32, device="cuda:0")
        o, _ = paa.paged_attn_decode(q, kc, vc, bt, sl, a["scale"], workspace=ws, lse=lse)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy().copy(), lse.cpu().numpy().copy()))
    lse = torch.empty((len(lens), H), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_attn_decode(q, kc, vc, bt, sl, a["scale"], lse=lse)  # fresh workspace
    torch.cuda.synchronize()
    outs.append((o.view(torch.int16).cpu().numpy().copy(), lse.cpu().numpy().copy()))
    for ob, lb in outs[1:]:
        assert np.array_equal(ob, outs[0][0]) and np.array_equal(lb.view(np.int32), outs[0][1].view(np.int32))
    ro, rl = _oracle(a)
    assert_close_bf16(host_f64(o), ro)
    assert_close_lse(outs[0][1].astype(np.float64), rl)


def test_decode_many_short_sequences():
    """600 sequences (more than one scan chunk per workgroup) of 0..40 tokens."""
    S = 600
    lens = np.random.default_rng(13).integers(0, 41, size=S)
    w = DecodeWorkload("many", S, 8, 8, 64, 0, 40, 16, 2000)
    _announce("decode 600 short sequences")
    a = decode_inputs(w, seed=13, seq_lens=lens)
    o, lse, _ = _run(a, 8)
    ro, rl = _oracle(a)
    empty = lens == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_decode_zero_page_table():
    """max_pages_per_seq == 0: every length clamps to 0, so O = 0 and LSE = -inf."""
    q = torch.randn((3, 4, 128), device="cuda:0").to(torch.bfloat16)
    kc = torch.zeros((2, 16, 1, 128), dtype=torch.bfloat16, device="cuda:0")
    bt = torch.zeros((3, 0), dtype=torch.int32, device="cuda:0")
    lens = torch.full((3,), 5, dtype=torch.int32, device="cuda:0")
    lse = torch.empty((3, 4), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_attn_decode(q, kc, kc, bt, lens, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_decode_repeated_calls_reuse_workspace():
    """A second call with other lengths on the same workspace gives the oracle's result (no stale partials)."""
    w = DecodeWorkload("reuse", 5, 16, 4, 128, 1, 900, 16, 400)
    ws_bytes = paa.paged_attn_decode_workspace_size(5, 16, 128, 16, w.max_pages_per_seq)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda:0")  # NaN-patterned garbage
    for seed, lens in ((21, [900, 3, 450, 0, 17]), (22, [16, 700, 1, 899, 300])):
        a = decode_inputs(w, seed=seed, seq_lens=lens)
        lse = torch.empty((5, 16), dtype=torch.float32, device="cuda:0")
        o, _ = paa.paged_attn_decode(dev_bf16(a["q"]), dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"]),
                                     dev_i32(a["block_table"]), dev_i32(a["seq_lens"]), a["scale"], workspace=ws,
                                     lse=lse)
        torch.cuda.synchronize()
        ro, rl = _oracle(a)
        assert_close_bf16(host_f64(o), ro)
        assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)


def test_decode_graph_replays_match_eager_and_oracle():
    """A captured decode step replayed four times, with new queries and lengths written in place by eager
    work between replays: every replay equals an eager call bitwise and the oracle within tolerance."""
    w = DecodeWorkload("graph", 6, 32, 8, 128, 100, 2000, 16, 1000)
    a = decode_inputs(w, seed=41)
    q, kc, vc = dev_bf16(a["q"]), dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"])
    bt, lens = dev_i32(a["block_table"]), dev_i32(a["seq_lens"])
    lse = torch.empty((6, 32), dtype=torch.float32, device="cuda:0")
    g = paa.PagedDecodeGraph([dict(q=q, k_cache=kc, v_cache=vc, block_table=bt, seq_lens=lens, scale=a["scale"],
                                   lse=lse)])
    rng = np.random.default_rng(42)
    try:
        for it in range(4):
            new_q = rng.standard_normal(a["q"].shape).astype(np.float32)
            from workloads import f32_to_bf16_bits
            q_bits = f32_to_bf16_bits(new_q)
            new_lens = np.array([rng.integers(0, L + 1) for L in a["seq_lens"]], dtype=np.int32)  # within the pages
            q.copy_(dev_bf16(q_bits))
            lens.copy_(dev_i32(new_lens))
            torch.cuda.synchronize()
            (o_g, l_g), = g.replay()
            torch.cuda.synchronize()
            o_g, l_g = o_g.clone(), l_g.clone()
            l_e = torch.empty_like(lse)
            o_e, _ = paa.paged_attn_decode(q, kc, vc, bt, lens, a["scale"], lse=l_e)
            torch.cuda.synchronize()
            assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"replay {it}"
            assert torch.equal(l_g, l_e), f"replay {it}"
            ro, rl = oracle.paged_decode(q_bits, a["k_cache"], a["v_cache"], a["block_table"], new_lens, a["scale"])
            assert_close_bf16(host_f64(o_g), ro)
            assert_close_lse(l_g.cpu().numpy().astype(np.float64), rl)
    finally:
        g.close()


def test_decode_graph_full_workload_matches_eager():
    """The 64-sequence workload captured once: replay equals the eager call bitwise."""
    w = WORKLOADS["paged_decode_s64h32kv8d128"]
    a = decode_inputs(w, seed=0)
    q, kc, vc = dev_bf16(a["q"]), dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"])
    bt, lens = dev_i32(a["block_table"]), dev_i32(a["seq_lens"])
    g = paa.PagedDecodeGraph([dict(q=q, k_cache=kc, v_cache=vc, block_table=bt, seq_lens=lens, scale=a["scale"])])
    try:
        o_g = g.replay()[0][0].clone()
        o_g2 = g.replay()[0][0]
        torch.cuda.synchronize()
        o_e, _ = paa.paged_attn_decode(q, kc, vc, bt, lens, a["scale"])
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16))
        assert torch.equal(o_g2.view(torch.int16), o_e.view(torch.int16))
    finally:
        g.close()


def test_decode_graph_mixes_fp8_and_bf16_caches():
    """Layers with E4M3 caches and layers with bf16 caches in one graph: every replay equals the eager calls
    bit for bit."""
    from workloads import decode_inputs_fp8
    lens = [5, 300, 1, 777]
    w = DecodeWorkload("mixed", len(lens), 32, 8, 128, 1, 800, 16, 300)
    layers, eager = [], []
    for i in range(4):
        fp8 = i % 2 == 1
        a = (decode_inputs_fp8 if fp8 else decode_inputs)(w, seed=70 + i, seq_lens=lens)
        kc, vc = ((torch.from_numpy(a["k_cache"]).to("cuda:0"), torch.from_numpy(a["v_cache"]).to("cuda:0")) if fp8
                  else (dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"])))
        c = dict(q=dev_bf16(a["q"]), k_cache=kc, v_cache=vc, block_table=dev_i32(a["block_table"]),
                 seq_lens=dev_i32(a["seq_lens"]), scale=a["scale"],
                 lse=torch.empty((len(lens), 32), dtype=torch.float32, device="cuda:0"))
        if fp8:
            c.update(k_scale=a["k_scale"], v_scale=a["v_scale"])
            o, _ = paa.paged_attn_decode_fp8(c["q"], kc, vc, c["block_table"], c["seq_lens"], a["k_scale"],
                                             a["v_scale"], a["scale"], lse=c["lse"])
        else:
            o, _ = paa.paged_attn_decode(c["q"], kc, vc, c["block_table"], c["seq_lens"], a["scale"], lse=c["lse"])
        torch.cuda.synchronize()
        eager.append((o.clone(), c["lse"].clone()))
        layers.append(c)
    _announce("decode graph mixing FP8 and bf16 caches")
    g = paa.PagedDecodeGraph(layers)
    try:
        for rep in range(2):
            for (o, lse) in g.outputs:
                o.zero_()
                lse.zero_()
            g.replay()
            torch.cuda.synchronize()
            for (o, lse), (eo, el) in zip(g.outputs, eager):
                assert torch.equal(o.view(torch.int16), eo.view(torch.int16))
                assert torch.equal(lse.view(torch.int32), el.view(torch.int32))
    finally:
        g.close()


def test_decode_graph_layers_in_one_submission():
    """Several decode calls (the layers of one decode step, with their own caches, head dims and group sizes,
    sharing one workspace as consecutive calls on one stream may) captured into one graph: every call's
    output equals its eager call bitwise and the oracle within tolerance, over two replays."""
    shapes = [(128, 32, 8), (64, 8, 8), (128, 16, 1), (128, 32, 8), (64, 6, 2)]
    lens = [1, 17, 300, 0, 1000, 64]
    inputs = [decode_inputs(DecodeWorkload("layer", len(lens), H, Hkv, d, 1, 1024, 16, 400), seed=60 + i,
                            seq_lens=lens) for i, (d, H, Hkv) in enumerate(shapes)]
    ws_bytes = max(paa.paged_attn_decode_workspace_size(len(lens), H, d, 16, a["block_table"].shape[1])
                   for (d, H, _), a in zip(shapes, inputs))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    layers = [dict(q=dev_bf16(a["q"]), k_cache=dev_bf16(a["k_cache"]), v_cache=dev_bf16(a["v_cache"]),
                   block_table=dev_i32(a["block_table"]), seq_lens=dev_i32(a["seq_lens"]), scale=a["scale"],
                   workspace=ws, lse=torch.empty((len(lens), H), dtype=torch.float32, device="cuda:0"))
              for (d, H, _), a in zip(shapes, inputs)]
    _announce(f"decode graph of {len(layers)} calls")
    g = paa.PagedDecodeGraph(layers)
    try:
        for rep in range(2):
            g.replay()
            torch.cuda.synchronize()
            outs = [(o.clone(), l.clone()) for o, l in g.outputs]
            for i, (c, a) in enumerate(zip(layers, inputs)):
                l_e = torch.empty_like(c["lse"])
                o_e, _ = paa.paged_attn_decode(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"],
                                               c["scale"], lse=l_e)
                torch.cuda.synchronize()
                o_g, l_g = outs[i]
                assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"replay {rep} call {i}"
                assert torch.equal(l_g, l_e), f"replay {rep} call {i}"
                ro, rl = _oracle(a)
                assert_close_bf16(host_f64(o_g), ro)
                assert_close_lse(l_g.cpu().numpy().astype(np.float64), rl)
    finally:
        g.close()


@pytest.mark.timeout(300)
def test_decode_zero_query_closed_form_full_size():
    """q = 0 on the full 64-sequence workload: every head returns the mean of its KV head's V rows over
    the sequence and LSE = ln L (closed form, no oracle), every element."""
    w = WORKLOADS["paged_decode_s64h32kv8d128"]
    _announce(f"{w.name} q=0")
    a = decode_inputs(w, seed=3)
    a["q"] = np.zeros_like(a["q"])
    o, lse, _ = _run(a, w.H)
    ro, rl = decode_zero_query_expected(oracle.bf16_bits_to_f64, a["v_cache"], a["block_table"], a["seq_lens"], w.H)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_decode_gqa_equals_mha_with_repeated_kv():
    """Decode with 32 query heads over 8 KV heads against the same call with each KV head repeated for its
    4 query heads (32 KV heads in the pool). The number of equal page ranges is the smaller of the pages
    the block table spans and the launch's wave budget over the KV heads, so it depends on Hkv: where the
    table spans few pages both calls cut the same ranges and agree bit for bit; where it spans many, the
    two calls merge different ranges: each stays within the oracle's bars, and they agree within the bound of
    _partition_bound."""
    small = DecodeWorkload("gqa_mha_small", 4, 32, 8, 128, 100, 250, 16, 400)
    large = DecodeWorkload("gqa_mha_large", 16, 32, 8, 128, 100, 2000, 16, 4000)
    for w, seed, bitwise in ((small, 77, True), (large, 78, False)):
        _announce(f"decode GQA vs MHA repeated {w.name}")
        a = decode_inputs(w, seed=seed)
        if bitwise:
            assert a["block_table"].size <= 64  # both calls cut one range per page
        o_g, l_g, _ = _run(a, w.H)
        b = dict(a, k_cache=np.repeat(a["k_cache"], 4, axis=2), v_cache=np.repeat(a["v_cache"], 4, axis=2))
        o_m, l_m, _ = _run(b, w.H)
        if bitwise:
            assert np.array_equal(o_g, o_m) and np.array_equal(l_g, l_m)
        else:
            ro, rl = _oracle(a)
            for o, lse in ((o_g, l_g), (o_m, l_m)):
                assert_close_bf16(o, ro)
                assert_close_lse(lse, rl)
            bound = _partition_bound(a)
            assert np.all(np.abs(o_g - o_m) <= bound + 2.0 ** -6 * np.maximum(np.abs(o_g), np.abs(o_m)))
            assert np.max(np.abs(l_g - l_m)) <= 1e-5


def test_decode_poisoned_slots_change_no_bit():
    """NaN in every slot no token occupies (the tail of each last page, every unreferenced page) against
    zeros there: the same bits out, so no kernel reads or multiplies a slot past a sequence's end."""
    w = DecodeWorkload("poison", 32, 32, 8, 128, 1, 2000, 16, 5000)
    _announce("decode poisoned against zero-filled slots")
    o1, l1, _ = _run(decode_inputs(w, seed=5, poison=True), w.H)
    o0, l0, _ = _run(decode_inputs(w, seed=5, poison=False), w.H)
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, o0) and np.array_equal(l1, l0)
