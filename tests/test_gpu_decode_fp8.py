"""GPU parity of paged_attn_decode_fp8 (through the C ABI) against the float64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import paged_attention_attn_amd as paa
from gpu_util import assert_close_bf16, assert_close_lse, decode_zero_query_expected, dev_bf16, dev_i32, host_f64
from workloads import WORKLOADS, DecodeWorkload, decode_inputs_fp8

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _run(a, H):
    lse = torch.empty((a["q"].shape[0], H), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_attn_decode_fp8(dev_bf16(a["q"]), _dev_u8(a["k_cache"]), _dev_u8(a["v_cache"]),
                                     dev_i32(a["block_table"]), dev_i32(a["seq_lens"]), a["k_scale"], a["v_scale"],
                                     a["scale"], lse=lse)
    torch.cuda.synchronize()
    return host_f64(o), lse.cpu().numpy().astype(np.float64), o


def _oracle(a, seqs=None):
    return oracle.paged_decode_fp8(a["q"], a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"],
                                   a["block_table"], a["seq_lens"], a["scale"], seqs=seqs)


@pytest.mark.parametrize("d,H,Hkv", [(128, 32, 8), (64, 8, 8), (128, 16, 1), (64, 6, 2)])
def test_fp8_decode_small_ragged_lengths(d, H, Hkv):
    """Lengths 0, 1, page edges and ragged tails; every unused slot holds the E4M3 NaN code."""
    lens = [0, 1, 15, 16, 17, 100, 255, 300]
    w = DecodeWorkload("fp8small", len(lens), H, Hkv, d, 1, 300, 16, 200)
    _announce(f"fp8 decode d{d} H{H} Hkv{Hkv}")
    a = decode_inputs_fp8(w, seed=d + H + Hkv, seq_lens=lens)
    o, lse, _ = _run(a, H)
    ro, rl = _oracle(a)
    empty = np.asarray(lens) == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    assert_close_bf16(o[~empty], ro[~empty])
    assert_close_lse(lse[~empty], rl[~empty])


@pytest.mark.timeout(300)
def test_fp8_decode_full_size_whole():
    """64 sequences, H=32, Hkv=8, d=128, lengths in [512, 8192], 40000-page pool, E4M3 cache: every
    sequence's O and LSE against the oracle."""
    w = WORKLOADS["paged_decode_s64h32kv8d128"]
    _announce("fp8 " + w.name)
    a = decode_inputs_fp8(w, seed=0)
    o, lse, _ = _run(a, w.H)
    ro, rl = oracle_pool.paged_decode_fp8(a["q"], a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"],
                                          a["block_table"], a["seq_lens"], a["scale"])
    st = assert_close_bf16(o, ro)
    st.update(assert_close_lse(lse, rl))
    _announce(f"fp8 {w.name}: {st}")


def test_fp8_decode_matches_bf16_decode_of_the_same_values():
    """With unit scales the FP8 decode turns each code into the bf16 value the bf16 decode reads from a bf16
    cache holding the same numbers; only the order of the sum over d in the scores differs, so LSEs agree
    within fp32 rounding and outputs within the bound derived below."""
    w = DecodeWorkload("fp8eq", 5, 32, 8, 128, 1, 700, 16, 300)
    a = decode_inputs_fp8(w, seed=31)
    lse8 = torch.empty((5, 32), dtype=torch.float32, device="cuda:0")
    o8, _ = paa.paged_attn_decode_fp8(dev_bf16(a["q"]), _dev_u8(a["k_cache"]), _dev_u8(a["v_cache"]),
                                      dev_i32(a["block_table"]), dev_i32(a["seq_lens"]), 1.0, 1.0, a["scale"],
                                      lse=lse8)
    as_bf16 = lambda x: torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.bfloat16).to("cuda:0")
    lse16 = torch.empty((5, 32), dtype=torch.float32, device="cuda:0")
    o16, _ = paa.paged_attn_decode(dev_bf16(a["q"]), as_bf16(a["k_cache"]), as_bf16(a["v_cache"]),
                                   dev_i32(a["block_table"]), dev_i32(a["seq_lens"]), a["scale"], lse=lse16)
    torch.cuda.synchronize()
    x, y = host_f64(o8), host_f64(o16)
    # a score that differs in its last fp32 bit can move a probability's bf16 rounding by one step (2^-7 of
    # its value), so O may differ by 2^-7 of (the softmax-weighted mean of |v| + |O|) besides the two
    # outputs' own rounding; the weighted mean comes from the oracle over |V| (sign bits cleared)
    a_abs = oracle.paged_decode_fp8(a["q"], a["k_cache"], a["v_cache"] & np.uint8(0x7F), 1.0, 1.0,
                                    a["block_table"], a["seq_lens"], a["scale"])[0]
    assert np.all(np.abs(x - y) <= 2.0 ** -7 * a_abs + 2.0 ** -6 * np.maximum(np.abs(x), np.abs(y)))
    # scores here reach the hundreds (E4M3 values up to 448 with unit scales): a few fp32 ulps of the LSE
    ulp = np.finfo(np.float32).eps * np.abs(lse16.cpu().numpy())
    assert np.all(np.abs(lse8.cpu().numpy() - lse16.cpu().numpy()) <= 4 * ulp)


def test_fp8_decode_argument_errors():
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device="cuda:0")
    kc = torch.zeros((4, 16, 1, 128), dtype=torch.uint8, device="cuda:0")
    bt = torch.zeros((2, 2), dtype=torch.int32, device="cuda:0")
    lens = torch.ones((2,), dtype=torch.int32, device="cuda:0")
    with pytest.raises(RuntimeError, match="scale"):
        paa.paged_attn_decode_fp8(q, kc, kc, bt, lens, 0.0, 1.0)
    with pytest.raises(TypeError):
        paa.paged_attn_decode_fp8(q, kc.to(torch.bfloat16), kc.to(torch.bfloat16), bt, lens, 1.0, 1.0)


def test_fp8_decode_zero_page_table():
    """max_pages_per_seq == 0: every length clamps to 0, so O = 0 and LSE = -inf."""
    q = torch.randn((3, 4, 128), device="cuda:0").to(torch.bfloat16)
    kc = torch.zeros((2, 16, 1, 128), dtype=torch.uint8, device="cuda:0")
    bt = torch.zeros((3, 0), dtype=torch.int32, device="cuda:0")
    lens = torch.full((3,), 5, dtype=torch.int32, device="cuda:0")
    lse = torch.empty((3, 4), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_attn_decode_fp8(q, kc, kc, bt, lens, 0.5, 0.5, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_fp8_decode_out_of_range_page_id_is_not_read():
    """A page id past num_pages is never dereferenced; its tokens count as absent (here the middle page of
    three), so the result is the decode over the other two pages."""
    w = DecodeWorkload("fp8oob", 1, 4, 1, 64, 48, 48, 16, 8)
    bt = np.array([[2, 5, 7]], dtype=np.int32)
    a = decode_inputs_fp8(w, seed=6, seq_lens=[48], block_table=bt)
    bad = dict(a)
    bad["block_table"] = np.array([[2, 1 << 30, 7]], dtype=np.int32)
    o, lse, _ = _run(bad, 4)
    # the same tokens with the middle page dropped: a two-page sequence over pages 2 and 7
    two = dict(a)
    two["block_table"] = np.array([[2, 7, -1]], dtype=np.int32)
    two["seq_lens"] = np.array([32], dtype=np.int32)
    ro, rl = _oracle(two)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


@pytest.mark.timeout(300)
def test_fp8_decode_zero_query_closed_form_full_size():
    """q = 0 on the full 64-sequence workload over the E4M3 cache: every head returns v_scale times the
    mean of its KV head's decoded V rows and LSE = ln L (closed form, no oracle), every element."""
    w = WORKLOADS["paged_decode_s64h32kv8d128"]
    _announce(f"{w.name} fp8 cache q=0")
    a = decode_inputs_fp8(w, seed=3)
    a["q"] = np.zeros_like(a["q"])
    o, lse, _ = _run(a, w.H)
    ro, rl = decode_zero_query_expected(lambda raw: oracle.e4m3_bits_to_f64(raw) * a["v_scale"], a["v_cache"],
                                        a["block_table"], a["seq_lens"], w.H)
    assert_close_bf16(o, ro)
    assert_close_lse(lse, rl)


def test_fp8_decode_gqa_equals_mha_with_repeated_kv():
    """E4M3-cache decode with 32 query heads over 8 KV heads against the same call with each KV head
    repeated for its 4 query heads. The block table spans 64 pages or fewer, so both calls cut one
    range per page and each query head's O and LSE agree bit for bit."""
    w = DecodeWorkload("fp8_gqa_mha", 4, 32, 8, 128, 100, 250, 16, 400)
    _announce("fp8 decode GQA vs MHA repeated")
    a = decode_inputs_fp8(w, seed=81)
    assert a["block_table"].size <= 64
    o_g, l_g, _ = _run(a, w.H)
    b = dict(a, k_cache=np.repeat(a["k_cache"], 4, axis=2), v_cache=np.repeat(a["v_cache"], 4, axis=2))
    o_m, l_m, _ = _run(b, w.H)
    assert np.array_equal(o_g, o_m) and np.array_equal(l_g, l_m)
    ro, rl = _oracle(a)
    assert_close_bf16(o_g, ro)
    assert_close_lse(l_g, rl)


def test_fp8_decode_poisoned_slots_change_no_bit():
    """The E4M3 NaN code in every slot no token occupies against zero codes there: the same bits out."""
    w = DecodeWorkload("fp8poison", 32, 32, 8, 128, 1, 2000, 16, 5000)
    _announce("fp8 decode poisoned against zero-filled slots")
    o1, l1, _ = _run(decode_inputs_fp8(w, seed=6, poison=True), w.H)
    o0, l0, _ = _run(decode_inputs_fp8(w, seed=6, poison=False), w.H)
    assert np.all(np.isfinite(o1)) and np.array_equal(o1, o0) and np.array_equal(l1, l0)
