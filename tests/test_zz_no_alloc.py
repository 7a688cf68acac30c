"""GPU test of paged_attn_decode_no_alloc (through the C ABI): the same outputs as paged_attn_decode with a
caller workspace, bit for bit, and within the oracle's bars, on two calls in a row (the second smaller) that
share the library's fixed scratch."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_attention_attn_amd as paa
from gpu_util import assert_close_bf16, assert_close_lse, dev_bf16, dev_i32, host_f64
from workloads import DecodeWorkload, decode_inputs

pytestmark = pytest.mark.gpu


def _case(w, seed):
    a = decode_inputs(w, seed=seed)
    t = dict(q=dev_bf16(a["q"]), kc=dev_bf16(a["k_cache"]), vc=dev_bf16(a["v_cache"]),
             bt=dev_i32(a["block_table"]), lens=dev_i32(a["seq_lens"]))
    return a, t


def _both(a, t, w):
    """(no-alloc O, LSE), (workspace O, LSE) for the same inputs."""
    o1 = torch.empty_like(t["q"])
    l1 = torch.empty((w.num_seqs, w.H), dtype=torch.float32, device="cuda:0")
    paa.paged_attn_decode_no_alloc(t["q"], t["kc"], t["vc"], t["bt"], t["lens"], a["scale"], out=o1, lse=l1)
    o2, l2 = paa.paged_attn_decode(t["q"], t["kc"], t["vc"], t["bt"], t["lens"], a["scale"],
                                   lse=torch.empty_like(l1))
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def test_no_alloc_decode_matches_workspace_decode_twice():
    big = DecodeWorkload("no_alloc_big", 24, 32, 8, 128, 256, 3000, 16, 6000)
    small = DecodeWorkload("no_alloc_small", 5, 8, 2, 64, 1, 700, 16, 300)
    for w, seed in ((big, 11), (small, 12)):  # the second call is smaller and reuses the same scratch
        print(f"[gpu] paged_attn_decode_no_alloc {w.name}", file=sys.stderr, flush=True)
        a, t = _case(w, seed)
        (o1, l1), (o2, l2) = _both(a, t, w)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        ro, rl = oracle.paged_decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], a["scale"])
        assert_close_bf16(host_f64(o1), ro)
        assert_close_lse(l1.cpu().numpy().astype(np.float64), rl)
