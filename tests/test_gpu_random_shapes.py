"""GPU parity over seeded random shapes: every entry point against the oracle.

Shapes are drawn once, from a fixed seed, at collection: head groupings 1, 2, 3, 4, 8 over 1, 2
or 4 KV heads, both head dims, ragged lengths (zero included where an entry point allows it),
windows below and beyond the sequence, and contexts and chunks on and off page and tile edges.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_attention_attn_amd as paa
from gpu_util import assert_close_bf16, assert_close_lse, dev_bf16, dev_i32, host_f64
from workloads import (ChunkedPrefillWorkload, DecodeWorkload, PrefillWorkload, chunked_prefill_inputs,
                       decode_inputs, decode_inputs_fp8, prefill_inputs)

pytestmark = pytest.mark.gpu

N_CASES = 12  # per entry point


def _draw():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(N_CASES):
        for kind in ("attn_fwd", "window", "decode", "decode_fp8", "paged_prefill"):
            Hkv = int(rng.choice([1, 2, 4]))
            H = Hkv * int(rng.choice([1, 2, 3, 4, 8]))
            d = int(rng.choice([64, 128]))
            c = {"kind": kind, "H": H, "Hkv": Hkv, "d": d, "seed": int(rng.integers(0, 1 << 30))}
            if kind in ("attn_fwd", "window"):
                c["B"] = int(rng.integers(1, 3))
                c["N"] = int(rng.integers(1, 600))
                c["causal"] = bool(rng.integers(0, 2))
                c["window"] = int(rng.integers(1, c["N"] + 20))
                c["n_global"] = int(rng.integers(0, 100))
            elif kind.startswith("decode"):
                c["lens"] = [int(x) for x in rng.integers(0, 1500, size=int(rng.integers(1, 12)))]
            else:
                S = int(rng.integers(1, 6))
                c["ctx"] = [int(x) for x in rng.integers(0, 1500, size=S)]
                c["q"] = [int(x) for x in rng.integers(0, 300, size=S)]
                c["q"][0] = max(1, c["q"][0])
            cases.append(c)
    return cases


CASES = _draw()


def _id(c):
    return f"{c['kind']}-H{c['H']}-Hkv{c['Hkv']}-d{c['d']}-{c['seed']}"


def _check(o, lse, ro, rl):
    torch.cuda.synchronize()
    assert_close_bf16(host_f64(o), ro)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)


@pytest.mark.parametrize("c", CASES, ids=_id)
def test_random_shape_parity(c):
    print(f"[gpu] random shape {c}", file=sys.stderr, flush=True)
    H, Hkv, d, seed = c["H"], c["Hkv"], c["d"], c["seed"]
    kind = c["kind"]
    if kind in ("attn_fwd", "window"):
        B, N = c["B"], c["N"]
        causal = c["causal"] or kind == "window"
        a = prefill_inputs(PrefillWorkload("random", B, H, Hkv, N, d, causal), seed=seed)
        q, k, v = dev_bf16(a["q"]), dev_bf16(a["k"]), dev_bf16(a["v"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        if kind == "attn_fwd":
            o, _ = paa.attn_fwd(q, k, v, causal, a["scale"], lse=lse)
            ro, rl = oracle.attention(a["q"], a["k"], a["v"], causal, a["scale"])
        else:
            o, _ = paa.attn_fwd_window(q, k, v, c["window"], c["n_global"], a["scale"], lse=lse)
            ro, rl = oracle.attention_window(a["q"], a["k"], a["v"], c["window"], c["n_global"], a["scale"])
        _check(o, lse, ro, rl)
    elif kind.startswith("decode"):
        lens = c["lens"]
        w = DecodeWorkload("random", len(lens), H, Hkv, d, 1, 1500, 16, sum(-(-L // 16) for L in lens) + 10)
        lse = torch.empty((len(lens), H), dtype=torch.float32, device="cuda:0")
        if kind == "decode_fp8":
            a = decode_inputs_fp8(w, seed=seed, seq_lens=lens)
            kc, vc = torch.from_numpy(a["k_cache"]).to("cuda:0"), torch.from_numpy(a["v_cache"]).to("cuda:0")
            o, _ = paa.paged_attn_decode_fp8(dev_bf16(a["q"]), kc, vc, dev_i32(a["block_table"]),
                                             dev_i32(a["seq_lens"]), a["k_scale"], a["v_scale"], a["scale"], lse=lse)
            ro, rl = oracle.paged_decode_fp8(a["q"], a["k_cache"], a["v_cache"], a["k_scale"], a["v_scale"],
                                             a["block_table"], a["seq_lens"], a["scale"])
        else:
            a = decode_inputs(w, seed=seed, seq_lens=lens)
            o, _ = paa.paged_attn_decode(dev_bf16(a["q"]), dev_bf16(a["k_cache"]), dev_bf16(a["v_cache"]),
                                         dev_i32(a["block_table"]), dev_i32(a["seq_lens"]), a["scale"], lse=lse)
            ro, rl = oracle.paged_decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"],
                                         a["scale"])
        _check(o, lse, ro, rl)
    else:
        ctx, ql = c["ctx"], c["q"]
        pages = sum(-(-(x + y) // 16) for x, y in zip(ctx, ql)) + 10
        w = ChunkedPrefillWorkload("random", len(ctx), H, Hkv, d, 0, 0, 1, num_pages=pages)
        a = chunked_prefill_inputs(w, seed=seed, ctx_lens=ctx, q_lens=ql)
        t = {n: dev_bf16(a[n]) for n in ("q", "k_new", "v_new", "k_cache", "v_cache")}
        lse = torch.empty((a["q"].shape[0], H), dtype=torch.float32, device="cuda:0")
        o, _ = paa.paged_prefill(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], dev_i32(a["block_table"]),
                                 dev_i32(a["ctx_lens"]), dev_i32(a["q_start"]), scale=a["scale"], lse=lse)
        ro, rl, rkc, rvc = oracle.paged_prefill(a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"],
                                                a["block_table"], a["ctx_lens"], a["q_start"], a["scale"])
        _check(o, lse, ro, rl)
        kc = t["k_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(kc, rkc)
