"""Calls on two streams at once: the library keeps no per-call state (the decode's partials live in the
caller's workspace), so concurrent calls give the same bits as the same calls made one after another."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import paged_attention_attn_amd as paa
from gpu_util import dev_bf16, dev_i32
from workloads import DecodeWorkload, PrefillWorkload, decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def test_concurrent_streams_match_serial_calls():
    _announce("prefill and decode on two streams at once")
    pa = prefill_inputs(PrefillWorkload("streams", 2, 32, 8, 2048, 128, True), seed=91)
    q, k, v = dev_bf16(pa["q"]), dev_bf16(pa["k"]), dev_bf16(pa["v"])
    da = decode_inputs(DecodeWorkload("streams", 16, 32, 8, 128, 100, 3000, 16, 4000), seed=92)
    dq, kc, vc = dev_bf16(da["q"]), dev_bf16(da["k_cache"]), dev_bf16(da["v_cache"])
    bt, lens = dev_i32(da["block_table"]), dev_i32(da["seq_lens"])

    def prefill(out, lse):
        paa.attn_fwd(q, k, v, True, pa["scale"], out=out, lse=lse)

    def decode(out, lse):
        paa.paged_attn_decode(dq, kc, vc, bt, lens, da["scale"], out=out, lse=lse)

    def buffers():
        return (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda:0"),
                torch.empty_like(dq), torch.empty(dq.shape[:2], dtype=torch.float32, device="cuda:0"))

    ref = buffers()
    prefill(ref[0], ref[1])
    decode(ref[2], ref[3])
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    got = [buffers() for _ in range(3)]
    torch.cuda.synchronize()
    for g in got:  # three rounds, each call of a round overlapping the other stream's
        with torch.cuda.stream(s1):
            prefill(g[0], g[1])
        with torch.cuda.stream(s2):
            decode(g[2], g[3])
            decode(g[2], g[3])  # twice on one stream: the workspace is reused in order
    torch.cuda.synchronize()
    as_bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()  # noqa: E731
    for g in got:
        for x, y in zip(g, ref):
            assert np.array_equal(as_bits(x), as_bits(y))
