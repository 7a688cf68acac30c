"""GPU parity at the largest sizes the C ABI accepts: a (batch, KV head) stream one row short of 2 GiB."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_attention_attn_amd as paa
from gpu_util import assert_close_bf16, assert_close_lse, host_f64

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def _bf16_randn(shape, gen):
    x = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    for i in range(0, shape[2], 1 << 21):  # in slices, so the fp32 draw stays small
        x[:, :, i:i + (1 << 21)] = torch.randn((shape[0], shape[1], min(1 << 21, shape[2] - i), shape[3]),
                                               generator=gen, device="cuda:0").to(torch.bfloat16)
    return x


@pytest.mark.timeout(600)
def test_window_prefill_at_the_largest_accepted_stream():
    """Sliding-window causal attention with N = 8,388,607 tokens at d = 128, so that Q, K, V and O of the
    one head are each 2^31 - 256 bytes (the largest stream the ABI accepts; one more row is refused) and
    the last key tile is ragged: sampled rows (the ends, tile and window edges, the middle, seeded
    random picks) against the oracle evaluated on exactly the keys each row sees."""
    N, d, window, n_global = (1 << 31) // 256 - 1, 128, 1024, 16
    assert N * d * 2 < 1 << 31 <= (N + 1) * d * 2
    _announce(f"attn_fwd_window max stream N{N} d{d} window {window} globals {n_global}")
    gen = torch.Generator(device="cuda:0").manual_seed(2024)
    q, k, v = (_bf16_randn((1, 1, N, d), gen) for _ in range(3))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    lse = torch.empty((1, 1, N), dtype=torch.float32, device="cuda:0")
    o, _ = paa.attn_fwd_window(q, k, v, window, n_global, scale, lse=lse)
    torch.cuda.synchronize()
    # the next row up is refused before any launch
    with pytest.raises(RuntimeError):
        big = torch.empty((1, 1, N + 1, d), dtype=torch.bfloat16, device="cuda:0")
        paa.attn_fwd_window(big, big, big, window, n_global, scale)
    rng = np.random.default_rng(7)
    rows = sorted({0, 1, 15, 16, 63, 64, window - 1, window, window + 16, N // 2, N - 65, N - 64, N - 63, N - 2,
                   N - 1} | {int(x) for x in rng.integers(0, N, 24)})
    got_o = host_f64(o[0, 0, rows])
    got_l = lse[0, 0, rows].cpu().numpy().astype(np.float64)
    want_o, want_l = [], []
    for i in rows:
        vis = sorted(set(range(min(n_global, i + 1))) | set(range(max(0, i - window + 1), i + 1)))
        idx = torch.tensor(vis, device="cuda:0")
        qi = host_f64(q[0, 0, i:i + 1])[None, None]          # [1, 1, 1, d]
        ki = host_f64(k[0, 0].index_select(0, idx))[None, None]
        vi = host_f64(v[0, 0].index_select(0, idx))[None, None]
        ro, rl = oracle.attention_rows(qi, ki, vi, False, scale, [(0, 0, 0)])  # softmax over exactly those keys
        want_o.append(ro[0])
        want_l.append(rl[0])
    assert_close_bf16(got_o, np.array(want_o))
    assert_close_lse(got_l, np.array(want_l))


def _big_pools(compact, n_big, seed):
    """Both caches of `compact` ([P, 16, Hkv, d] uint16 bf16 bits) moved into pools of n_big pages on the
    device, compact page p at a distinct page id drawn from the top quarter of the pool (so that page
    offsets pass 4 GiB); every other slot holds bfloat16 NaN.  Returns the pools and the id map."""
    P = compact.shape[0]
    ids = np.random.default_rng(seed).choice(np.arange(n_big * 3 // 4, n_big), size=P, replace=False)
    big = torch.full((n_big,) + compact.shape[1:], 0x7FC0, dtype=torch.int16, device="cuda:0")
    big[torch.from_numpy(ids).to("cuda:0")] = torch.from_numpy(compact.view(np.int16)).to("cuda:0")
    return big.view(torch.bfloat16), ids


def _remap(bt, ids):
    out = bt.copy()
    out[bt >= 0] = ids[bt[bt >= 0]]
    return out


@pytest.mark.timeout(600)
def test_decode_and_chunked_prefill_over_a_pool_past_4_gib():
    """A 200,000-page pool (6.5 GB per cache) with every referenced page in its top quarter, so that page
    offsets are past 4 GiB: decode and chunked prefill (with its append) against the oracle on the same
    pages renumbered into a small pool; the appended rows land at the remapped pages, nothing else moves."""
    from workloads import ChunkedPrefillWorkload, DecodeWorkload, chunked_prefill_inputs, decode_inputs
    from gpu_util import dev_bf16, dev_i32
    n_big = 200_000
    # decode
    w = DecodeWorkload("bigpool", 4, 32, 8, 128, 100, 3000, 16, 800)
    a = decode_inputs(w, seed=31)
    _announce(f"paged decode over a {n_big}-page pool")
    kc, ids = _big_pools(a["k_cache"], n_big, 1)
    vc, _ = _big_pools(a["v_cache"], n_big, 1)
    bt = _remap(a["block_table"], ids)
    lse = torch.empty((w.num_seqs, w.H), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_attn_decode(dev_bf16(a["q"]), kc, vc, dev_i32(bt), dev_i32(a["seq_lens"]), a["scale"],
                                 num_pages=n_big, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], a["scale"])
    assert_close_bf16(host_f64(o), ro)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)
    del kc, vc
    torch.cuda.empty_cache()
    # chunked prefill, ping-pong sized grid (32 sequences x 8 KV heads x 4 query tiles)
    cw = ChunkedPrefillWorkload("bigpool", 32, 32, 8, 128, 0, 1500, 256, num_pages=32 * 110)
    c = chunked_prefill_inputs(cw, seed=32)
    _announce(f"paged prefill over a {n_big}-page pool")
    kc, ids = _big_pools(c["k_cache"], n_big, 2)
    vc, _ = _big_pools(c["v_cache"], n_big, 2)
    bt = _remap(c["block_table"], ids)
    T = c["q"].shape[0]
    lse = torch.empty((T, cw.H), dtype=torch.float32, device="cuda:0")
    o, _ = paa.paged_prefill(dev_bf16(c["q"]), dev_bf16(c["k_new"]), dev_bf16(c["v_new"]), kc, vc, dev_i32(bt),
                             dev_i32(c["ctx_lens"]), dev_i32(c["q_start"]), max_q_len=c["max_q_len"],
                             scale=c["scale"], lse=lse)
    torch.cuda.synchronize()
    ro, rl, rkc, rvc = oracle.paged_prefill(c["q"], c["k_new"], c["v_new"], c["k_cache"], c["v_cache"],
                                            c["block_table"], c["ctx_lens"], c["q_start"], c["scale"])
    assert_close_bf16(host_f64(o), ro)
    assert_close_lse(lse.cpu().numpy().astype(np.float64), rl)
    idx = torch.from_numpy(ids).to("cuda:0")
    got_k = kc.view(torch.int16)[idx].cpu().numpy().view(np.uint16)
    got_v = vc.view(torch.int16)[idx].cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, rkc) and np.array_equal(got_v, rvc)
    # no other page changed: a sample of the rest still holds NaN
    rest = np.setdiff1d(np.arange(n_big), ids)[:: 997]
    other = kc.view(torch.int16)[torch.from_numpy(rest).to("cuda:0")].cpu().numpy()
    assert np.all(other == 0x7FC0)
