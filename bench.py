#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one causal bf16 prefill (attn_fwd) of the causal_b4h16n1024d64
workload (B=4, H=16, N=1024, d=64) followed by one paged decode
(paged_attn_decode) of the paged_decode_s64h32kv8d128 workload (64 sequences,
H=32, Hkv=8, d=128, lengths uniform in [512, 8192], 16-token pages in a
40000-page pool), both on the current stream, inputs resident in HBM.

Prints ONE JSON line.  ``value`` is the prefill throughput in TFLOP/s on
algorithmic flops (4*d*B*H*visible pairs); the decode object reports GB/s on
algorithmic bytes (K/V of valid tokens + Q + O + LSE + table entries read).
Each kernel call is bracketed by HIP events on the stream it runs on; the
dominant call of the step (by time) gives the top-level ``roofline``.
``cpu_baseline`` times the float64 oracle on the host cores on a bounded
sample (the oracle is imported only for that leg).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attention TFLOP/s + paged decode KV GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")
KERNEL_SOURCES = ["prefill_bf16.hip", "paged_decode.hip", "device_common.hpp"]


def prefill_flops(w) -> float:
    return 4.0 * w.d * w.B * w.H * w.visible_pairs()


def prefill_bytes(w) -> float:
    el = 2
    return el * (w.B * w.H * w.N * w.d * 2 + w.B * w.Hkv * w.N * w.d * 2) + 4 * w.B * w.H * w.N


def decode_bytes(w, lens) -> float:
    lens = np.asarray(lens, dtype=np.int64)
    kv = float(lens.sum()) * w.Hkv * w.d * 2 * 2
    qo = 2.0 * len(lens) * w.H * w.d * 2
    return kv + qo + 4.0 * len(lens) * w.H + 4.0 * float((-(-lens // w.page_size)).sum()) + 4.0 * len(lens)


def source_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_attention_attn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, if taken on the current sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    entries = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                e = json.loads(line)
                entries[e["kernel"]] = e
    e = entries.get(kernel)
    if e is None or e.get("sources") != source_digest(KERNEL_SOURCES):
        return None
    return e["hbm_bytes_per_launch"]


def roofline(kind, achieved, peak, unit, traffic):
    return {"bound": kind, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def to_dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def to_dev_i32(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")


def timed(torch, fn, iters, warmup):
    """Median and mean of event-timed calls of fn on the current stream (ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return statistics.median(ts), statistics.fmean(ts)


def cpu_baseline(pw, pa, dw, da, budget_s=30.0):
    """The float64 oracle on host cores: the prefill workload's leading heads and 8 decode sequences."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = sum(p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas") or 1
    # prefill: whole (b, h) slices, as many as fit about half the budget (at least one)
    heads = pw.B * pw.H
    t0 = time.perf_counter()
    oracle.attention(pa["q"][:1, :1], pa["k"][:1, :1], pa["v"][:1, :1], pw.causal, pa["scale"])
    per_head = time.perf_counter() - t0
    n = int(max(1, min(heads, (budget_s / 2) / max(per_head, 1e-6))))
    bsel, hsel = n // pw.H, n % pw.H
    t0 = time.perf_counter()
    if bsel:
        oracle.attention(pa["q"][:bsel], pa["k"][:bsel], pa["v"][:bsel], pw.causal, pa["scale"])
    if hsel:
        g = (hsel - 1) // (pw.H // pw.Hkv) + 1
        oracle.attention(pa["q"][bsel:bsel + 1, :hsel], pa["k"][bsel:bsel + 1, :g], pa["v"][bsel:bsel + 1, :g],
                         pw.causal, pa["scale"])
    t_pre = time.perf_counter() - t0
    flops = 4.0 * pw.d * n * pw.visible_pairs()
    # decode: 8 sequences of the decode workload
    seqs = list(range(8))
    t0 = time.perf_counter()
    oracle.paged_decode(da["q"], da["k_cache"], da["v_cache"], da["block_table"], da["seq_lens"], da["scale"],
                        seqs=seqs)
    t_dec = time.perf_counter() - t0
    lens = da["seq_lens"][seqs]
    return {"value": round(flops / t_pre / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{pw.name}: {n} of {heads} (batch, head) slices, {t_pre:.1f} s",
            "decode": {"value": round(decode_bytes(dw, lens) / t_dec / 1e9, 4), "unit": "GB/s",
                       "sample": f"{dw.name}: sequences 0-7 ({int(lens.sum())} tokens), {t_dec:.1f} s"},
            "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prefill-workload", default="causal_b4h16n1024d64")
    ap.add_argument("--decode-workload", default="paged_decode_s64h32kv8d128")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-more", action="store_true", help="skip the larger prefill workloads")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "the kernels run on one MI355X and have no multi-GPU path", file=sys.stderr)
        return 2

    import torch

    import paged_attention_attn_amd as paa
    from workloads import WORKLOADS, decode_inputs, prefill_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if not os.path.exists(paa.LIB_PATH):
        from paged_attention_attn_amd import build
        build.build()

    pw = WORKLOADS[args.prefill_workload]
    dw = WORKLOADS[args.decode_workload]
    pa = prefill_inputs(pw, seed=args.seed)
    da = decode_inputs(dw, seed=args.seed)
    print(f"[bench] inputs ready: {pw.name}, {dw.name}", file=sys.stderr, flush=True)

    q, k, v = to_dev_bf16(torch, pa["q"]), to_dev_bf16(torch, pa["k"]), to_dev_bf16(torch, pa["v"])
    o = torch.empty_like(q)
    lse = torch.empty((pw.B, pw.H, pw.N), dtype=torch.float32, device="cuda:0")
    dq = to_dev_bf16(torch, da["q"])
    kc, vc = to_dev_bf16(torch, da["k_cache"]), to_dev_bf16(torch, da["v_cache"])
    bt, lens = to_dev_i32(torch, da["block_table"]), to_dev_i32(torch, da["seq_lens"])
    ws = torch.empty(paa.paged_attn_decode_workspace_size(dw.num_seqs, dw.H, dw.d, dw.page_size,
                                                          dw.max_pages_per_seq), dtype=torch.uint8, device="cuda:0")
    do = torch.empty_like(dq)
    dlse = torch.empty((dw.num_seqs, dw.H), dtype=torch.float32, device="cuda:0")

    def prefill():
        paa.attn_fwd(q, k, v, pw.causal, pa["scale"], out=o, lse=lse)

    def decode():
        paa.paged_attn_decode(dq, kc, vc, bt, lens, da["scale"], workspace=ws, out=do, lse=dlse)

    # ---- timed steps: W untimed, then exactly K, synchronised on both sides ----
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_beg.record()
    for i in range(K):
        ev[i][0].record()
        prefill()
        ev[i][1].record()
        decode()
        ev[i][2].record()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_beg.elapsed_time(t_end) / K
    pre_ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = statistics.fmean(e[1].elapsed_time(e[2]) for e in ev)
    print(f"[bench] {K} steps: {ms_step:.4f} ms/step (prefill {pre_ms:.4f} ms, decode {dec_ms:.4f} ms)",
          file=sys.stderr, flush=True)

    pf = prefill_flops(pw)
    db = decode_bytes(dw, da["seq_lens"])
    pre_tf = pf / (pre_ms * 1e-3) / 1e12
    dec_gbs = db / (dec_ms * 1e-3) / 1e9
    pre_roof = roofline("mfma", pre_tf, PEAK_BF16_TFLOPS, "TFLOP/s", read_traffic("prefill_bf16_kernel"))
    dec_roof = roofline("hbm", dec_gbs, PEAK_HBM_GBS, "GB/s", read_traffic("decode_partial_kernel"))

    # decode with the 256 MB last-level cache evicted before every call (512 MB write in between)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")
    cold = []
    for i in range(10 + 2):
        scratch.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        decode()
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            cold.append(a.elapsed_time(b))
    del scratch
    cold_ms = statistics.median(cold)

    more = []
    if not args.no_more:
        for name in ("causal_gqa_b2h32kv8n4096d128", "causal_gqa_long_b1h32kv8n16384d128"):
            w = WORKLOADS[name]
            a_ = prefill_inputs(w, seed=args.seed)
            q2, k2, v2 = to_dev_bf16(torch, a_["q"]), to_dev_bf16(torch, a_["k"]), to_dev_bf16(torch, a_["v"])
            o2 = torch.empty_like(q2)
            l2 = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
            med, mean = timed(torch, lambda: paa.attn_fwd(q2, k2, v2, True, a_["scale"], out=o2, lse=l2), 20, 3)
            tf = prefill_flops(w) / (mean * 1e-3) / 1e12
            more.append({"workload": name, "ms": round(mean, 4), "ms_median": round(med, 4),
                         "value": round(tf, 2), "unit": "TFLOP/s",
                         "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", None)})
            del q2, k2, v2, o2, l2
            print(f"[bench] {name}: {mean:.4f} ms, {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(pw, pa, dw, da)
        print(f"[bench] cpu baseline: {base['sample']}; {base['decode']['sample']}", file=sys.stderr, flush=True)

    dominant = dec_roof if dec_ms >= pre_ms else pre_roof
    dominant = dict(dominant, kernel="paged decode (decode_partial_kernel + decode_reduce_kernel)"
                    if dec_ms >= pre_ms else "prefill_bf16_kernel")
    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC,
        "value": round(pre_tf, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{pw.name} + {dw.name}",
                   "prefill": {"B": pw.B, "H": pw.H, "Hkv": pw.Hkv, "N": pw.N, "d": pw.d, "causal": pw.causal},
                   "decode": {"num_seqs": dw.num_seqs, "H": dw.H, "Hkv": dw.Hkv, "d": dw.d,
                              "L": [dw.L_lo, dw.L_hi], "page_size": dw.page_size, "num_pages": dw.num_pages,
                              "tokens": int(da["seq_lens"].sum())},
                   "seed": args.seed},
        "roofline": dominant,
        "prefill": {"workload": pw.name, "ms": round(pre_ms, 5), "value": round(pre_tf, 3), "unit": "TFLOP/s",
                    "algorithmic_gflop": round(pf / 1e9, 4), "algorithmic_mb": round(prefill_bytes(pw) / 1e6, 3),
                    "roofline": pre_roof},
        "decode": {"workload": dw.name, "ms": round(dec_ms, 5), "value": round(dec_gbs, 2), "unit": "GB/s",
                   "algorithmic_gb": round(db / 1e9, 5), "roofline": dec_roof,
                   "cold_ms": round(cold_ms, 5), "cold_value": round(db / (cold_ms * 1e-3) / 1e9, 2)},
        "prefill_more": more,
        "cpu_baseline": base,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
