#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one causal bf16 GQA prefill (attn_fwd) of the long workload
causal_gqa_long_b1h32kv8n16384d128 (B=1, H=32, Hkv=8, N=16384, d=128, Q x4, 1%
of K rows x8) followed by one paged decode (paged_attn_decode) of
paged_decode_s64h32kv8d128 (64 sequences, H=32, Hkv=8, d=128, lengths uniform
in [512, 8192], 16-token pages in a 40000-page pool), both on the current
stream, inputs resident in HBM.

Prints ONE JSON line.  ``value`` is the prefill throughput in TFLOP/s on
algorithmic flops (4*d*B*H*visible pairs); the prefill kernel takes most of the
step, so it gives the top-level ``roofline`` (against the bf16 MFMA peak).  The
decode object reports GB/s on algorithmic bytes (K/V of valid tokens + Q + O +
LSE + block-table entries and lengths read); its headline ``value`` is the
cold-cache rate (the 256 MB last-level cache evicted before each call), the
warm rate is reported beside it.  Each call is bracketed by HIP events on the
stream it is launched on.  The other workloads (the short causal d=64 prefill,
the 4096-token GQA prefill, the windowed, chunked and FP8 paths, the decode
graph) are secondary entries.  ``cpu_baseline`` times the float64 oracle on the
host cores on a bounded sample of each workload (the oracle is imported only
there).

Other modes (used to produce the summaries kept under profiles/):
  --pmc-pass                 a few launches of every kernel plus a plain copy
                             of known size, for a rocprofv3 --pmc run
  --summarize-trace DIR      markdown summary of a rocprofv3 --kernel-trace run
  --summarize-mfma D P       MFMA utilisation per workload from a counter run (D)
                             MFMA_COUNTERS
  --summarize-counters F W   HBM bytes per launch from a FETCH_SIZE run (F)
                             and a WRITE_SIZE run (W), calibrated by the copy
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attention TFLOP/s + paged decode KV GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0  # dense fp8 MFMA
PEAK_CLOCK_GHZ = 2.4  # the engine clock both MFMA peaks are quoted at
CLOCK_SAMPLE_S = 2.0  # seconds of back-to-back prefill calls while the shader clocks are sampled
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_counters.txt")
CSRC = os.path.join(ROOT, "paged_attention_attn_amd", "csrc")
PHASE_GAP_S = 0.05         # idle time left between phases so a trace can be split by them
COPY_BYTES = 1 << 30       # calibration copy: 1 GiB read + 1 GiB written
COPY_KERNEL_TAG = "neg_kernel"  # torch's elementwise negate, used as the plain copy kernel
PMC_CALLS = 3              # calls of each workload in a counter pass

PREFILL_DEFAULT = "causal_gqa_long_b1h32kv8n16384d128"
SMALL_DECODE = "paged_decode_s4h32kv8d128_short"  # launch-bound: eager calls against graph replays
FP8_MORE = ("fp8_causal_gqa_b2h32kv8n4096d128", "fp8_causal_gqa_long_b1h32kv8n16384d128")
FP8_DECODE_SUFFIX = "_fp8kv"  # the decode workload over an E4M3 cache
CHUNKED = "chunked_prefill_s16h32kv8d128_ctx0to4096_q512"  # chunked prefill over a paged cache, with append
GRAPH_LAYERS = 32  # decode calls per step in the graph comparison, each with its own KV cache
PREWARM_S = 0.25  # untimed calls of the step before its W warm-up steps (see prewarm)
DECODE_DEFAULT = "paged_decode_s64h32kv8d128"
PREFILL_MORE = ("causal_b4h16n1024d64", "causal_gqa_b2h32kv8n4096d128", "window_gqa_b1h32kv8n16384d128_w4096_g64")
TINY_F32 = "tiny_f32_b1h2n128d64"


# ----------------------------------------------------------------- algorithmic counts

def prefill_flops(w) -> float:
    """4*d flops (two matmuls) per visible query-key pair."""
    return 4.0 * w.d * w.B * w.H * w.visible_pairs()


def prefill_bytes(w) -> float:
    """Q, K, V read once, O and LSE written once (K/V once per KV head)."""
    el = 2 if w.dtype == "bf16" else 4
    return el * (w.B * w.H * w.N * w.d * 2 + w.B * w.Hkv * w.N * w.d * 2) + 4 * w.B * w.H * w.N


def decode_bytes(w, lens, kv_bytes: int = 2) -> float:
    """K and V of the valid tokens (kv_bytes per element: 2 for bf16, 1 for E4M3), Q, O, LSE, the block-table
    entries used and the lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    kv = float(lens.sum()) * w.Hkv * w.d * kv_bytes * 2
    qo = 2.0 * len(lens) * w.H * w.d * 2
    return kv + qo + 4.0 * len(lens) * w.H + 4.0 * float((-(-lens // w.page_size)).sum()) + 4.0 * len(lens)


def chunked_flops(w, ctx_lens) -> float:
    """4 d H per visible (query, key) pair; chunk query i of a sequence with ctx cached tokens sees ctx + i + 1."""
    q = w.q_len
    pairs = sum(q * int(c) + q * (q + 1) // 2 for c in ctx_lens)
    return 4.0 * w.d * w.H * pairs


def chunked_bytes(w, ctx_lens) -> float:
    """Compulsory bytes: Q, O, the chunk's K/V read once, the context's K/V read once, the chunk's K/V
    written to the cache, LSE written."""
    T = w.num_seqs * w.q_len
    ctx = int(sum(int(c) for c in ctx_lens))
    return 2.0 * (2 * T * w.H * w.d + 2 * T * w.Hkv * w.d + 2 * ctx * w.Hkv * w.d + 2 * T * w.Hkv * w.d) + 4.0 * T * w.H


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks and empty lines (none of which changes a kernel)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest() -> str:
    """Digest of the code of every kernel source: counter figures are only valid for the code they were
    taken on (comment edits keep them)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per call of ``workload`` from the committed counter summary, if taken on these sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("{"):
                continue
            e = json.loads(line)
            if e.get("workload") == workload and e.get("sources") == source_digest():
                return e["hbm_bytes_per_call"]
    return None


def read_mfma_busy(workload: str):
    """(MfmaUtil %, MFMA flops executed per algorithmic flop) of the workload's attention kernel from the
    committed counter summary, if taken on these sources; (None, None) otherwise."""
    if not os.path.exists(MFMA_FILE):
        return None, None
    with open(MFMA_FILE) as f:
        for line in f:
            if line.startswith("{"):
                e = json.loads(line)
                if e.get("workload") == workload and e.get("sources") == source_digest() and \
                        e.get("mfma_tflop_per_call", 0) > 0:
                    alg = e.get("algorithmic_tflop")
                    return e["mfma_util_pct"], (e["mfma_tflop_per_call"] / alg if alg else None)
    return None, None


def roofline(kind, achieved, peak, unit, traffic, mfma=(None, None)):
    r = {"bound": kind, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if kind == "mfma":
        r["mfma_busy_pct"] = mfma[0]  # matrix-core busy share of active cycles (counters), or None
    return r


# ----------------------------------------------------------------- device helpers

def to_dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def to_dev_i32(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")


def prewarm(torch, fn, seconds=0.2):
    """Call fn for ``seconds`` of wall time before anything is timed: after idle gaps (input set-up on
    the host) the GPU clock takes tens of milliseconds of load to return to its steady value."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed(torch, fn, iters, warmup):
    """Median and mean (ms) of event-timed calls of fn on the current stream (after a pre-warm)."""
    prewarm(torch, fn, 0.1)
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


def gfx_clocks_from_amd_smi(data):
    """{gpu: [MHz of gfx_0, gfx_1, ...]} from the JSON of `amd-smi metric -c --json` (a dict holding
    "gpu_data", or the list itself), or None if it holds no shader clock."""
    gpus = data.get("gpu_data", []) if isinstance(data, dict) else data
    out = {}
    for g in gpus if isinstance(gpus, list) else []:
        clk = g.get("clock", {}) if isinstance(g, dict) else {}
        names = [k for k in clk if k.startswith("gfx_") and k[4:].isdigit()]
        vals = []
        for k in sorted(names, key=lambda k: int(k[4:])):
            inner = clk[k].get("clk") if isinstance(clk[k], dict) else None
            v = inner.get("value") if isinstance(inner, dict) else None
            if isinstance(v, (int, float)):
                vals.append(float(v))
        if vals:
            out[g.get("gpu")] = vals
    return out or None


def sample_gfx_clocks(torch, fn, seconds=CLOCK_SAMPLE_S):
    """Shader clocks while fn runs back to back: `amd-smi metric -c` read about every 0.1 s from a second
    thread, averaged per die (gfx_0, gfx_1, ...) over the samples after the first quarter second.  Of the
    GPUs amd-smi lists, the one with the highest clocks is taken (the busy one).  None where amd-smi is not
    installed or its output cannot be read."""
    import shutil
    import subprocess
    import threading
    exe = shutil.which("amd-smi")
    if exe is None:
        return None

    def read():
        try:
            r = subprocess.run([exe, "metric", "-c", "--json"], capture_output=True, text=True, timeout=30)
            return gfx_clocks_from_amd_smi(json.loads(r.stdout))
        except (OSError, subprocess.SubprocessError, ValueError):
            return None

    samples, stop = [], threading.Event()

    def loop():
        t0 = time.perf_counter()
        while not stop.is_set():
            got = read()
            if got is None:
                return
            samples.append((time.perf_counter() - t0, got))
            stop.wait(0.1)

    th = threading.Thread(target=loop, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=60)
    use = [got for t, got in samples if t >= 0.25]
    if not use:
        return None

    def per_die(g):
        rows = [got[g] for got in use if g in got]
        return [statistics.fmean(r[i] for r in rows) for i in range(min(len(r) for r in rows))]

    best = max({g for got in use for g in got}, key=lambda g: statistics.fmean(per_die(g)))
    dies = per_die(best)
    return {"mean_mhz": round(statistics.fmean(dies), 1), "per_die_mhz": [round(x, 1) for x in dies],
            "samples": len(use), "seconds": seconds, "gpu_index_in_amd_smi": best,
            "source": "amd-smi metric -c about every 0.1 s while the workload ran back to back"}


class Phases:
    """Named phases separated by idle gaps, so a kernel trace of this run can be split per workload."""

    def __init__(self, torch):
        self.torch = torch
        self.names = []

    def start(self, name):
        self.torch.cuda.synchronize()
        time.sleep(PHASE_GAP_S)
        self.names.append(name)
        print(f"[bench] phase {len(self.names) - 1}: {name}", file=sys.stderr, flush=True)


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------- workload setup

class PrefillCase:
    def __init__(self, torch, paa, w, seed):
        from workloads import prefill_inputs
        self.w = w
        self.a = prefill_inputs(w, seed=seed)
        self.q, self.k, self.v = (to_dev_bf16(torch, self.a[n]) for n in ("q", "k", "v"))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
        self.paa = paa

    def __call__(self):
        if self.w.window:
            self.paa.attn_fwd_window(self.q, self.k, self.v, self.w.window, self.w.n_global, self.a["scale"],
                                     out=self.o, lse=self.lse)
        else:
            self.paa.attn_fwd(self.q, self.k, self.v, self.w.causal, self.a["scale"], out=self.o, lse=self.lse)


class DecodeCase:
    def __init__(self, torch, paa, w, seed):
        from workloads import decode_inputs
        self.w = w
        self.a = a = decode_inputs(w, seed=seed)
        self.q = to_dev_bf16(torch, a["q"])
        self.kc, self.vc = to_dev_bf16(torch, a["k_cache"]), to_dev_bf16(torch, a["v_cache"])
        self.bt, self.lens = to_dev_i32(torch, a["block_table"]), to_dev_i32(torch, a["seq_lens"])
        self.ws = torch.empty(paa.paged_attn_decode_workspace_size(w.num_seqs, w.H, w.d, w.page_size,
                                                                   w.max_pages_per_seq),
                              dtype=torch.uint8, device="cuda:0")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.num_seqs, w.H), dtype=torch.float32, device="cuda:0")
        self.paa = paa

    def __call__(self):
        self.paa.paged_attn_decode(self.q, self.kc, self.vc, self.bt, self.lens, self.a["scale"],
                                   workspace=self.ws, out=self.o, lse=self.lse)


class Fp8DecodeCase:
    """The decode workload with its K/V cache held as E4M3 bytes and per-tensor scales."""

    def __init__(self, torch, paa, w, seed):
        from workloads import decode_inputs_fp8
        self.w = w
        self.name = w.name + FP8_DECODE_SUFFIX
        self.a = a = decode_inputs_fp8(w, seed=seed)
        self.q = to_dev_bf16(torch, a["q"])
        self.kc, self.vc = torch.from_numpy(a["k_cache"]).to("cuda:0"), torch.from_numpy(a["v_cache"]).to("cuda:0")
        self.bt, self.lens = to_dev_i32(torch, a["block_table"]), to_dev_i32(torch, a["seq_lens"])
        self.ws = torch.zeros(paa.paged_attn_decode_workspace_size(w.num_seqs, w.H, w.d, w.page_size,
                                                                   w.max_pages_per_seq),
                              dtype=torch.uint8, device="cuda:0")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.num_seqs, w.H), dtype=torch.float32, device="cuda:0")
        self.paa = paa

    def __call__(self):
        a = self.a
        self.paa.paged_attn_decode_fp8(self.q, self.kc, self.vc, self.bt, self.lens, a["k_scale"], a["v_scale"],
                                       a["scale"], workspace=self.ws, out=self.o, lse=self.lse)


class Fp8Case:
    def __init__(self, torch, paa, w, seed):
        from workloads import prefill_inputs
        self.w = w
        self.a = a = prefill_inputs(w, seed=seed)
        self.q, self.k, self.vt = (torch.from_numpy(a[n]).to("cuda:0") for n in ("q8", "k8", "vt8"))
        self.o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda:0")
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
        self.paa = paa

    def __call__(self):
        a = self.a
        self.paa.attn_fwd_fp8(self.q, self.k, self.vt, self.w.causal, a["scale"], a["q_scale"], a["k_scale"],
                              a["v_scale"], out=self.o, lse=self.lse)


class ChunkedCase:
    def __init__(self, torch, paa, w, seed):
        from workloads import chunked_prefill_inputs
        self.w = w
        self.a = a = chunked_prefill_inputs(w, seed=seed)
        self.q = to_dev_bf16(torch, a["q"])
        self.kn, self.vn = to_dev_bf16(torch, a["k_new"]), to_dev_bf16(torch, a["v_new"])
        self.kc, self.vc = to_dev_bf16(torch, a["k_cache"]), to_dev_bf16(torch, a["v_cache"])
        self.bt, self.ctx = to_dev_i32(torch, a["block_table"]), to_dev_i32(torch, a["ctx_lens"])
        self.qs = to_dev_i32(torch, a["q_start"])
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((self.q.shape[0], w.H), dtype=torch.float32, device="cuda:0")
        self.paa = paa

    def __call__(self):
        # the same chunk appended again each call: the cache holds the same values afterwards
        self.paa.paged_prefill(self.q, self.kn, self.vn, self.kc, self.vc, self.bt, self.ctx, self.qs,
                               max_q_len=self.a["max_q_len"], scale=self.a["scale"], out=self.o, lse=self.lse)


# ----------------------------------------------------------------- CPU baseline (oracle)

def _blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return sum(p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas") or 1


def cpu_baseline(seed, dc, min_seconds=10.0):
    """The float64 oracle, as it stands, on the host cores, on a bounded sample of every workload.

    Per workload the sample is: the whole tiny fp32 and d=64 causal prefills; one query head (with its
    KV head) of the 4096- and 16384-token GQA prefills, whose heads all cost the same; the whole paged
    decode.  Each sample is repeated until ``min_seconds`` have passed in total and the mean per pass is
    reported, scaled to the metric's unit on the sample's own algorithmic work.  ``value`` is the rate on
    the step's prefill workload (the long GQA prefill), ``decode`` the rate on the step's decode.
    """
    import oracle
    from workloads import WORKLOADS, PrefillWorkload, prefill_inputs

    def head_sample(name, n_heads):
        w = WORKLOADS[name]
        a = prefill_inputs(w, seed=seed)
        g = w.H // w.Hkv
        q = a["q"][:1, :n_heads]
        k, v = a["k"][:1, : -(-n_heads // g)], a["v"][:1, : -(-n_heads // g)]
        sw = PrefillWorkload(w.name + "_sample", 1, n_heads, k.shape[1], w.N, w.d, w.causal)
        return sw, (lambda: oracle.attention(q, k, v, w.causal, a["scale"])), w

    samples = []
    for name, heads in ((TINY_F32, None), ("causal_b4h16n1024d64", None), ("causal_gqa_b2h32kv8n4096d128", 1),
                        (PREFILL_DEFAULT, 1)):
        if heads is None:
            w = WORKLOADS[name]
            a = prefill_inputs(w, seed=seed)
            samples.append((name, f"whole workload", w, prefill_flops(w),
                            (lambda a=a, w=w: oracle.attention(a["q"], a["k"], a["v"], w.causal, a["scale"]))))
        else:
            sw, fn, w = head_sample(name, heads)
            samples.append((name, f"{heads} of {w.H} query heads (batch entry 0)", sw, prefill_flops(sw), fn))
    da, dw = dc.a, dc.w
    samples.append((dw.name, "whole workload", dw, decode_bytes(dw, da["seq_lens"]),
                    lambda: oracle.paged_decode(da["q"], da["k_cache"], da["v_cache"], da["block_table"],
                                                da["seq_lens"], da["scale"])))
    per, times = [], [0.0] * len(samples)
    passes = 0
    while passes == 0 or sum(times) < min_seconds:
        for i, (*_, fn) in enumerate(samples):
            t0 = time.perf_counter()
            fn()
            times[i] += time.perf_counter() - t0
        passes += 1
    for (name, what, w, work, _), t in zip(samples, times):
        t /= passes
        if name == dw.name:
            per.append({"workload": name, "sample": what, "seconds": round(t, 4), "value": round(work / t / 1e9, 4),
                        "unit": "GB/s"})
        else:
            per.append({"workload": name, "sample": what, "seconds": round(t, 4),
                        "value": round(work / t / 1e12, 6), "unit": "TFLOP/s"})
    head = next(e for e in per if e["workload"] == PREFILL_DEFAULT)
    dec = next(e for e in per if e["workload"] == dw.name)
    return {"value": head["value"], "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{PREFILL_DEFAULT}: {head['sample']} ({head['seconds']:.2f} s per pass); the other "
                      f"workloads' samples in per_config; {passes} passes, mean reported",
            "decode": {"value": dec["value"], "unit": "GB/s", "sample": dec["sample"]},
            "per_config": per, "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------- modes

def run_bench(args, torch, paa) -> dict:
    from workloads import WORKLOADS

    phases = Phases(torch)
    pc = PrefillCase(torch, paa, WORKLOADS[args.prefill_workload], args.seed)
    dc = DecodeCase(torch, paa, WORKLOADS[args.decode_workload], args.seed)
    pw, dw = pc.w, dc.w
    _log(f"inputs ready: {pw.name}, {dw.name}")

    # ---- W untimed steps, then exactly K timed steps, synchronised on both sides ----
    phases.start(f"step: prefill {pw.name} + decode {dw.name}")

    def step():
        pc()
        dc()

    prewarm(torch, step, PREWARM_S)
    for _ in range(args.warmup):
        pc()
        dc()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_beg.record()
    for i in range(K):
        ev[i][0].record()
        pc()
        ev[i][1].record()
        dc()
        ev[i][2].record()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_beg.elapsed_time(t_end) / K
    pre_ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
    dec_ms = statistics.fmean(e[1].elapsed_time(e[2]) for e in ev)
    _log(f"{K} steps: {ms_step:.4f} ms/step (prefill {pre_ms:.4f} ms, decode {dec_ms:.4f} ms)")

    pf = prefill_flops(pw)
    db = decode_bytes(dw, dc.a["seq_lens"])
    pre_tf = pf / (pre_ms * 1e-3) / 1e12
    dec_gbs = db / (dec_ms * 1e-3) / 1e9
    pre_roof = roofline("mfma", pre_tf, PEAK_BF16_TFLOPS, "TFLOP/s", read_traffic(pw.name), read_mfma_busy(pw.name))

    # ---- the shader clocks the prefill runs at (outside the timed region) ----
    phases.start(f"prefill {pw.name} back to back, shader clocks sampled")
    clocks = sample_gfx_clocks(torch, pc)
    pre_roof["measured_clock_ghz"] = round(clocks["mean_mhz"] / 1000.0, 3) if clocks else None
    # the same rate against the peak scaled to that clock (the peak is quoted at PEAK_CLOCK_GHZ)
    pre_roof["frac_at_measured_clock"] = (round(pre_tf / (PEAK_BF16_TFLOPS * clocks["mean_mhz"] / 1000.0 / PEAK_CLOCK_GHZ), 4)
                                          if clocks else None)
    _log(f"shader clocks under {pw.name}: {clocks['per_die_mhz'] if clocks else 'not available'}")

    # ---- decode with the 256 MB last-level cache evicted before every call ----
    # (by reading a 512 MB buffer: a read leaves clean lines, so no write-back lands inside the timed call)
    phases.start(f"decode {dw.name}, caches evicted before each call")
    scratch = torch.ones(512 << 18, dtype=torch.float32, device="cuda:0")
    cold = []
    for i in range(12):
        scratch.max()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dc()
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            cold.append(a.elapsed_time(b))
    del scratch
    cold_ms = statistics.median(cold)
    cold_gbs = db / (cold_ms * 1e-3) / 1e9
    dec_roof = roofline("hbm", cold_gbs, PEAK_HBM_GBS, "GB/s", read_traffic(dw.name))
    warm_roof = roofline("hbm", dec_gbs, PEAK_HBM_GBS, "GB/s", read_traffic(dw.name))
    _log(f"{dw.name}: cold {cold_ms * 1e3:.1f} us ({cold_gbs:.0f} GB/s), warm {dec_ms * 1e3:.1f} us")

    # ---- a decode step of many layers on a small batch, where launch overhead matters: one eager call per
    # layer against one replay of a graph holding every layer's call ----
    sw = WORKLOADS[SMALL_DECODE]
    phases.start(f"decode {sw.name} x {GRAPH_LAYERS} layers: eager calls, then graph replays")
    layers = [DecodeCase(torch, paa, sw, args.seed + i) for i in range(GRAPH_LAYERS)]
    graph = paa.PagedDecodeGraph([dict(q=c.q, k_cache=c.kc, v_cache=c.vc, block_table=c.bt, seq_lens=c.lens,
                                       scale=c.a["scale"], workspace=layers[0].ws, out=c.o, lse=c.lse)
                                  for c in layers])

    def loop_ms(fn, n=50):
        prewarm(torch, fn, 0.1)
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def eager_step():
        for c in layers:
            c()

    eager_ms = loop_ms(eager_step)
    graph_ms = loop_ms(graph.replay)
    graph.close()
    sdb = sum(decode_bytes(c.w, c.a["seq_lens"]) for c in layers)
    small = {"workload": sw.name, "layers": GRAPH_LAYERS, "eager_us_per_step": round(eager_ms * 1e3, 1),
             "graph_us_per_step": round(graph_ms * 1e3, 1), "algorithmic_bytes": round(sdb),
             "eager_gbs": round(sdb / (eager_ms * 1e-3) / 1e9, 1), "graph_gbs": round(sdb / (graph_ms * 1e-3) / 1e9, 1)}
    _log(f"{sw.name} x {GRAPH_LAYERS}: eager {eager_ms * 1e3:.1f} us/step, graph replay {graph_ms * 1e3:.1f} us/step")
    del layers, graph

    # ---- chunked prefill over a paged cache, with the chunk appended ----
    cc = ChunkedCase(torch, paa, WORKLOADS[CHUNKED], args.seed)
    phases.start(f"chunked prefill {CHUNKED}")
    med, mean = timed(torch, cc, 20, 3)
    c_tf = chunked_flops(cc.w, cc.a["ctx_lens"]) / (mean * 1e-3) / 1e12
    chunked = {"workload": CHUNKED, "ms": round(mean, 4), "ms_median": round(med, 4), "value": round(c_tf, 2),
               "unit": "TFLOP/s", "algorithmic_gflop": round(chunked_flops(cc.w, cc.a["ctx_lens"]) / 1e9, 3),
               "exponentials_g": round(chunked_flops(cc.w, cc.a["ctx_lens"]) / (4.0 * cc.w.d) / 1e9, 4),
               "algorithmic_mb": round(chunked_bytes(cc.w, cc.a["ctx_lens"]) / 1e6, 3),
               "roofline": roofline("mfma", c_tf, PEAK_BF16_TFLOPS, "TFLOP/s", read_traffic(CHUNKED),
                                    read_mfma_busy(CHUNKED))}
    _log(f"{CHUNKED}: {mean:.4f} ms, {c_tf:.1f} TFLOP/s")
    del cc

    more = []
    if not args.no_more:
        for name in PREFILL_MORE:
            c = PrefillCase(torch, paa, WORKLOADS[name], args.seed)
            phases.start(f"prefill {name}")
            med, mean = timed(torch, c, 20, 3)
            tf = prefill_flops(c.w) / (mean * 1e-3) / 1e12
            more.append({"workload": name, "ms": round(mean, 4), "ms_median": round(med, 4),
                         "value": round(tf, 2), "unit": "TFLOP/s",
                         "roofline": roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", read_traffic(name),
                                              read_mfma_busy(name))})
            del c
            _log(f"{name}: {mean:.4f} ms, {tf:.1f} TFLOP/s")

    fp8 = []
    if not args.no_more:
        for name in FP8_MORE:
            c = Fp8Case(torch, paa, WORKLOADS[name], args.seed)
            phases.start(f"prefill {name}")
            med, mean = timed(torch, c, 20, 3)
            tf = prefill_flops(c.w) / (mean * 1e-3) / 1e12
            fp8.append({"workload": name, "ms": round(mean, 4), "ms_median": round(med, 4), "value": round(tf, 2),
                        "unit": "TFLOP/s", "dtype": "fp8 e4m3 in, bf16 out",
                        "roofline": roofline("mfma", tf, PEAK_FP8_TFLOPS, "TFLOP/s", read_traffic(name),
                                             read_mfma_busy(name))})
            del c
            _log(f"{name}: {mean:.4f} ms, {tf:.1f} TFLOP/s")

    fp8_decode = None
    if not args.no_more:
        c = Fp8DecodeCase(torch, paa, dw, args.seed)
        phases.start(f"decode {c.name}")
        med, mean = timed(torch, c, 50, 5)
        fb = decode_bytes(dw, c.a["seq_lens"], kv_bytes=1)
        gbs = fb / (mean * 1e-3) / 1e9
        fp8_decode = {"workload": c.name, "ms": round(mean, 5), "ms_median": round(med, 5), "value": round(gbs, 2),
                      "unit": "GB/s", "dtype": "e4m3 K/V cache, bf16 q and out", "algorithmic_gb": round(fb / 1e9, 5),
                      "tokens_per_s": round(float(c.a["seq_lens"].sum()) / (mean * 1e-3)),
                      "speedup_vs_bf16_cache": round(dec_ms / mean, 3),
                      "roofline": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", read_traffic(c.name))}
        del c
        _log(f"{fp8_decode['workload']}: {mean:.4f} ms, {gbs:.1f} GB/s")

    base = None
    if not args.no_cpu_baseline:
        base = cpu_baseline(args.seed, dc)
        _log(f"cpu baseline: {base['sample']}")

    props = torch.cuda.get_device_properties(0)
    return {
        "metric": METRIC,
        "value": round(pre_tf, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "prewarm_s": PREWARM_S,
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
                              "tokens": int(dc.a["seq_lens"].sum())},
                   "seed": args.seed},
        "roofline": dict(pre_roof, kernel="attn_fwd: prefill_pp_kernel<128, causal, 4 heads, 2 stages>",
                         workload=pw.name, flops_per_call=round(pf)),
        "targets": {"prefill_frac_of_bf16_peak": 0.5, "decode_frac_of_hbm_peak": 0.7},
        "prefill": {"workload": pw.name, "ms": round(pre_ms, 5), "value": round(pre_tf, 3), "unit": "TFLOP/s",
                    "algorithmic_gflop": round(pf / 1e9, 4), "algorithmic_mb": round(prefill_bytes(pw) / 1e6, 3),
                    "exponentials_g": round(pw.B * pw.H * pw.visible_pairs() / 1e9, 4), "roofline": pre_roof,
                    "clocks": clocks},
        "decode": {"workload": dw.name, "ms": round(cold_ms, 5), "value": round(cold_gbs, 2), "unit": "GB/s",
                   "caches": "evicted before each call (512 MB read between calls)",
                   "algorithmic_gb": round(db / 1e9, 5), "roofline": dict(dec_roof, kernel=(
                       "paged_attn_decode: decode_partial_kernel + decode_reduce_kernel"), bytes_per_call=round(db)),
                   "warm_ms": round(dec_ms, 5), "warm_value": round(dec_gbs, 2), "warm_roofline": warm_roof},
        "prefill_more": more,
        "chunked_prefill": chunked,
        "fp8_prefill": fp8,
        "fp8_decode": fp8_decode,
        "decode_graph": small,
        "cpu_baseline": base,
        "phases": phases.names,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }


def run_pmc_pass(args, torch, paa) -> dict:
    """A short run for hardware counters: a calibration copy, then a few calls of each workload."""
    from workloads import WORKLOADS

    phases = Phases(torch)
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    phases.start(f"copy {COPY_BYTES} bytes")
    for _ in range(PMC_CALLS):
        torch.neg(src, out=dst)
    del src, dst
    cases = [DecodeCase(torch, paa, WORKLOADS[args.decode_workload], args.seed),
             PrefillCase(torch, paa, WORKLOADS[args.prefill_workload], args.seed)]
    cases += [PrefillCase(torch, paa, WORKLOADS[n], args.seed) for n in PREFILL_MORE]
    cases.append(ChunkedCase(torch, paa, WORKLOADS[CHUNKED], args.seed))
    cases += [Fp8Case(torch, paa, WORKLOADS[n], args.seed) for n in FP8_MORE]
    cases.append(Fp8DecodeCase(torch, paa, WORKLOADS[args.decode_workload], args.seed))
    for c in cases:
        phases.start(getattr(c, "name", c.w.name))
        for _ in range(PMC_CALLS):
            c()
    torch.cuda.synchronize()
    return {"phases": phases.names, "sources": source_digest()}


# ----------------------------------------------------------------- rocprofv3 summaries

def _split_phases(dispatches, n_phases):
    """Split dispatches (sorted by start) into phases at the n_phases-1 largest idle gaps."""
    if n_phases <= 1 or len(dispatches) < 2:
        return [dispatches]
    gaps = sorted(range(1, len(dispatches)),
                  key=lambda i: dispatches[i]["start"] - dispatches[i - 1]["end"], reverse=True)[:n_phases - 1]
    cuts = [0] + sorted(gaps) + [len(dispatches)]
    return [dispatches[a:b] for a, b in zip(cuts, cuts[1:])]


def _short(name: str) -> str:
    name = name.replace("paa::(anonymous namespace)::", "")
    return name.split("(")[0] if name.startswith("void ") is False else name[5:].split("(")[0]


def _load_dispatches(d):
    out = []
    for p in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(p)):
            out.append({"name": r["Kernel_Name"], "start": int(r["Start_Timestamp"]), "end": int(r["End_Timestamp"]),
                        "grid": (r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"]), "wg": r["Workgroup_Size_X"],
                        "vgpr": r["VGPR_Count"], "agpr": r.get("Accum_VGPR_Count", ""), "lds": r["LDS_Block_Size"]})
    out.sort(key=lambda x: x["start"])
    return out


def summarize_trace(trace_dir, bench_json, command) -> str:
    with open(bench_json) as f:
        line = [l for l in f if l.startswith("{")][-1]
    bench = json.loads(line)
    names = bench["phases"]
    ds = _load_dispatches(trace_dir)
    ours = [d for d in ds if "paa::" in d["name"] or "reduce_kernel" in d["name"]]
    groups = _split_phases(ours, len(names))
    out = ["# rocprofv3 kernel trace: attention kernels on the bench workloads", "",
           f"Command (run from the repository root): `{command}`", "",
           f"Kernel sources digest: `{source_digest()}`", "",
           "Durations are rocprofv3 kernel-trace start/end per dispatch (ns), grouped by the bench phase the "
           "dispatch fell in (phases are separated by idle gaps) and by kernel.", "",
           "| phase | kernel | grid | wg | calls | avg us | min us | max us |", "|---|---|---|---|---|---|---|---|"]
    for name, g in zip(names, groups):
        by = {}
        for d in g:
            by.setdefault((_short(d["name"]), d["grid"], d["wg"]), []).append(d["end"] - d["start"])
        for (k, grid, wg), t in by.items():
            out.append(f"| {name} | `{k}` | {'x'.join(grid)} | {wg} | {len(t)} | {statistics.fmean(t) / 1e3:.2f} | "
                       f"{min(t) / 1e3:.2f} | {max(t) / 1e3:.2f} |")
    out += ["", "Bench line of the same run (event-timed, not under the profiler's overhead):", "",
            "```", json.dumps({k: bench.get(k) for k in ("ms_per_step", "prefill", "decode", "prefill_more")},
                              indent=1), "```"]
    return "\n".join(out) + "\n"


def _load_counters(d, counter):
    rows = []
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(p)):
            if r["Counter_Name"] != counter:
                continue
            if "paa::" not in r["Kernel_Name"] and COPY_KERNEL_TAG not in r["Kernel_Name"]:
                continue
            rows.append({"name": r["Kernel_Name"], "value": float(r["Counter_Value"]),
                         "start": int(r["Start_Timestamp"]), "end": int(r["End_Timestamp"])})
    rows.sort(key=lambda x: x["start"])
    return rows


def summarize_counters(fetch_dir, write_dir, pass_json, command) -> str:
    """JSON lines: per workload, HBM bytes per call (FETCH_SIZE + WRITE_SIZE, calibrated by the copy)."""
    with open(pass_json) as f:
        meta = json.loads([l for l in f if l.startswith("{")][-1])
    names = meta["phases"]
    per = {}
    factors = {}
    lines = ["# HBM traffic per call from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch).",
             f"# Commands (repository root): {command}",
             f"# Each counter is scaled by the factor that maps its reading for a plain copy kernel "
             f"(elementwise negate of {COPY_BYTES} bytes of bf16) to the {COPY_BYTES} bytes it must read "
             f"and the {COPY_BYTES} bytes it must write."]
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        groups = _split_phases(_load_counters(d, counter), len(names))
        if len(groups) != len(names) or any(COPY_KERNEL_TAG not in r["name"] for r in groups[0]):
            raise SystemExit(f"{counter}: dispatches do not split into the pass's phases {names}")
        kib = statistics.median(r["value"] for r in groups[0])
        factors[counter] = COPY_BYTES / (kib * 1024.0)
        lines.append(f"# {counter}: the copy reads {kib:.0f} KiB per dispatch -> factor {factors[counter]:.4f}")
        for name, g in zip(names[1:], groups[1:]):
            per.setdefault(name, {})[counter] = sum(r["value"] for r in g) / PMC_CALLS * 1024.0 * factors[counter]
            per[name].setdefault("kernels", sorted({_short(r["name"]) for r in g}))
    for name in names[1:]:
        e = {"workload": name, "kernels": per[name]["kernels"],
             "fetch_bytes_per_call": round(per[name]["FETCH_SIZE"]),
             "write_bytes_per_call": round(per[name]["WRITE_SIZE"]),
             "hbm_bytes_per_call": round(per[name]["FETCH_SIZE"] + per[name]["WRITE_SIZE"]),
             "sources": meta["sources"]}
        lines.append(json.dumps(e))
    return "\n".join(lines) + "\n"


MFMA_COUNTERS = ("MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8")


def summarize_mfma(mfma_dir, pass_json, command) -> str:
    """JSON lines: per workload and kernel, the matrix-core use one rocprofv3 --pmc run of MFMA_COUNTERS
    measured: MfmaUtil (MFMA-busy cycles over GPU-active cycles times SIMDs, %), the MFMA flops executed per
    call (MOPS x 512) against the workload's algorithmic flops, and the share of MFMA-busy cycles in which a
    VALU instruction also issued."""
    from workloads import WORKLOADS, PrefillWorkload
    with open(pass_json) as f:
        meta = json.loads([l for l in f if l.startswith("{")][-1])
    names = meta["phases"]
    per = {}
    for counter in MFMA_COUNTERS:
        groups = _split_phases(_load_counters(mfma_dir, counter), len(names))
        if len(groups) != len(names) or any(COPY_KERNEL_TAG not in r["name"] for r in groups[0]):
            raise SystemExit(f"{counter}: dispatches do not split into the pass's phases {names}")
        for name, g in zip(names[1:], groups[1:]):
            for r in g:
                k = per.setdefault((name, _short(r["name"])), {})
                k.setdefault(counter, []).append(r["value"])
    lines = ["# Matrix-core use per workload and kernel from one rocprofv3 --pmc run (per-dispatch means).",
             f"# Command (repository root): {command}",
             "# mfma_util_pct: MfmaUtil = sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) x 100.",
             "# mfma_tflop_per_call: (SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F8) x 512 / 1e12; algorithmic_tflop: the",
             "# workload's 4*d*visible-pairs count (prefill only); coexec_share: SQ_VALU_MFMA_COEXEC_CYCLES /",
             "# SQ_VALU_MFMA_BUSY_CYCLES, the MFMA-busy cycles in which a VALU instruction issued too."]
    for (name, kernel), c in per.items():
        mean = {k: statistics.fmean(v) for k, v in c.items()}
        flops = (mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + mean.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)) * 512
        e = {"workload": name, "kernel": kernel, "mfma_util_pct": round(mean["MfmaUtil"], 2),
             "mfma_tflop_per_call": round(flops / 1e12, 5)}
        w = WORKLOADS.get(name)
        if isinstance(w, PrefillWorkload):
            e["algorithmic_tflop"] = round(prefill_flops(w) / 1e12, 5)
        busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        if busy > 0:
            e["coexec_share"] = round(mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy, 4)
        e["sources"] = meta["sources"]
        lines.append(json.dumps(e))
    return "\n".join(lines) + "\n"


WAVE_COUNTERS = (("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VMEM"),
                 ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
                  "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_MISC", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_LDS"))


def summarize_waves(dir1, dir2, pass_json, command) -> str:
    """JSON lines: per workload and kernel, where the waves' cycles go, from two rocprofv3 --pmc runs of
    WAVE_COUNTERS: the shares of all wave-cycles spent issuing (any instruction, and VALU including MFMA, LDS,
    VMEM, scalar), waiting for an instruction to issue (the pipe is taken by the SIMD's other wave, or an
    operand is not ready) and waiting at s_waitcnt or a barrier; LDS bank-conflict cycles per LDS-active
    cycle."""
    with open(pass_json) as f:
        meta = json.loads([l for l in f if l.startswith("{")][-1])
    names = meta["phases"]
    per = {}
    for d, counters in zip((dir1, dir2), WAVE_COUNTERS):
        for counter in counters:
            groups = _split_phases(_load_counters(d, counter), len(names))
            if len(groups) != len(names) or any(COPY_KERNEL_TAG not in r["name"] for r in groups[0]):
                raise SystemExit(f"{counter}: dispatches do not split into the pass's phases {names}")
            for name, g in zip(names[1:], groups[1:]):
                for r in g:
                    per.setdefault((name, _short(r["name"])), {}).setdefault(counter, []).append(r["value"])
    lines = ["# Where the waves' cycles go, per workload and kernel, from two rocprofv3 --pmc runs (per-dispatch",
             "# means of counters summed over waves), as % of SQ_WAVE_CYCLES.",
             f"# Command (repository root): {command}",
             "# issuing: SQ_ACTIVE_INST_ANY (of it VALU incl. MFMA, LDS, VMEM, scalar); waiting_to_issue:",
             "# SQ_WAIT_INST_ANY; waiting_waitcnt_or_barrier: SQ_WAIT_ANY; lds_bank_conflict: SQ_LDS_BANK_CONFLICT /",
             "# SQ_LDS_IDX_ACTIVE."]
    for (name, kernel), c in per.items():
        mean = {k: statistics.fmean(v) for k, v in c.items()}
        wc = mean.get("SQ_WAVE_CYCLES", 0.0)
        if wc <= 0:
            continue
        pct = lambda k: round(100.0 * mean.get(k, 0.0) / wc, 1)  # noqa: E731
        lds = mean.get("SQ_LDS_IDX_ACTIVE", 0.0)
        lines.append(json.dumps({
            "workload": name, "kernel": kernel, "issuing_pct": pct("SQ_ACTIVE_INST_ANY"),
            "valu_incl_mfma_pct": pct("SQ_ACTIVE_INST_VALU"), "lds_pct": pct("SQ_ACTIVE_INST_LDS"),
            "vmem_pct": pct("SQ_ACTIVE_INST_VMEM"), "scalar_pct": pct("SQ_ACTIVE_INST_SCA"),
            "waiting_to_issue_pct": pct("SQ_WAIT_INST_ANY"), "waiting_to_issue_lds_pct": pct("SQ_WAIT_INST_LDS"),
            "waiting_waitcnt_or_barrier_pct": pct("SQ_WAIT_ANY"),
            "lds_bank_conflict_pct": round(100.0 * mean.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds, 2) if lds else None,
            "sources": meta["sources"]}))
    return "\n".join(lines) + "\n"


# ----------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--prefill-workload", default=PREFILL_DEFAULT)
    ap.add_argument("--decode-workload", default=DECODE_DEFAULT)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-more", action="store_true", help="skip the larger prefill workloads")
    ap.add_argument("--pmc-pass", action="store_true", help="short run for a rocprofv3 --pmc pass")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"))
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "PASS_JSON"))
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_DIR", "PASS_JSON"))
    ap.add_argument("--summarize-waves", nargs=3, metavar=("PASS1_DIR", "PASS2_DIR", "PASS_JSON"))
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    args = ap.parse_args()

    if args.summarize_trace:
        sys.stdout.write(summarize_trace(*args.summarize_trace, args.command))
        return 0
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(*args.summarize_counters, args.command))
        return 0
    if args.summarize_mfma:
        sys.stdout.write(summarize_mfma(*args.summarize_mfma, args.command))
        return 0
    if args.summarize_waves:
        sys.stdout.write(summarize_waves(*args.summarize_waves, args.command))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "the kernels run on one MI355X and have no multi-GPU path", file=sys.stderr)
        return 2

    import torch

    import paged_attention_attn_amd as paa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if not os.path.exists(paa.LIB_PATH):
        from paged_attention_attn_amd import build
        build.build()

    line = run_pmc_pass(args, torch, paa) if args.pmc_pass else run_bench(args, torch, paa)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
