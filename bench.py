#!/usr/bin/env python3
"""Benchmark of the gemm15 hot path on one MI355X.

Headline: TFLOPS = 2*M*N*K / median call time at M = N = K = 4096 with bf16
inputs, fp32 accumulation and fp32 C (the square-GEMM workload), reported as a
fraction of the gfx950 dense bf16 matrix peak; the same 4096^3 product with
fp32 inputs (SGEMM) is measured beside it against the fp32 peak. Inputs are
seeded synthetic uniform[-1, 1) matrices already resident in HBM.

Protocol: W untimed warm-up calls (continued until the product has run for at
least SETTLE_S seconds, so the clocks have left their idle state), then K timed
calls, each bracketed by a pair of HIP events recorded on the stream the kernel runs on; per-call time is the
median (throughput) and the mean (roofline: average launch duration). The
whole timed region is also bracketed by device synchronisation.

``cpu_baseline`` times the fp64 host oracle on a bounded row-block of the same
product on the host's cores.

The same line carries ``configs``: every configuration of the benchmark set (FP16
512^3, FP32 4096^3, BF16/FP16 4096^3, the encoder FFN pair and chain, the 96
attention-score heads and the odd shapes), each timed by the protocol below and
inside a replayed HIP graph, with its roofline fraction against its own bound.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--all] [--no-cpu] [--vendor]
       [--ladder] [--no-configs]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}  # 256 CU x 2.4 GHz x {4096, 256}
PEAK_HBM_GBS = 8000.0
# Minimum length of the untimed warm-up. Coming out of idle the GPU's clocks take
# tens of milliseconds to settle: at 4096^3 bf16 the per-call median after 10 calls
# (1.3 ms) is 127-131 us, after 0.05 s of calls 121 us, and it stays there up to
# 3 s (the vendor library's product goes 120 -> 106 us alike). The timed calls are
# meant to see the steady state, so the warm-up lasts W calls and at least this long.
SETTLE_S = 0.25
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# Sources each measured kernel is built from (its file and the headers it
# includes): its counter data are stale once any of them changes.
_COMMON = ["kernels.hpp", "device_common.hpp"]
KERNEL_SOURCES = {
    "m16d": ["kernel_mfma16_dlds.hip", "m16_common.hpp"] + _COMMON,
    "m16n": ["kernel_mfma16_nt.hip", "m16_common.hpp"] + _COMMON,
    "m16t": ["kernel_mfma16_nt.hip", "m16_common.hpp"] + _COMMON,
    "m16s": ["kernel_mfma16_k1.hip", "m16_common.hpp"] + _COMMON,
    "m16w": ["kernel_mfma16_w.hip", "m16_common.hpp"] + _COMMON,
    "f32d": ["kernel_f32_dlds.hip"] + _COMMON,
    "gemv": ["kernel_gemv.hip"] + _COMMON,
}


def kernel_source_hash(config: str | None = None) -> str:
    """Hash of the device sources of configuration `config` (all of them when the
    configuration's family is not listed)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "dense_gemm_15_amd", "csrc")
    names = KERNEL_SOURCES.get((config or "").split("_")[0])
    files = ([os.path.join(csrc, n) for n in names] if names
             else sorted(glob.glob(os.path.join(csrc, "*"))))
    h = hashlib.sha256()
    for f in files:
        with open(f) as fh:
            h.update(os.path.basename(f).encode() + code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def code_only(src: str) -> str:
    """C++ source without comments, trailing blanks and empty lines: what a hash of
    the code should see (editing a comment does not change the kernel)."""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())


def measured_traffic(kernel_config: str):
    """Bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary, or None
    when it is missing or was taken from other sources of that kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    row = t.get("kernels", {}).get(kernel_config)
    if row is None or row.get("source_hash") != kernel_source_hash(kernel_config):
        return None
    return row.get("traffic_bytes")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr + json)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration block (every workload of the benchmark set)")
    ap.add_argument("--json-out", default=None, help="write per-workload results here")
    ap.add_argument("--ladder", action="store_true",
                    help="also time the optimisation ladder V0..V4 on the 4096^3 fp16 product "
                         "and the fp16-accumulation variant")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch.mm (the vendor library) and this library on the "
                         "4096^3 bf16 product with bf16 output, for context")
    ap.add_argument("--attention", action="store_true",
                    help="also time the attention workload alone (its stages, the fused "
                         "QK^T + softmax kernel and both chains); part of --all")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def time_calls(fn, steps, warmup, settle_s=None):
    """Median and mean per-call milliseconds over `steps` event-bracketed calls,
    after `warmup` untimed calls that continue until the GPU has run the product
    for `settle_s` seconds (see SETTLE_S)."""
    import torch
    settle_s = SETTLE_S if settle_s is None else settle_s
    t_warm = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t_warm < settle_s:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2])
    return med, sum(ms) / len(ms), wall


def time_protocol(fn, steps, warmup):
    """The measurement protocol of the benchmark: warm-up (as time_calls), then
    `steps` samples, each an event pair around R back-to-back calls, R = 1 when a call
    takes at least 50 us, otherwise enough calls for a sample of 200 us; per-call time
    = median sample / R. Returns (median_ms, mean_ms, R)."""
    import torch
    med1, _, _ = time_calls(fn, 5, warmup)
    reps = 1 if med1 >= 0.05 else max(1, int(0.2 / max(med1, 1e-4)) + 1)
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) / reps for a, b in ev)
    med = ms[len(ms) // 2] if len(ms) % 2 else 0.5 * (ms[len(ms) // 2 - 1] + ms[len(ms) // 2])
    return med, sum(ms) / len(ms), reps


def time_graph(fn, reps=20, replays=7):
    """Median per-call milliseconds of `reps` calls captured in one HIP graph and
    replayed: the GPU time of a call without the host's launch overhead, which
    dominates the event-per-call time of a kernel of a few microseconds."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    ts = []
    st = torch.cuda.current_stream()
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        graph.replay()
        b.record(st)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / reps)
    del graph
    return sorted(ts)[len(ts) // 2]


def workspace_for(plan, dev):
    """The plan's scratch, allocated once outside the timed calls (None: needs none)."""
    import torch
    n = plan.workspace_bytes
    return torch.empty(n, dtype=torch.uint8, device=dev) if n else None


def gemm_workload(g, name, steps, warmup, graph=False, b_layout="kn"):
    import torch
    import synth
    w = synth.WORKLOADS[name]
    A, B = synth.gemm_inputs(name)
    if b_layout == "nk":
        B = B.t().contiguous()  # the same product with B stored transposed (Bt [N x K])
    dev = torch.device("cuda")
    A, B = A.to(dev), B.to(dev)
    M, N, K = w["M"], w["N"], w["K"]
    plan = g.Plan(M, N, K, w["dtype"], b_layout=b_layout)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = workspace_for(plan, dev)
    run = lambda: plan.run(A, B, out=C, workspace=ws)  # noqa: E731
    med, mean, wall = time_calls(run, steps, warmup)
    flops = 2 * M * N * K
    es = 4 if w["dtype"] == "f32" else 2
    byts = (M * K + K * N) * es + M * N * 4
    r = dict(workload=name + ("_nt" if b_layout == "nk" else ""), M=M, N=N, K=K, dtype=w["dtype"],
             config=plan.config_name, b_layout=b_layout,
             median_ms=med, mean_ms=mean, wall_s=wall, flops=flops, bytes=byts,
             tflops=flops / (med * 1e-3) / 1e12,
             tflops_mean=flops / (mean * 1e-3) / 1e12,
             gbs=byts / (med * 1e-3) / 1e9,
             frac_peak=flops / (mean * 1e-3) / 1e12 / PEAK_TFLOPS[w["dtype"]])
    if graph:
        gms = time_graph(run)
        r.update(graph_ms=gms, graph_tflops=flops / (gms * 1e-3) / 1e12,
                 graph_gbs=byts / (gms * 1e-3) / 1e9)
    return r


# The optimisation ladder of the DeepGEMM page (section 4.1) on this chip: V0 one
# thread per element, V1 LDS tiles, V2 register tiles, V3 padded LDS rows (and
# V3a, padding that keeps 16-byte rows: section 5.2), V4 matrix instructions on
# the same 64 x 64 tile, then this library's own choice.
LADDER = [("V0 one thread per element", "ladder_v0_f16_16x16"),
          ("V1 LDS tiles", "ladder_v1_f16_16x16x16"),
          ("V2 register tiles", "ladder_v2_f16_64x64x16"),
          ("V3 padded LDS rows (65 floats)", "ladder_v3_f16_64x64x16"),
          ("V3a aligned padding (68 floats)", "ladder_v3a_f16_64x64x16"),
          ("V4 matrix instructions", "mfma16_f16_64x64_w2x2"),
          ("this library", None)]


def ladder_workload(g, steps):
    """Each rung on the 4096^3 fp16 product (fp32 accumulation, fp32 C), with as
    many calls as fit about half a second (at least 3, at most `steps`); then the
    fp16-accumulating rung and its maximum absolute difference from this
    library's fp32-accumulating result on the same inputs (DeepGEMM page, section
    3.4)."""
    import torch
    import synth
    A, B = synth.gemm_inputs("fp16_4096")
    dev = torch.device("cuda")
    A, B = A.to(dev), B.to(dev)
    n = A.shape[0]
    flops = 2 * n * n * n
    rungs = []
    outs = {}
    for tag, cfg in LADDER + [("V3, fp16 accumulator", "ladder_v3acc16_f16_64x64x16")]:
        plan = g.Plan(n, n, n, "f16", config=cfg if cfg else -1)
        C = torch.empty((n, n), dtype=torch.float32, device=dev)
        run = lambda: plan.run(A, B, out=C)  # noqa: E731
        t0 = time.perf_counter()
        run()
        torch.cuda.synchronize()
        first = time.perf_counter() - t0
        k = max(3, min(steps, int(0.5 / max(first, 1e-6))))
        med, mean, _ = time_calls(run, k, 1, settle_s=min(SETTLE_S, 10 * first))
        rungs.append(dict(rung=tag, config=plan.config_name, calls=k, median_ms=med,
                          tflops=flops / (med * 1e-3) / 1e12,
                          frac_peak=flops / (med * 1e-3) / 1e12 / PEAK_TFLOPS["f16"]))
        print(f"[bench] ladder {json.dumps(rungs[-1])}", file=sys.stderr, flush=True)
        if cfg is None or "acc16" in (cfg or ""):
            outs[tag] = C
    ref = outs["this library"].double()
    err16 = (outs["V3, fp16 accumulator"].double() - ref).abs().max().item()
    return dict(rungs=rungs, fp16_accumulation_max_abs_diff=err16,
                note="fp16-accumulator result against this library's fp32-accumulating "
                     "result on the same 4096^3 fp16 inputs")


def vendor_reference(g, steps, warmup):
    """4096^3 bf16 with bf16 output: torch.mm (the vendor library) and this library,
    timed alike, one after the other on the same inputs. Context only."""
    import torch
    import synth
    A, B = synth.gemm_inputs("bf16_4096")
    dev = torch.device("cuda")
    A, B = A.to(dev), B.to(dev)
    n = A.shape[0]
    C = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    plan = g.Plan(n, n, n, "bf16", out_dtype="bf16")
    flops = 2 * n * n * n
    out = {}
    for tag, fn in (("torch_mm", lambda: torch.mm(A, B, out=C)),
                    ("gemm15", lambda: plan.run(A, B, out=C))):
        med, mean, _ = time_calls(fn, steps, warmup)
        out[tag] = dict(median_ms=med, mean_ms=mean, tflops=flops / (med * 1e-3) / 1e12)
    out["gemm15"]["config"] = plan.config_name
    return out


def ffn_workload(g, steps, warmup, b_layout="kn"):
    """The encoder FFN pair; b_layout="nk" keeps the weights in [out, in] order."""
    import torch
    import synth
    X, W1, b1, W2, b2 = synth.ffn_inputs()
    T, Hd, F = X.shape[0], X.shape[1], W1.shape[1]
    if b_layout == "nk":
        W1, W2 = W1.t().contiguous(), W2.t().contiguous()
    dev = torch.device("cuda")
    X, W1, b1, W2, b2 = (t.to(dev) for t in (X, W1, b1, W2, b2))
    p1 = g.Plan(T, F, Hd, "bf16", bias=True, gelu=True, out_dtype="bf16", b_layout=b_layout)
    p2 = g.Plan(T, Hd, F, "bf16", bias=True, resid=True, out_dtype="bf16", b_layout=b_layout)
    H = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((T, Hd), dtype=torch.bfloat16, device=dev)
    out = {}
    sfx = "_nt" if b_layout == "nk" else ""
    for tag, fn, fl, by in (
        ("ffn1" + sfx, lambda: p1.run(X, W1, bias=b1, out=H), 2 * T * F * Hd,
         (T * Hd + Hd * F + T * F) * 2 + F * 4),
        ("ffn2" + sfx, lambda: p2.run(H, W2, bias=b2, resid=X, out=Y), 2 * T * F * Hd,
         (T * F + F * Hd + 2 * T * Hd) * 2 + Hd * 4),
    ):
        med, mean, wall = time_calls(fn, steps, warmup)
        gms = time_graph(fn)
        out[tag] = dict(workload=tag, median_ms=med, mean_ms=mean, flops=fl, bytes=by,
                        config=(p1 if tag.startswith("ffn1") else p2).config_name,
                        tflops=fl / (med * 1e-3) / 1e12, gbs=by / (med * 1e-3) / 1e9,
                        frac_peak=fl / (mean * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                        graph_ms=gms, graph_tflops=fl / (gms * 1e-3) / 1e12)
    return out


def qk_workload(g, steps, warmup, b_layout="kn"):
    """96 heads of Q K^T; "kn" takes the materialised K^T [64 x 512] per head,
    "nk" takes K as stored [512 x 64] (no transposed copy)."""
    import torch
    import synth
    Q, Kt = synth.qk_inputs()
    if b_layout == "nk":
        Kt = Kt.transpose(1, 2).contiguous()
    dev = torch.device("cuda")
    Q, Kt = Q.to(dev), Kt.to(dev)
    nb, S, D = Q.shape
    plan = g.Plan(S, S, D, "bf16", batch_hint=nb, b_layout=b_layout)
    out = torch.empty((nb, S, S), dtype=torch.float32, device=dev)
    run = lambda: plan.run_batched(Q, Kt, out=out)  # noqa: E731
    med, mean, wall = time_calls(run, steps, warmup)
    gms = time_graph(run)
    fl = 2 * nb * S * S * D
    by = nb * (2 * S * D * 2 + S * S * 4)
    return dict(workload="qk_96x512x512x64" + ("_nt" if b_layout == "nk" else ""), median_ms=med,
                mean_ms=mean, flops=fl, bytes=by,
                config=plan.config_name, tflops=fl / (med * 1e-3) / 1e12,
                gbs=by / (med * 1e-3) / 1e9, frac_hbm=by / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS,
                graph_ms=gms, graph_tflops=fl / (gms * 1e-3) / 1e12,
                graph_frac_hbm=by / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS)


def attention_workload(g, steps, warmup):
    """Attention continuation (tutorial page, section 2: Softmax(Q K^T) V) on the 96
    heads of sequence 512, dimension 64: S = Q K^T (fp32), P = softmax(S) row by row
    (bf16), O = P V (fp32), each stage timed alone and the chain as a whole; then the
    first two stages as the one kernel of gemm_attention_probs and that chain. The
    softmax is HBM-bound: its bytes are S read once and P written once."""
    import torch
    import synth
    Q, Kt, V = synth.attention_inputs()
    dev = torch.device("cuda")
    Q, Kt, V = Q.to(dev), Kt.to(dev), V.to(dev)
    nb, Sq, D = Q.shape
    qk = g.Plan(Sq, Sq, D, "bf16", batch_hint=nb)
    pv = g.Plan(Sq, D, Sq, "bf16", batch_hint=nb)
    S = torch.empty((nb, Sq, Sq), dtype=torch.float32, device=dev)
    P = torch.empty((nb, Sq, Sq), dtype=torch.bfloat16, device=dev)
    O = torch.empty((nb, Sq, D), dtype=torch.float32, device=dev)
    stages = {
        "qk": (lambda: qk.run_batched(Q, Kt, out=S), 2 * nb * Sq * Sq * D,
               nb * (2 * Sq * D * 2 + Sq * Sq * 4), qk.config_name),
        "softmax": (lambda: g.softmax_rows(S, 1.0, "bf16", out=P), 0, nb * Sq * Sq * (4 + 2),
                    "softmax_rows"),
        # QK^T and the softmax in one kernel: Q and K^T read, P written, S never stored
        "probs": (lambda: g.attention_probs(Q, Kt, 1.0, "kn", "bf16", out=P), 2 * nb * Sq * Sq * D,
                  nb * (2 * Sq * D * 2 + Sq * Sq * 2), "attention_probs"),
        "pv": (lambda: pv.run_batched(P, V, out=O), 2 * nb * Sq * Sq * D,
               nb * (Sq * Sq * 2 + Sq * D * 2 + Sq * D * 4), pv.config_name),
    }
    out = {}
    for name, (fn, fl, by, cfg) in stages.items():
        med, mean, _ = time_calls(fn, steps, warmup)
        gms = time_graph(fn)
        out[name] = dict(config=cfg, median_ms=med, graph_ms=gms, flops=fl, bytes=by,
                         gbs=by / (gms * 1e-3) / 1e9, frac_hbm=by / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         tflops=fl / (gms * 1e-3) / 1e12)

    def chain():
        qk.run_batched(Q, Kt, out=S)
        g.softmax_rows(S, 1.0, "bf16", out=P)
        pv.run_batched(P, V, out=O)
    med, mean, _ = time_calls(chain, steps, warmup)
    gms = time_graph(chain)
    out["chain"] = dict(median_ms=med, graph_ms=gms)

    def chain_fused():
        g.attention_probs(Q, Kt, 1.0, "kn", "bf16", out=P)
        pv.run_batched(P, V, out=O)
    med, mean, _ = time_calls(chain_fused, steps, warmup)
    gms = time_graph(chain_fused)
    out["chain_fused"] = dict(median_ms=med, graph_ms=gms)
    return dict(workload="attention_96x512x64", stages=out)


def baseline_configs(g, steps, warmup, head, f32):
    """Every configuration of the benchmark set on this chip, each with its bound:
    (1) FP16 512^3, (2) FP32 4096^3, (3) BF16 and FP16 4096^3, (4) the encoder FFN pair
    and its chain, (5) 96 attention-score heads and the three odd shapes. Times: `ms` by
    the event protocol (time_protocol), `graph_ms` per call inside a replayed HIP graph
    (GPU time without host launch gaps); the roofline fraction uses graph_ms, against
    the dense matrix peak of the input type (bound "mfma") or 8 TB/s of algorithmic
    bytes (bound "hbm": A and B read once, C written once, bias and residual read
    once); launch-bound shapes report both."""
    import torch
    import synth
    dev = torch.device("cuda")
    out = {}

    def entry(fn, flops, byts, bound, kernel, dtype):
        med, mean, reps = time_protocol(fn, steps, warmup)
        gms = time_graph(fn)
        e = dict(kernel=kernel, ms=round(med, 5), calls_per_sample=reps, graph_ms=round(gms, 5),
                 tflops=round(flops / (gms * 1e-3) / 1e12, 2),
                 gbs=round(byts / (gms * 1e-3) / 1e9, 1), bound=bound)
        f_m = flops / (gms * 1e-3) / 1e12 / PEAK_TFLOPS[dtype]
        f_h = byts / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS
        if bound == "mfma":
            e["frac"] = round(f_m, 4)
        elif bound == "hbm":
            e["frac"] = round(f_h, 4)
        else:  # launch/latency-bound: both figures
            e["frac_mfma"], e["frac_hbm"] = round(f_m, 4), round(f_h, 4)
        return e

    def gemm_entry(name, bound):
        w = synth.WORKLOADS[name]
        A, B = (t.to(dev) for t in synth.gemm_inputs(name))
        M, N, K, dt = w["M"], w["N"], w["K"], w["dtype"]
        plan = g.Plan(M, N, K, dt)
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = workspace_for(plan, dev)
        es = 4 if dt == "f32" else 2
        return entry(lambda: plan.run(A, B, out=C, workspace=ws), 2 * M * N * K,
                     (M * K + K * N) * es + M * N * 4, bound, plan.config_name, dt)

    out["1_fp16_512"] = gemm_entry("fp16_512", "launch")
    print(f"[bench] configs 1 {json.dumps(out['1_fp16_512'])}", file=sys.stderr, flush=True)
    out["2_fp32_4096"] = dict(kernel=f32["config"], ms=round(f32["median_ms"], 5),
                              tflops=round(f32["tflops"], 2), bound="mfma",
                              frac=round(f32["frac_peak"], 4))
    out["3_bf16_4096"] = dict(kernel=head["config"], ms=round(head["median_ms"], 5),
                              tflops=round(head["tflops"], 2), bound="mfma",
                              frac=round(head["frac_peak"], 4))
    out["3_fp16_4096"] = gemm_entry("fp16_4096", "mfma")
    print(f"[bench] configs 3 {json.dumps(out['3_fp16_4096'])}", file=sys.stderr, flush=True)

    X, W1, b1, W2, b2 = (t.to(dev) for t in synth.ffn_inputs())
    T, Hd, F = X.shape[0], X.shape[1], W1.shape[1]
    p1 = g.Plan(T, F, Hd, "bf16", bias=True, gelu=True, out_dtype="bf16")
    p2 = g.Plan(T, Hd, F, "bf16", bias=True, resid=True, out_dtype="bf16")
    H = torch.empty((T, F), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((T, Hd), dtype=torch.bfloat16, device=dev)
    w1, w2 = workspace_for(p1, dev), workspace_for(p2, dev)
    f1 = lambda: p1.run(X, W1, bias=b1, out=H, workspace=w1)  # noqa: E731
    f2 = lambda: p2.run(H, W2, bias=b2, resid=X, out=Y, workspace=w2)  # noqa: E731
    fl = 2 * T * F * Hd
    by1 = (T * Hd + Hd * F + T * F) * 2 + F * 4
    by2 = (T * F + F * Hd + 2 * T * Hd) * 2 + Hd * 4
    out["4_ffn1_bias_gelu_bf16"] = entry(f1, fl, by1, "mfma", p1.config_name, "bf16")
    out["4_ffn2_bias_resid_bf16"] = entry(f2, fl, by2, "mfma", p2.config_name, "bf16")

    def chain():
        f1()
        f2()
    out["4_ffn_chain"] = entry(chain, 2 * fl, by1 + by2, "mfma", "ffn1+ffn2", "bf16")
    print(f"[bench] configs 4 {json.dumps(out['4_ffn_chain'])}", file=sys.stderr, flush=True)

    Q, Kt = (t.to(dev) for t in synth.qk_inputs())
    nb, S, D = Q.shape
    pq = g.Plan(S, S, D, "bf16", batch_hint=nb)
    Sc = torch.empty((nb, S, S), dtype=torch.float32, device=dev)
    wq = workspace_for(pq, dev)
    out["5_qk_96x512x512x64"] = entry(lambda: pq.run_batched(Q, Kt, out=Sc, workspace=wq),
                                      2 * nb * S * S * D, nb * (2 * S * D * 2 + S * S * 4), "hbm",
                                      pq.config_name, "bf16")
    out["5_gemv_1x4096x4096"] = gemm_entry("gemv_1x4096x4096", "hbm")
    out["5_odd_127x1000x771"] = gemm_entry("odd_127x1000x771", "launch")
    out["5_odd_4095x4097x63"] = gemm_entry("odd_4095x4097x63", "hbm")
    # what a plain device-to-device copy reaches on this machine, beside the HBM-bound rows
    src = torch.empty(64 * 2**20, dtype=torch.float32, device=dev)  # 256 MiB
    dst = torch.empty_like(src)
    out["5_copy_reference_256MiB"] = entry(lambda: dst.copy_(src), 0, 2 * src.numel() * 4, "hbm",
                                           "device copy (torch)", "f32")
    del src, dst
    print(f"[bench] configs 5 {json.dumps({k: v for k, v in out.items() if k[0] == '5'})}",
          file=sys.stderr, flush=True)
    return out


def cpu_baseline(target_s=15.0):
    """The fp64 oracle on the 4096^3 bf16 product on all host cores: a row block
    sized to about `target_s` seconds, or the whole product repeated until that
    much time has passed when the whole product is faster."""
    import oracle
    import synth
    A, B = synth.gemm_inputs("bf16_4096")
    Ab, Bb = synth.bits(A), synth.bits(B)
    lib = oracle.load()
    oracle.gemm(Ab[:16], Bb, "bf16", lib=lib)  # first call: thread pool start-up
    rows = 128
    t0 = time.perf_counter()
    oracle.gemm(Ab[:rows], Bb, "bf16", lib=lib)
    t1 = time.perf_counter() - t0
    rows2 = int(max(16, min(4096, rows * target_s / max(t1, 1e-3))))
    reps, t2 = 0, 0.0
    while reps == 0 or (rows2 == 4096 and t2 < 0.66 * target_s):
        t0 = time.perf_counter()
        oracle.gemm(Ab[:rows2], Bb, "bf16", lib=lib)
        t2 += time.perf_counter() - t0
        reps += 1
    fl = 2 * rows2 * 4096 * 4096 * reps
    what = (f"rows 0..{rows2 - 1} of" if rows2 < 4096 else f"{reps} x the whole")
    # one core: the whole fp16 512^3 product on a single thread
    A5, B5 = synth.gemm_inputs("fp16_512")
    A5b, B5b = synth.bits(A5), synth.bits(B5)
    t0 = time.perf_counter()
    oracle.gemm(A5b, B5b, "f16", nthreads=1, lib=lib)
    t1 = time.perf_counter() - t0
    return dict(value=fl / t2 / 1e12, unit="TFLOPS", cores=oracle.threads(lib), kind="oracle",
                sample=f"{what} 4096^3 bf16 product (fp64 loop), {t2:.1f} s",
                cpu_model=cpu_model(),
                single_core_512_gflops=round(2 * 512 ** 3 / t1 / 1e9, 3))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def symbol_to_config(sym: str):
    """Configuration name of a gemm15 kernel symbol (None for other kernels)."""
    import re
    m = re.search(r"gemm_m16d_kernel<g15::(\w+)_t, (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)>", sym)
    if m:
        t, bm, bn, wm, wn, sa, kr, r = m.groups()
        return f"m16d_{t}_{bm}x{bn}x64_w{wm}x{wn}_a{sa}_b{kr}_r{r}"
    m = re.search(r"gemm_m16n_kernel<g15::(\w+)_t, (\d+), (\d+), (\d+), (\d+), (\d+), (\d+),"
                  r" (true|false)>", sym)
    if m:
        t, bm, bn, wm, wn, sa, sb, brow = m.groups()
        kind = "m16t" if brow == "true" else "m16n"
        return f"{kind}_{t}_{bm}x{bn}x64_w{wm}x{wn}_a{sa}_b{sb}"
    m = re.search(r"gemm_m16s_kernel<g15::(\w+)_t, (\d+), (\d+), (\d+), (\d+)"
                  r"(?:, (true|false))?(?:, (true|false))?>", sym)
    if m:
        t, bm, bn, wm, wn, brow, un = m.groups()
        return (f"m16s_{t}_{bm}x{bn}x64_w{wm}x{wn}" + ("_nk" if brow == "false" else "")
                + ("_u" if un == "true" else ""))
    m = re.search(r"gemm_m16w_kernel<g15::(\w+)_t, (\d+), (\d+), (\d+), (true|false)>", sym)
    if m:
        t, bm, bn, r, brow = m.groups()
        return f"m16w_{t}_{bm}x{bn}x32_r{r}" + ("" if brow == "true" else "_nk")
    m = re.search(r"gemm_f32d_kernel<(\d+), (\d+), (\d+), (\d+), (\d+)(?:, (true|false))?>", sym)
    if m:
        bm, bn, wm, wn, sa, bnk = m.groups()
        return f"f32d_{bm}x{bn}x16_w{wm}x{wn}_a{sa}" + ("_nk" if bnk == "true" else "")
    m = re.search(r"gemv_kernel<g15::(\w+)_t, (\d+), (\d+), (\d+)>", sym)
    if m:
        return f"gemv_{m.group(1)}_m{m.group(2)}"
    m = re.search(r"gemm_f32_kernel<(\d+), (\d+), (\d+), (\d+), (\w+), (\w+)>", sym)
    if m:
        bm, bn, wm, wn, va, vb = m.groups()
        return f"f32_{bm}x{bn}_w{wm}x{wn}" + ("" if va == "true" else "_scalar")
    return None


def summarize(db_dir: str, kind: str) -> None:
    """Print a text summary of rocprofv3 results under db_dir (kernel trace or
    FETCH_SIZE / WRITE_SIZE counters) and, for counters, update the traffic file."""
    import collections
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True)
    if kind == "trace":
        for db in dbs:
            d = sqlite3.connect(db)
            print(f"{'kernel':96s} {'calls':>6s} {'avg_us':>10s} {'pct':>6s}")
            for name, calls, tot, avg, pct in d.execute(
                    "select name, total_calls, total_duration, average, percentage from top_kernels"):
                print(f"{name[:96]:96s} {calls:6d} {avg:10.2f} {pct:6.2f}")
        return
    acc = collections.defaultdict(list)
    for db in dbs:
        d = sqlite3.connect(db)
        for name, cn, val in d.execute("select kernel_name, counter_name, value from counters_collection"):
            acc[(name, cn)].append(val)
    print(f"{'kernel':96s} {'counter':24s} {'n':>4s} {'per dispatch':>16s}")
    for (name, cn), v in sorted(acc.items()):
        print(f"{name[:96]:96s} {cn:24s} {len(v):4d} {sum(v) / len(v):16.1f}")
    # update the traffic file with the scale of each counter on the 256 MiB copy
    t = {"kernels": {}}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    # the calibration copies are the largest device copies of the run (inputs copied
    # from the host are smaller and read host memory)
    copy = {cn: max(v) for (name, cn), v in acc.items()
            if "copyBuffer" in name and cn in ("FETCH_SIZE", "WRITE_SIZE")}
    for cn, kib in copy.items():
        t.setdefault("scale", {})[cn] = 262144.0 / kib
    for (name, cn), v in acc.items():
        cfg = symbol_to_config(name)
        if cfg is None or cn not in ("FETCH_SIZE", "WRITE_SIZE"):
            continue
        row = t["kernels"].setdefault(cfg, {})
        row[cn + "_kib"] = sum(v) / len(v)
        row["source_hash"] = kernel_source_hash(cfg)
    sc = t.get("scale", {})
    for cfg, row in t["kernels"].items():
        if "FETCH_SIZE_kib" in row and "WRITE_SIZE_kib" in row and sc:
            row["traffic_bytes"] = round(row["FETCH_SIZE_kib"] * 1024 * sc.get("FETCH_SIZE", 1.0)
                                         + row["WRITE_SIZE_kib"] * 1024 * sc.get("WRITE_SIZE", 1.0))
    t.pop("source_hash", None)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1, sort_keys=True)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize":
        summarize(sys.argv[2], sys.argv[3])
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the product "
              "would shard by rows of A across GPUs, and only one GPU's share is measured",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import dense_gemm_15_amd as g

    print("[bench] bf16_4096", file=sys.stderr, flush=True)
    head = gemm_workload(g, "bf16_4096", args.steps, args.warmup)
    print(f"[bench] {json.dumps(head)}", file=sys.stderr, flush=True)
    print("[bench] fp32_4096", file=sys.stderr, flush=True)
    f32 = gemm_workload(g, "fp32_4096", args.steps, args.warmup)
    print(f"[bench] {json.dumps(f32)}", file=sys.stderr, flush=True)

    extra = {}
    if args.ladder:
        extra["ladder"] = ladder_workload(g, args.steps)
        print(f"[bench] ladder fp16-accumulation max abs diff "
              f"{extra['ladder']['fp16_accumulation_max_abs_diff']:.4g}", file=sys.stderr, flush=True)
    if args.vendor:
        extra["vendor_bf16_out"] = vendor_reference(g, args.steps, args.warmup)
        print(f"[bench] vendor {json.dumps(extra['vendor_bf16_out'])}", file=sys.stderr, flush=True)
    if args.attention and not args.all:
        extra["attention"] = attention_workload(g, args.steps, args.warmup)
        print(f"[bench] {json.dumps(extra['attention'])}", file=sys.stderr, flush=True)
    if args.copy_calibration:
        import torch as _t
        src = _t.empty(64 * 2**20, dtype=_t.float32, device="cuda")  # 256 MiB
        dst = _t.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        _t.cuda.synchronize()
        print("[bench] copy calibration: 3 x 256 MiB device copies", file=sys.stderr, flush=True)
    if args.all:
        for name in ("fp16_4096", "fp16_512", "gemv_1x4096x4096", "odd_127x1000x771",
                     "odd_4095x4097x63", "longk_256x256x4096", "longk_64x4096x4096"):
            extra[name] = gemm_workload(g, name, args.steps, args.warmup, graph=True)
            print(f"[bench] {json.dumps(extra[name])}", file=sys.stderr, flush=True)
        extra.update(ffn_workload(g, args.steps, args.warmup))
        print(f"[bench] ffn {json.dumps(extra['ffn1'])} {json.dumps(extra['ffn2'])}",
              file=sys.stderr, flush=True)
        extra["qk"] = qk_workload(g, args.steps, args.warmup)
        print(f"[bench] {json.dumps(extra['qk'])}", file=sys.stderr, flush=True)
        extra["attention"] = attention_workload(g, args.steps, args.warmup)
        print(f"[bench] {json.dumps(extra['attention'])}", file=sys.stderr, flush=True)
        # the same products with B stored transposed (weights [out, in], K as stored)
        extra["bf16_4096_nt"] = gemm_workload(g, "bf16_4096", args.steps, args.warmup,
                                              b_layout="nk")
        print(f"[bench] {json.dumps(extra['bf16_4096_nt'])}", file=sys.stderr, flush=True)
        extra.update(ffn_workload(g, args.steps, args.warmup, b_layout="nk"))
        print(f"[bench] ffn_nt {json.dumps(extra['ffn1_nt'])} {json.dumps(extra['ffn2_nt'])}",
              file=sys.stderr, flush=True)
        extra["qk_nt"] = qk_workload(g, args.steps, args.warmup, b_layout="nk")
        print(f"[bench] {json.dumps(extra['qk_nt'])}", file=sys.stderr, flush=True)

    configs = None
    if not args.no_configs:
        configs = baseline_configs(g, args.steps, args.warmup, head, f32)

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline()

    line = {
        "metric": "TFLOPS (2MNK/median time) at 4096^3 BF16 & FP32; % of gfx950 peak",
        "value": round(head["tflops"], 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": SETTLE_S,
        "ms_per_step": round(head["median_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "square GEMM M=N=K=4096, bf16 A and B ~U[-1,1), fp32 accumulate, "
                               "fp32 C", "M": 4096, "N": 4096, "K": 4096,
                   "kernel": head["config"]},
        "pct_of_peak": round(100 * head["tflops"] / PEAK_TFLOPS["bf16"], 2),
        "roofline": {"bound": "mfma", "achieved": round(head["tflops_mean"], 2),
                     "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                     "frac": round(head["frac_peak"], 4),
                     "traffic": measured_traffic(head["config"])},
        "fp32_sgemm_4096": {"value": round(f32["tflops"], 2), "unit": "TFLOPS",
                            "ms_per_call": round(f32["median_ms"], 5),
                            "kernel": f32["config"],
                            "pct_of_peak": round(100 * f32["tflops"] / PEAK_TFLOPS["f32"], 2),
                            "roofline": {"bound": "mfma", "achieved": round(f32["tflops_mean"], 2),
                                         "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                                         "frac": round(f32["frac_peak"], 4),
                                         "traffic": measured_traffic(f32["config"])}},
        "configs": configs,
        "cpu_baseline": cpu,
    }
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as f:
            json.dump(dict(headline=head, fp32=f32, extra=extra, cpu=cpu), f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
