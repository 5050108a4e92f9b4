"""Benchmark of the block-quantized decode GEMV on one MI355X.

Workload (one step): the 8B-class FFN-up projection 14336 x 4096 in GGUF
Q8_0 and in Q4_1; activations fp32 N(0,1), 5 rows (1 decode row + 4
speculative-verify rows).  A step quantizes the 5 activation rows to Q8_0 and
runs the GEMV over each weight format at batch 1 and at batch 5 (4 GEMVs).
Weights are resident in HBM before timing; every GEMV reads a different copy
of its weights (>= 512 MB of copies per format) so no launch is served from
the 256 MB Infinity Cache.

Printed: one JSON line.  value = weight bytes streamed per step / step time
(GB/s).  roofline: the Q8_0 batch-5 GEMV (the largest launch), algorithmic
bytes (weights + activation blocks + outputs) over its average launch
duration from HIP events on the launch stream around a burst of back-to-back
launches right after the timed steps; the average of events recorded around
its launch in every 10th timed step is reported beside it (those brackets
also hold the kernel-boundary time, about 3 us).  traffic: HBM bytes per launch
from the committed rocprofv3 counter summary, null once the GEMV source has
changed since it was taken.
cpu_baseline: the CPU oracle on the same step (fp64 reference, not a tuned
CPU kernel).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
GEMV_SOURCES = ("quantized_gguf_block_amd/csrc/gemv.hip", "quantized_gguf_block_amd/csrc/cq_device.h")


def gemv_source_sha():
    import hashlib
    m = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()


def profiled(kernel):
    """HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy of
    known size) and profiled average duration of `kernel`, from the summaries
    under profiles/ -- or None for each when the GEMV source has changed
    since they were taken."""
    sha = gemv_source_sha()
    traffic = prof_us = None
    try:
        with open(os.path.join(ROOT, "profiles", "gemv_ffn_up_hbm_traffic.md")) as fh:
            for line in fh:
                if line.strip().startswith("TRAFFIC "):
                    rec = json.loads(line.strip()[len("TRAFFIC "):])
                    if rec["kernel"] == kernel and rec["source_sha256"] == sha:
                        traffic = int(rec["traffic_bytes"])
        with open(os.path.join(ROOT, "profiles", "gemv_ffn_up_q8_0_q4_1_kernel_stats.md")) as fh:
            text = fh.read()
        if sha in text:
            for line in text.splitlines():
                if line.startswith("| " + kernel):
                    prof_us = float(line.split("|")[3])
    except (OSError, ValueError, KeyError):
        pass
    return traffic, prof_us


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the LM-head, prefill-GEMM and routed-FFN measurements")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gguf_synth as gs
    import quantized_gguf_block_amd as cq

    cq.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    n, k, B = 14336, 4096, 5
    fmts = [gs.Q8_0, gs.Q4_1]
    cfg_id = {gs.Q8_0: 1, gs.Q4_1: 11}
    host_w = {f: gs.weights(f, n, k, cfg=cfg_id[f]) for f in fmts}
    x = gs.activations(B, k, cfg=1)
    wbytes = {f: host_w[f].nbytes for f in fmts}
    copies = {}
    for f in fmts:
        base = torch.from_numpy(host_w[f]).to(dev)
        ncopy = max(2, -(-512 * 2**20 // wbytes[f]) + 1)
        copies[f] = [base] + [base.clone() for _ in range(ncopy - 1)]
    xd = torch.from_numpy(x).to(dev)
    xq = torch.empty((B, k // 32 * 34), dtype=torch.uint8, device=dev)
    y = torch.empty((B, n), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    counter = {f: 0 for f in fmts}
    ev_pairs = []

    def gemv(f, batch, record):
        w = copies[f][counter[f] % len(copies[f])]
        counter[f] += 1
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        cq.cq_gemv(f, w, n, k, xq, batch, y=y)
        if record:
            e1.record(stream)
            ev_pairs.append((e0, e1))

    def step(record=False):
        cq.cq_quantize_q8_0(xd, xq)
        gemv(gs.Q8_0, 1, False)
        gemv(gs.Q8_0, B, record)
        gemv(gs.Q4_1, 1, False)
        gemv(gs.Q4_1, B, False)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(record=(i % 10 == 0))  # bracketing events on every 10th step only
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    step_bytes = 2 * sum(wbytes.values())
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: Q8_0 batch-5 GEMV.  Two live HIP-event figures on the
    # launch stream: events around its launch in every 10th timed step (they
    # also hold the event packets and the dispatch/completion gap, ~3 us;
    # recording them on every step would add that gap to every step), and a
    # burst of back-to-back launches on rotating copies
    # right after the timed steps (per-launch duration without that gap,
    # the figure the profiler's kernel duration corresponds to).
    durs = [a.elapsed_time(b) for a, b in ev_pairs]
    avg_ms = float(np.mean(durs))
    reps = 100
    torch.cuda.synchronize()
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for _ in range(reps):
        gemv(gs.Q8_0, B, False)
    b1.record(stream)
    torch.cuda.synchronize()
    burst_ms = b0.elapsed_time(b1) / reps
    alg = wbytes[gs.Q8_0] + B * (k // 32 * 34) + B * n * 4
    achieved = alg / (burst_ms * 1e-3) / 1e9

    traffic, prof_us = profiled("gemv_stream_kernel<8, 5, 2, 4, false, false, 1>")

    extra = None if args.no_extra else secondary(cq, gs, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(host_w, x, n, k, B, args.cpu_seconds)

    out = {
        "metric": "decode GEMV weight GB/s (% HBM peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot4 + fp32 scale (Q8_0/Q4_1 weights, Q8_0 activations)",
        "data": "synthetic",
        "config": {"workload": "FFN-up decode GEMV 14336x4096, GGUF Q8_0 and Q4_1, "
                               "batch 1 and 5, activations quantized to Q8_0 each step",
                   "n": n, "k": k, "batches": [1, B], "formats": ["q8_0", "q4_1"],
                   "weight_copies": {gs.NAMES[f]: len(copies[f]) for f in fmts}},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "gemv_stream_kernel<8, 5, 2, 4, false, false, 1> (Q8_0, batch 5)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(burst_ms * 1e3, 3),
                     "avg_launch_us_event_bracketed": round(avg_ms * 1e3, 3),
                     "alg_bytes_per_launch": alg,
                     "traffic_over_alg": round(traffic / alg, 3) if traffic else None,
                     "rocprof_avg_kernel_us": prof_us},
        "cpu_baseline": cpu,
        "other_workloads": extra,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


MFMA_I8_PEAK_TOPS = 5030.0


def _burst_us(fn, reps, stream):
    """Average duration of `reps` back-to-back calls, HIP events on the
    launch stream around the whole burst."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _graph_us(fn, nsteps, reps, stream):
    """Average duration of one call of fn(i) with the launches captured in a
    HIP graph (fn(0) .. fn(nsteps-1) in one graph, replayed `reps` times
    between HIP events): the GPU time of launch-bound sequences without the
    Python call overhead."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nsteps):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsteps):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * nsteps) * 1e3


def secondary(cq, gs, dev, stream):
    """The other workloads, each timed as a burst of back-to-back launches
    (weights rotated through >= 512 MB of copies where they would fit the
    Infinity Cache): the 128K-vocabulary LM head (Q4_K, and Q6_K as for a
    tied embedding) at batch 1 and 4, the Q5_K FFN-up GEMV at batch 1 and 5,
    the fused Q4_K gate/up/SwiGLU GEMV against the separate kernels, the Q1_0
    10240 x 5120 matvec at batch 1 and 4,
    the 2048 x 2048 Q4_0 GEMV, the Q4_0 prefill GEMM at 512 and 2048 tokens,
    the Q5_K and Q6_K prefill GEMMs at 512 tokens, the greedy arg-max over
    the LM-head logits, the router, the whole routed FFN, and one decode
    token through the routed FFN (quantize, group, gate, up, SwiGLU + requantize,
    down, combine)."""
    import numpy as np
    import torch
    out = {}

    def copies(host, min_bytes=512 * 2**20):
        base = torch.from_numpy(host).to(dev)
        ncopy = max(2, -(-min_bytes // host.nbytes) + 1)
        return [base] + [base.clone() for _ in range(ncopy - 1)]

    # LM head, Q4_K and the tied-embedding Q6_K
    n, k = 128256, 4096
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(4, k, cfg=2)).to(dev))
    y = torch.empty((4, n), dtype=torch.float32, device=dev)
    for fmt, cfg in ((gs.Q4_K, 2), (gs.Q6_K, 22)):
        wl = copies(gs.weights(fmt, n, k, cfg=cfg))
        for b in (1, 4):
            us = _burst_us(lambda i: cq.cq_gemv(fmt, wl[i % len(wl)], n, k, xq, b, y=y), 50, stream)
            gbs = wl[0].numel() / us / 1e3
            out[f"{gs.NAMES[fmt]}_lm_head_128256x4096_b{b}"] = {
                "us": round(us, 2), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        del wl
    # greedy verify on the device: arg-max over the 128256 logits per row
    for b in (1, 4):
        ws = torch.empty(cq.load().cq_argmax_workspace_bytes(b, n), dtype=torch.uint8, device=dev)
        idx = torch.empty(b, dtype=torch.int32, device=dev)
        fn = (lambda i, b=b, idx=idx, ws=ws: cq.cq_argmax(y[:b], idx=idx, workspace=ws))
        us = _graph_us(fn, 8, 50, stream)
        out[f"argmax_128256_logits_b{b}"] = {"graph_us": round(us, 2),
                                             "python_burst_us": round(_burst_us(fn, 200, stream), 2),
                                             "GB/s": round(b * n * 4 / us / 1e3, 1)}
    # Q5_K FFN-up GEMV 14336 x 4096 (the FFN type of Q5_K_M models)
    n, k = 14336, 4096
    c5 = gs.CONFIGS["q5_k_gemv_ffn_up"]
    w5 = copies(gs.weights(gs.Q5_K, n, k, cfg=c5["cfg"]))
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(5, k, cfg=c5["cfg"])).to(dev))
    y = torch.empty((5, n), dtype=torch.float32, device=dev)
    for b in (1, 5):
        us = _burst_us(lambda i: cq.cq_gemv(gs.Q5_K, w5[i % len(w5)], n, k, xq, b, y=y), 100, stream)
        gbs = w5[0].numel() / us / 1e3
        out[f"q5_k_gemv_14336x4096_b{b}"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                             "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    del w5
    # FFN-down GEMV 4096 x 14336 (rows of 3.5 wave widths: the four waves of a
    # workgroup split k), Q8_0 and Q4_K, synthetic weights of those types
    n, k = 4096, 14336
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(5, k, cfg=16)).to(dev))
    y = torch.empty((5, n), dtype=torch.float32, device=dev)
    for fmt in (gs.Q8_0, gs.Q4_K):
        wd = copies(gs.weights(fmt, n, k, cfg=16))
        for b in (1, 5):
            # (in a graph: a Q4_K launch is shorter than a Python call)
            us = _graph_us(lambda i: cq.cq_gemv(fmt, wd[i % len(wd)], n, k, xq, b, y=y), 8, 50,
                           stream)
            gbs = wd[0].numel() / us / 1e3
            out[f"{gs.NAMES[fmt]}_gemv_4096x14336_b{b}"] = {
                "graph_us": round(us, 2), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        del wd
    # Q4_K rows of 1.25 and 2 wave widths (two-wave k-split streams): the
    # FFN-up 13824 x 5120 of 13B-class models, the gate 28672 x 8192 of
    # 70B-class models
    for n, k in ((13824, 5120), (28672, 8192)):
        xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(5, k, cfg=17)).to(dev))
        y = torch.empty((5, n), dtype=torch.float32, device=dev)
        wd = copies(gs.weights(gs.Q4_K, n, k, cfg=17))
        for b in (1, 5):
            us = _graph_us(lambda i: cq.cq_gemv(gs.Q4_K, wd[i % len(wd)], n, k, xq, b, y=y), 8, 50,
                           stream)
            gbs = wd[0].numel() / us / 1e3
            out[f"q4_k_gemv_{n}x{k}_b{b}"] = {
                "graph_us": round(us, 2), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        del wd
    n, k = 14336, 4096
    # decode FFN front half, Q4_K gate/up 14336 x 4096: fused gate + up +
    # SwiGLU GEMV then the Q8_0 of h, against two GEMVs and the SwiGLU +
    # requantization kernel (both produce the down GEMV's input)
    wgt = copies(gs.weights(gs.Q4_K, n, k, cfg=810, tensor=0), 256 * 2**20)
    wup = copies(gs.weights(gs.Q4_K, n, k, cfg=810, tensor=1), 256 * 2**20)
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(5, k, cfg=810)).to(dev))
    g = torch.empty((5, n), dtype=torch.float32, device=dev)
    u = torch.empty_like(g)
    h = torch.empty_like(g)
    hq = torch.empty((5, n // 32 * 34), dtype=torch.uint8, device=dev)
    for b in (1, 5):
        def fused(i, b=b):
            cq.cq_gemv_swiglu(gs.Q4_K, wgt[i % len(wgt)], wup[i % len(wup)], n, k, xq, b, h=h)
            cq.cq_quantize_q8_0(h[:b], hq[:b])

        def separate(i, b=b):
            cq.cq_gemv(gs.Q4_K, wgt[i % len(wgt)], n, k, xq, b, y=g)
            cq.cq_gemv(gs.Q4_K, wup[i % len(wup)], n, k, xq, b, y=u)
            cq.cq_swiglu_quantize_q8_0(g[:b], u[:b], hq=hq[:b])

        ns = min(len(wgt), len(wup))
        us_f = _graph_us(fused, ns, 20, stream)
        us_s = _graph_us(separate, ns, 20, stream)
        wb = 2 * wgt[0].numel()
        out[f"q4_k_ffn_gate_up_swiglu_14336x4096_b{b}"] = {
            "fused_graph_us": round(us_f, 2), "separate_graph_us": round(us_s, 2),
            "fused_python_burst_us": round(_burst_us(fused, 100, stream), 2),
            "fused_weight_GB/s": round(wb / us_f / 1e3, 1),
            "fused_pct_hbm_peak": round(100 * wb / us_f / 1e3 / HBM_PEAK_GBS, 1)}
    del wgt, wup
    # Q1_0 attention QKV matvec 10240 x 5120 (the pages' Q1_0 micro-benchmark
    # shape, 5.9 MB of weights), batch 1 and 4, weights rotated through copies
    c1 = gs.CONFIGS["q1_0_gemv_qkv"]
    n1, k1 = c1["n"], c1["k"]
    w1 = copies(gs.weights(gs.Q1_0, n1, k1, cfg=c1["cfg"]), 256 * 2**20)
    xq1 = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(4, k1, cfg=c1["cfg"])).to(dev))
    y1q = torch.empty((4, n1), dtype=torch.float32, device=dev)
    for b in (1, 4):
        fn = (lambda i, b=b: cq.cq_gemv(gs.Q1_0, w1[i % len(w1)], n1, k1, xq1, b, y=y1q))
        us = _graph_us(fn, len(w1), 5, stream)
        gbs = w1[0].numel() / us / 1e3
        out[f"q1_0_gemv_10240x5120_b{b}"] = {"graph_us": round(us, 2), "GB/s": round(gbs, 1),
                                             "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    del w1
    # 2048 x 2048 Q4_0 GEMV (2.36 MB per call: launch-latency bound)
    n, k = 2048, 2048
    w0 = copies(gs.weights(gs.Q4_0, n, k, cfg=0))
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(1, k, cfg=0)).to(dev))
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    us = _burst_us(lambda i: cq.cq_gemv(gs.Q4_0, w0[i % len(w0)], n, k, xq, 1, y=y), 400, stream)
    gbs = w0[0].numel() / us / 1e3
    out["q4_0_gemv_2048x2048_b1"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                     "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    del w0
    # prefill GEMM
    n, k = 14336, 4096
    wg = torch.from_numpy(gs.weights(gs.Q4_0, n, k, cfg=3)).to(dev)
    for m in (512, 2048):
        xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(m, k, cfg=3)).to(dev))
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        us = _burst_us(lambda i: cq.cq_gemm(gs.Q4_0, wg, n, k, xq, m, y=y), 20, stream)
        tops = 2 * m * n * k / us / 1e6
        out[f"q4_0_gemm_{m}x14336x4096"] = {"us": round(us, 2), "TOPS": round(tops, 1),
                                            "pct_int8_mfma_peak": round(100 * tops / MFMA_I8_PEAK_TOPS, 2)}
    del wg
    for fmt, name in ((gs.Q5_K, "q5_k_gemm_prefill_512"), (gs.Q6_K, "q6_k_gemm_prefill_512")):
        c5 = gs.CONFIGS[name]
        wg = torch.from_numpy(gs.weights(fmt, n, k, cfg=c5["cfg"])).to(dev)
        m = c5["m"]
        xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(m, k, cfg=c5["cfg"])).to(dev))
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        us = _burst_us(lambda i: cq.cq_gemm(fmt, wg, n, k, xq, m, y=y), 20, stream)
        tops = 2 * m * n * k / us / 1e6
        out[f"{gs.NAMES[fmt]}_gemm_{m}x14336x4096"] = {
            "us": round(us, 2), "TOPS": round(tops, 1),
            "pct_int8_mfma_peak": round(100 * tops / MFMA_I8_PEAK_TOPS, 2)}
        del wg
    # routed FFN
    c = gs.CONFIGS["q4_k_moe_ffn"]
    T, H, F, E, K = c["n_tokens"], c["hidden"], c["ffn"], c["n_experts"], c["top_k"]
    mats = [gs.expert_weights(gs.Q4_K, E, F, H, 4, 0), gs.expert_weights(gs.Q4_K, E, F, H, 4, 1),
            gs.expert_weights(gs.Q4_K, E, H, F, 4, 2)]
    wbytes = sum(m_.nbytes for m_ in mats)
    sets = [[torch.from_numpy(m_).to(dev) for m_ in mats]]
    while len(sets) * wbytes < 512 * 2**20 + wbytes:
        sets.append([t.clone() for t in sets[0]])
    x = torch.from_numpy(gs.activations(T, H, 4)).to(dev)
    ids, rw = gs.routing(T, E, K, 4)
    ids, rw = torch.from_numpy(ids).to(dev), torch.from_numpy(rw).to(dev)
    xq = torch.empty((T, H // 32 * 34), dtype=torch.uint8, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pairs = torch.empty(T * K, dtype=torch.int32, device=dev)
    gst = torch.zeros(1, dtype=torch.int32, device=dev)
    g = torch.empty((T * K, F), dtype=torch.float32, device=dev)
    u = torch.empty_like(g)
    hq = torch.empty((T * K, F // 32 * 34), dtype=torch.uint8, device=dev)
    d = torch.empty((T * K, H), dtype=torch.float32, device=dev)
    yt = torch.empty((T, H), dtype=torch.float32, device=dev)

    def ffn(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x, xq)
        cq.cq_moe_group(ids, E, offs, pairs, gst)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wg_, E, F, H, xq, False, offs, pairs, T, K, y=g)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wu_, E, F, H, xq, False, offs, pairs, T, K, y=u)
        cq.cq_swiglu_quantize_q8_0(g, u, hq=hq)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wd_, E, H, F, hq, True, offs, pairs, T, K, y=d)
        cq.cq_moe_combine(d, rw, y=yt)

    us = _burst_us(ffn, 50, stream)

    # router: top 4 of 32 with softmax, 256 tokens
    lg = torch.from_numpy(np.random.default_rng(5).standard_normal((T, E)).astype(np.float32)).to(dev)
    rid = torch.empty((T, K), dtype=torch.int32, device=dev)
    rwt = torch.empty((T, K), dtype=torch.float32, device=dev)
    rfn = (lambda i: cq.cq_topk_softmax(lg, K, ids=rid, w=rwt))
    out["router_top4_of_32_256tok"] = {"graph_us": round(_graph_us(rfn, 8, 50, stream), 2),
                                       "python_burst_us": round(_burst_us(rfn, 200, stream), 2)}
    # decode: one token, top 4, the whole FFN through the per-pair GEMV path
    # (no grouping call) against the grouped path on the same token
    ids1, rw1 = gs.routing(1, E, K, 850)
    ids1, rw1 = torch.from_numpy(ids1).to(dev), torch.from_numpy(rw1).to(dev)
    x1 = torch.from_numpy(gs.activations(1, H, 850)).to(dev)
    h1 = torch.empty((K, F), dtype=torch.float32, device=dev)
    hq1 = torch.empty((K, F // 32 * 34), dtype=torch.uint8, device=dev)
    d1 = torch.empty((K, H), dtype=torch.float32, device=dev)
    y1 = torch.empty((1, H), dtype=torch.float32, device=dev)

    def ffn_decode(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x1, xq[:1])
        cq.cq_moe_gemv_swiglu(gs.Q4_K, wg_, wu_, E, F, H, xq[:1], ids1, h=h1, status=gst)
        cq.cq_quantize_q8_0(h1, hq1)
        cq.cq_moe_gemv(gs.Q4_K, wd_, E, H, F, hq1, True, ids1, y=d1, status=gst)
        cq.cq_moe_combine(d1, rw1, y=y1)

    def ffn_decode_grouped(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x1, xq[:1])
        cq.cq_moe_group(ids1, E, offs, pairs[:K], gst)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wg_, E, F, H, xq[:1], False, offs, pairs[:K], 1, K, y=g[:K])
        cq.cq_moe_gemm_grouped(gs.Q4_K, wu_, E, F, H, xq[:1], False, offs, pairs[:K], 1, K, y=u[:K])
        cq.cq_swiglu_quantize_q8_0(g[:K], u[:K], hq=hq1)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wd_, E, H, F, hq1, True, offs, pairs[:K], 1, K, y=d1)
        cq.cq_moe_combine(d1, rw1, y=y1)

    us_dec = _graph_us(ffn_decode, len(sets), 20, stream)
    us_dec_g = _graph_us(ffn_decode_grouped, len(sets), 20, stream)
    wdec = K * sum(m_.nbytes for m_ in mats) // E
    out["q4_k_moe_ffn_decode_1tok_top4"] = {
        "graph_us": round(us_dec, 2), "grouped_path_graph_us": round(us_dec_g, 2),
        "python_burst_us": round(_burst_us(ffn_decode, 100, stream), 2),
        "expert_weight_GB/s": round(wdec / us_dec / 1e3, 1)}
    ops = 2 * T * K * (2 * F * H + H * F)
    out["q4_k_moe_ffn_256tok_32x_top4"] = {
        "us": round(us, 2), "expert_weight_GB/s": round(wbytes / us / 1e3, 1),
        "pct_hbm_peak": round(100 * wbytes / us / 1e3 / HBM_PEAK_GBS, 1),
        "int8_TOPS": round(ops / us / 1e6, 1),
        "pct_int8_mfma_peak": round(100 * ops / us / 1e6 / MFMA_I8_PEAK_TOPS, 2)}
    return out


def cpu_baseline(host_w, x, n, k, B, seconds):
    """The CPU oracle on the same step (quantize + the four GEMVs), repeated
    for about `seconds`; GB/s of weights streamed."""
    import oracle
    import gguf_synth as gs
    threads = oracle.default_threads()
    steps = 0
    t0 = time.perf_counter()
    while True:
        xq = oracle.quantize_q8_0(x)
        for f in (gs.Q8_0, gs.Q4_1):
            oracle.matmul(f, host_w[f], n, k, xq[:1], 1, n_threads=threads, want_s=False)
            oracle.matmul(f, host_w[f], n, k, xq, B, n_threads=threads, want_s=False)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    step_bytes = 2 * sum(w.nbytes for w in host_w.values())
    return {"value": round(step_bytes * steps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full steps (quantize + Q8_0/Q4_1 GEMV at batch 1 and 5), "
                      f"{el:.1f} s, fp64 oracle with {threads} threads"}


if __name__ == "__main__":
    main()
