"""Benchmark of the block-quantized GGUF matmul on one MI355X.

Headline step: the 128K-vocabulary LM head, 128256 x 4096 in GGUF Q4_K (the
largest decode GEMV of the workloads), with 4 activation rows of fp32
N(0,1) (1 decode row + 3 speculative-verify rows).  A step quantizes the 4
rows to Q8_0 and runs the GEMV at batch 1 (decode) and at batch 4 (the
batched verify).  Weights are resident in HBM before timing; each GEMV reads
a different copy of the weights (3 copies, 887 MB) so no launch is served
from the 256 MB Infinity Cache.

Printed: one JSON line.
  value      weight bytes streamed per step / step time (GB/s).
  roofline   the batch-4 GEMV, the longest kernel of the step: algorithmic
             bytes (weights + Q8_0 activations + fp32 logits) over its average
             launch duration, from HIP events on the launch stream around a
             burst of back-to-back launches right after the timed steps.
             traffic: HBM bytes per launch from the committed rocprofv3
             counter summary (FETCH_SIZE, WRITE_SIZE scaled by a plain copy),
             null once the GEMV source has changed since it was taken.
  gemm       the prefill GEMM (Q4_0, 14336 x 4096) at 2048 and 512 tokens,
             weights rotated through copies, in int8 TOPS; its roofline
             against the int8 MFMA peak (each launch between its own pair of
             HIP events), with the MFMA-busy fraction from the
             committed counter summary (null once the GEMM source changed).
  cpu_baseline  the CPU oracle (fp64, plain C++) on the same step, on all
             the cores this process may use and on one core.
  other_workloads  the remaining workloads: the 2048 x 2048 Q4_0 GEMV
             (per-launch duration and steady state over 256 distinct
             matrices in a HIP graph), the FFN-up GEMVs (Q8_0, Q4_1, Q5_K),
             the Q6_K LM head, the Q5_K / Q6_K prefill GEMMs, the routed FFN,
             and the decode-side kernels (fused FFN front half, arg-max,
             router, one routed decode token).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_I8_PEAK_TOPS = 5030.0
CSRC = "quantized_gguf_block_amd/csrc/"
GEMV_SOURCES = (CSRC + "gemv.hip", CSRC + "gemv_mfma.hip", CSRC + "cq_device.h")
GEMM_SOURCES = (CSRC + "gemm.hip", CSRC + "cq_device.h")


def source_sha(files):
    m = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            m.update(fh.read())
    return m.hexdigest()


def profile_record(fname, tag, kernel, sha):
    """The JSON record `tag {...}` for `kernel` in profiles/fname, if it was
    taken on sources with hash `sha`; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as fh:
            for line in fh:
                line = line.strip()
                if line.startswith(tag + " "):
                    rec = json.loads(line[len(tag) + 1:])
                    if rec.get("kernel") == kernel and rec.get("source_sha256") == sha:
                        return rec
    except (OSError, ValueError):
        pass
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-gemm", action="store_true", help="skip the prefill GEMM line")
    ap.add_argument("--no-extra", action="store_true", help="skip other_workloads")
    return ap.parse_args()


def events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def burst_us(fn, reps, stream, warm=3):
    """Average duration of `reps` back-to-back calls fn(i), HIP events on the
    launch stream around the whole burst."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = events()
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def graph_us(fn, nsteps, reps, stream):
    """Average duration of one call fn(i) with fn(0) .. fn(nsteps-1) captured
    in one HIP graph and replayed `reps` times between HIP events: the GPU
    time of launch-bound sequences without the Python call overhead."""
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
    e0, e1 = events()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * nsteps) * 1e3


def copies_of(host, dev, min_bytes, min_copies=2):
    import torch
    base = torch.from_numpy(host).to(dev)
    ncopy = max(min_copies, -(-min_bytes // host.nbytes))
    return [base] + [base.clone() for _ in range(ncopy - 1)]


def lm_head_kernel(batch):
    return f"gemv_q4k_mfma_kernel<{batch}>"


def gemm_kernel_name():
    return "gemm2_kernel<2>"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import gguf_synth as gs
    import quantized_gguf_block_amd as cq

    cq.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    c = gs.CONFIGS["q4_k_gemv_lm_head"]
    fmt, n, k, B = c["fmt"], c["n"], c["k"], max(c["batches"])
    host_w = gs.weights(fmt, n, k, cfg=c["cfg"])
    x = gs.activations(B, k, cfg=c["cfg"])
    wbytes = host_w.nbytes
    wl = copies_of(host_w, dev, 768 * 2**20, 3)
    xd = torch.from_numpy(x).to(dev)
    xq = torch.empty((B, k // 32 * 34), dtype=torch.uint8, device=dev)
    y = torch.empty((B, n), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    counter = [0]

    def gemv(batch):
        w = wl[counter[0] % len(wl)]
        counter[0] += 1
        cq.cq_gemv(fmt, w, n, k, xq, batch, y=y)

    def step():
        cq.cq_quantize_q8_0(xd, xq)
        gemv(1)
        gemv(B)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = events()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    value = 2 * wbytes / (ms_step * 1e-3) / 1e9

    # dominant kernel: the batch-4 GEMV, right after the timed steps, as a
    # burst of back-to-back launches on the rotating copies between two HIP
    # events on the launch stream (an event pair around every launch would
    # add the event packets' own few microseconds to each); the batch-1 GEMV
    # and the quantizer beside it
    us_b4 = burst_us(lambda i: gemv(B), 60, stream)
    us_b1 = burst_us(lambda i: gemv(1), 60, stream)
    us_q = graph_us(lambda i: cq.cq_quantize_q8_0(xd, xq), 50, 10, stream)
    alg = {b: wbytes + b * (k // 32 * 34) + b * n * 4 for b in (1, B)}
    achieved = alg[B] / (us_b4 * 1e-6) / 1e9
    gsha = source_sha(GEMV_SOURCES)
    tr = profile_record("lm_head_q4_k_hbm_traffic.md", "TRAFFIC", lm_head_kernel(B), gsha)
    kt = profile_record("lm_head_q4_k_gemv_kernel_stats.md", "KTRACE", lm_head_kernel(B), gsha)
    traffic = tr["traffic_bytes"] if tr else None
    del wl
    torch.cuda.empty_cache()

    gemm = None if args.no_gemm else prefill_gemm(cq, gs, dev, stream)
    extra = None if args.no_extra else secondary(cq, gs, dev, stream)
    cpu = None if args.no_cpu_baseline else cpu_baseline(host_w, x, n, k, B, args.cpu_seconds)

    out = {
        "metric": "decode GEMV weight GB/s (% HBM peak); prefill GEMM int8 TOPS (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 MFMA dots + fp32 scale (Q4_K weights, Q8_0 activations)",
        "data": "synthetic",
        "config": {"workload": "LM-head decode GEMV 128256x4096, GGUF Q4_K, batch 1 (decode) and "
                               "batch 4 (speculative verify), the 4 activation rows quantized to "
                               "Q8_0 each step",
                   "n": n, "k": k, "batches": [1, B], "format": "q4_k", "weight_copies": 3},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": lm_head_kernel(B) + " (Q4_K LM head, batch 4)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(us_b4, 3),
                     "alg_bytes_per_launch": alg[B],
                     "traffic_over_alg": round(traffic / alg[B], 4) if traffic else None,
                     "rocprof_avg_kernel_us": kt["avg_us"] if kt else None,
                     "rocprof_timed_steps_avg_us": kt.get("timed_steps_avg_us") if kt else None},
        "step_kernels_us": {"quantize_4_rows": round(us_q, 2),
                            "gemv_b1": round(us_b1, 2), "gemv_b4": round(us_b4, 2),
                            "gemv_b1_GB/s": round(alg[1] / us_b1 / 1e3, 1),
                            "gemv_b1_pct_hbm_peak": round(100 * alg[1] / us_b1 / 1e3 / HBM_PEAK_GBS, 1)},
        "gemm": gemm,
        "cpu_baseline": cpu,
        "other_workloads": extra,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


def prefill_gemm(cq, gs, dev, stream):
    """Q4_0 prefill GEMM 14336 x 4096 at 2048 and 512 tokens: weights rotated
    through copies (>= 512 MB), activations quantized once; int8 TOPS from
    HIP events around bursts of back-to-back launches after a warm-up."""
    import torch
    out = {}
    res = {}
    for name in ("q4_0_gemm_prefill_2048", "q4_0_gemm_prefill_512"):
        c = gs.CONFIGS[name]
        n, k, m = c["n"], c["k"], c["m"]
        wl = copies_of(gs.weights(c["fmt"], n, k, cfg=c["cfg"]), dev, 512 * 2**20)
        xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(m, k, cfg=c["cfg"])).to(dev))
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        # ~12 ms of untimed launches first (as for the GEMV steps: the first
        # milliseconds of sustained load after lighter work run slower), then
        # a burst of back-to-back launches between two HIP events (an event
        # pair around each launch would add the packets' own ~5 us to each)
        us = burst_us(lambda i: cq.cq_gemm(c["fmt"], wl[i % len(wl)], n, k, xq, m, y=y),
                      40 if m == 2048 else 100, stream, warm=30 if m == 2048 else 120)
        tops = 2 * m * n * k / us / 1e6
        res[m] = (us, tops)
        out[f"q4_0_gemm_{m}x{n}x{k}"] = {"us": round(us, 2), "TOPS": round(tops, 1),
                                         "pct_int8_mfma_peak": round(100 * tops / MFMA_I8_PEAK_TOPS, 2),
                                         "weight_copies": len(wl)}
        del wl, y
    us, tops = res[2048]
    sha = source_sha(GEMM_SOURCES)
    pmc = profile_record("prefill_gemm_q4_0_mfma_counters.md", "MFMA", gemm_kernel_name(), sha)
    out["roofline"] = {"bound": "mfma", "kernel": gemm_kernel_name() + " (Q4_0, 2048 tokens)",
                       "achieved": round(tops, 1), "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s (int8)",
                       "frac": round(tops / MFMA_I8_PEAK_TOPS, 4),
                       "avg_launch_us": round(us, 2),
                       "ops_per_launch": 2 * 2048 * 14336 * 4096,
                       "mfma_busy": pmc.get("mfma_busy") if pmc else None,
                       "traffic": pmc.get("traffic_bytes") if pmc else None}
    torch.cuda.empty_cache()
    return out


def secondary(cq, gs, dev, stream):
    """The other workloads (weights rotated through >= 512 MB of copies where
    one copy would fit the Infinity Cache)."""
    import numpy as np
    import torch
    out = {}

    # 2048 x 2048 Q4_0 GEMV (2.36 MB per call): the per-launch duration of a
    # burst issued from Python, and the steady state over 256 distinct
    # matrices (604 MB) launched back to back from a HIP graph
    c = gs.CONFIGS["q4_0_gemv_2048"]
    n, k = c["n"], c["k"]
    host = gs.weights(gs.Q4_0, n, k, cfg=c["cfg"])
    big = torch.from_numpy(host).to(dev).repeat(256, 1)        # 256 copies, one tensor
    mats = [big[i * n:(i + 1) * n] for i in range(256)]
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(1, k, cfg=c["cfg"])).to(dev))
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    fn = (lambda i: cq.cq_gemv(gs.Q4_0, mats[i % 256], n, k, xq, 1, y=y))
    us_g = graph_us(fn, 256, 5, stream)
    us_b = burst_us(fn, 512, stream)
    out["q4_0_gemv_2048x2048_b1"] = {
        "graph_256_matrices_us_per_launch": round(us_g, 3),
        "graph_GB/s": round(host.nbytes / us_g / 1e3, 1),
        "graph_pct_hbm_peak": round(100 * host.nbytes / us_g / 1e3 / HBM_PEAK_GBS, 1),
        "python_burst_us": round(us_b, 2)}
    del big, mats

    # FFN-up decode GEMVs 14336 x 4096: Q8_0 and Q4_1 at batch 1 and 5, Q5_K;
    # the Q1_0 27B QKV projection 10240 x 5120 and the 2-bit ternary 70B gate
    # projection 28672 x 8192 at batch 1 and 4
    for name in ("q8_0_gemv_ffn_up", "q4_1_gemv_ffn_up", "q5_k_gemv_ffn_up", "q1_0_gemv_qkv",
                 "tq2_gemv_70b_gate"):
        c = gs.CONFIGS[name]
        n, k = c["n"], c["k"]
        wl = copies_of(gs.weights(c["fmt"], n, k, cfg=c["cfg"]), dev, 512 * 2**20)
        xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(5, k, cfg=c["cfg"])).to(dev))
        y = torch.empty((5, n), dtype=torch.float32, device=dev)
        for b in c["batches"]:
            us = graph_us(lambda i: cq.cq_gemv(c["fmt"], wl[i % len(wl)], n, k, xq, b, y=y),
                          len(wl), 10, stream)
            gbs = wl[0].numel() / us / 1e3
            out[f"{gs.NAMES[c['fmt']]}_gemv_{n}x{k}_b{b}"] = {
                "graph_us": round(us, 2), "GB/s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
        del wl

    # the tied-embedding LM head in Q6_K
    c = gs.CONFIGS["q6_k_gemv_lm_head"]
    n, k = c["n"], c["k"]
    wl = copies_of(gs.weights(gs.Q6_K, n, k, cfg=c["cfg"]), dev, 768 * 2**20)
    xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(4, k, cfg=c["cfg"])).to(dev))
    y = torch.empty((4, n), dtype=torch.float32, device=dev)
    for b in (1, 4):
        # ~8 ms of warm-up launches first: the first milliseconds of a sustained
        # burst after lighter work run slower (the batch-4 launches up to 30 %)
        us = burst_us(lambda i: cq.cq_gemv(gs.Q6_K, wl[i % len(wl)], n, k, xq, b, y=y), 40, stream,
                      warm=100)
        gbs = wl[0].numel() / us / 1e3
        out[f"q6_k_lm_head_{n}x{k}_b{b}"] = {"us": round(us, 2), "GB/s": round(gbs, 1),
                                             "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    del wl
    # greedy verify on the device: arg-max over the 128256 logits per row
    for b in (1, 4):
        ws = torch.empty(cq.load().cq_argmax_workspace_bytes(b, n), dtype=torch.uint8, device=dev)
        idx = torch.empty(b, dtype=torch.int32, device=dev)
        fn = (lambda i, b=b, idx=idx, ws=ws: cq.cq_argmax(y[:b], idx=idx, workspace=ws))
        us = graph_us(fn, 8, 50, stream)
        out[f"argmax_128256_logits_b{b}"] = {"graph_us": round(us, 2),
                                             "GB/s": round(b * n * 4 / us / 1e3, 1)}
    torch.cuda.empty_cache()

    # Q5_K and Q6_K prefill GEMMs at 512 tokens
    for name in ("q5_k_gemm_prefill_512", "q6_k_gemm_prefill_512"):
        c = gs.CONFIGS[name]
        n, k, m = c["n"], c["k"], c["m"]
        wl = copies_of(gs.weights(c["fmt"], n, k, cfg=c["cfg"]), dev, 512 * 2**20)
        xq = cq.cq_quantize_q8_0(torch.from_numpy(gs.activations(m, k, cfg=c["cfg"])).to(dev))
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        us = burst_us(lambda i: cq.cq_gemm(c["fmt"], wl[i % len(wl)], n, k, xq, m, y=y), 40, stream,
                      warm=60)
        tops = 2 * m * n * k / us / 1e6
        out[f"{gs.NAMES[c['fmt']]}_gemm_{m}x{n}x{k}"] = {
            "us": round(us, 2), "TOPS": round(tops, 1),
            "pct_int8_mfma_peak": round(100 * tops / MFMA_I8_PEAK_TOPS, 2)}
        del wl

    # decode FFN front half, Q4_K gate/up 14336 x 4096: fused gate + up +
    # SwiGLU GEMV then the Q8_0 of h, against two GEMVs and the SwiGLU +
    # requantization kernel
    n, k = 14336, 4096
    wgt = copies_of(gs.weights(gs.Q4_K, n, k, cfg=810, tensor=0), dev, 256 * 2**20)
    wup = copies_of(gs.weights(gs.Q4_K, n, k, cfg=810, tensor=1), dev, 256 * 2**20)
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
        us_f = graph_us(fused, ns, 10, stream)
        us_s = graph_us(separate, ns, 10, stream)
        wb = 2 * wgt[0].numel()
        out[f"q4_k_ffn_gate_up_swiglu_14336x4096_b{b}"] = {
            "fused_graph_us": round(us_f, 2), "separate_graph_us": round(us_s, 2),
            "fused_weight_GB/s": round(wb / us_f / 1e3, 1),
            "fused_pct_hbm_peak": round(100 * wb / us_f / 1e3 / HBM_PEAK_GBS, 1)}
    del wgt, wup

    # routed FFN (lfm2moe shape) through the one-call routed projection
    # (grouping + grouped GEMM + combine on a caller workspace)
    c = gs.CONFIGS["q4_k_moe_ffn"]
    T, H, F, E, K = c["n_tokens"], c["hidden"], c["ffn"], c["n_experts"], c["top_k"]
    mats = [gs.expert_weights(gs.Q4_K, E, F, H, c["cfg"], 0),
            gs.expert_weights(gs.Q4_K, E, F, H, c["cfg"], 1),
            gs.expert_weights(gs.Q4_K, E, H, F, c["cfg"], 2)]
    wbytes = sum(m_.nbytes for m_ in mats)
    sets = [[torch.from_numpy(m_).to(dev) for m_ in mats]]
    while len(sets) * wbytes < 512 * 2**20 + wbytes:
        sets.append([t.clone() for t in sets[0]])
    x = torch.from_numpy(gs.activations(T, H, c["cfg"])).to(dev)
    ids, rw = gs.routing(T, E, K, c["cfg"])
    ids, rw = torch.from_numpy(ids).to(dev), torch.from_numpy(rw).to(dev)
    xq = torch.empty((T, H // 32 * 34), dtype=torch.uint8, device=dev)
    g = torch.empty((T * K, F), dtype=torch.float32, device=dev)
    u = torch.empty_like(g)
    hq = torch.empty((T * K, F // 32 * 34), dtype=torch.uint8, device=dev)
    yt = torch.empty((T, H), dtype=torch.float32, device=dev)
    f_gu = cq.MOE_X_PER_TOKEN | cq.MOE_OUT_PER_PAIR
    f_dn = cq.MOE_X_PER_PAIR | cq.MOE_OUT_COMBINE
    ws = torch.empty(max(cq.cq_moe_workspace_bytes(T, K, E, F, f_gu),
                         cq.cq_moe_workspace_bytes(T, K, E, H, f_dn)), dtype=torch.uint8, device=dev)

    def ffn(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x, xq)
        cq.cq_moe_gemm(gs.Q4_K, wg_, E, F, H, xq, f_gu, ids, y=g, workspace=ws)
        cq.cq_moe_gemm(gs.Q4_K, wu_, E, F, H, xq, f_gu, ids, y=u, workspace=ws)
        cq.cq_swiglu_quantize_q8_0(g, u, hq=hq)
        cq.cq_moe_gemm(gs.Q4_K, wd_, E, H, F, hq, f_dn, ids, route_w=rw, y=yt, workspace=ws)

    us = graph_us(ffn, len(sets), 10, stream)

    # the same FFN with the grouping computed once and shared by the three
    # projections (split form; gate and up in one call over one split of each
    # expert's rows), D per pair, then the slot-order combine
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    prs = torch.empty(T * K, dtype=torch.int32, device=dev)
    gst = torch.empty(1, dtype=torch.int32, device=dev)
    dpp = torch.empty((T * K, H), dtype=torch.float32, device=dev)

    def ffn_grouped(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x, xq)
        cq.cq_moe_group(ids, E, offsets=offs, pairs=prs, status=gst)
        cq.cq_moe_gemm_grouped2(gs.Q4_K, wg_, wu_, E, F, H, xq, False, offs, prs, T, K, y_a=g, y_b=u)
        cq.cq_swiglu_quantize_q8_0(g, u, hq=hq)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wd_, E, H, F, hq, True, offs, prs, T, K, y=dpp)
        cq.cq_moe_combine(dpp, rw, y=yt)

    def ffn_grouped_separate(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x, xq)
        cq.cq_moe_group(ids, E, offsets=offs, pairs=prs, status=gst)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wg_, E, F, H, xq, False, offs, prs, T, K, y=g)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wu_, E, F, H, xq, False, offs, prs, T, K, y=u)
        cq.cq_swiglu_quantize_q8_0(g, u, hq=hq)
        cq.cq_moe_gemm_grouped(gs.Q4_K, wd_, E, H, F, hq, True, offs, prs, T, K, y=dpp)
        cq.cq_moe_combine(dpp, rw, y=yt)

    us_g = graph_us(ffn_grouped, len(sets), 10, stream)
    us_gs = graph_us(ffn_grouped_separate, len(sets), 10, stream)
    ops = 2 * T * K * (2 * F * H + H * F)
    out["q4_k_moe_ffn_256tok_32x_top4"] = {
        "graph_us": round(us_g, 2), "expert_weight_GB/s": round(wbytes / us_g / 1e3, 1),
        "pct_hbm_peak": round(100 * wbytes / us_g / 1e3 / HBM_PEAK_GBS, 1),
        "int8_TOPS": round(ops / us_g / 1e6, 1),
        "pct_int8_mfma_peak": round(100 * ops / us_g / 1e6 / MFMA_I8_PEAK_TOPS, 2),
        "sequence": "quantize, group once, gate+up in one call, SwiGLU+requant, down, combine",
        "gate_and_up_separate_calls_graph_us": round(us_gs, 2),
        "one_call_per_projection_graph_us": round(us, 2),
        "weight_sets": len(sets)}

    # router: top 4 of 32 with softmax, 256 tokens
    lg = torch.from_numpy(np.random.default_rng(5).standard_normal((T, E)).astype(np.float32)).to(dev)
    rid = torch.empty((T, K), dtype=torch.int32, device=dev)
    rwt = torch.empty((T, K), dtype=torch.float32, device=dev)
    out["router_top4_of_32_256tok"] = {
        "graph_us": round(graph_us(lambda i: cq.cq_topk_softmax(lg, K, ids=rid, w=rwt), 8, 50,
                                   stream), 2)}
    # decode: one token, top 4, the whole FFN through the per-pair GEMV path
    ids1, rw1 = gs.routing(1, E, K, 850)
    ids1, rw1 = torch.from_numpy(ids1).to(dev), torch.from_numpy(rw1).to(dev)
    x1 = torch.from_numpy(gs.activations(1, H, 850)).to(dev)
    h1 = torch.empty((K, F), dtype=torch.float32, device=dev)
    hq1 = torch.empty((K, F // 32 * 34), dtype=torch.uint8, device=dev)
    d1 = torch.empty((K, H), dtype=torch.float32, device=dev)
    y1 = torch.empty((1, H), dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)

    def ffn_decode(i):
        wg_, wu_, wd_ = sets[i % len(sets)]
        cq.cq_quantize_q8_0(x1, xq[:1])
        cq.cq_moe_gemv_swiglu(gs.Q4_K, wg_, wu_, E, F, H, xq[:1], ids1, h=h1, status=st)
        cq.cq_quantize_q8_0(h1, hq1)
        cq.cq_moe_gemv(gs.Q4_K, wd_, E, H, F, hq1, True, ids1, y=d1, status=st)
        cq.cq_moe_combine(d1, rw1, y=y1)

    us_dec = graph_us(ffn_decode, len(sets), 20, stream)
    wdec = K * wbytes // E
    out["q4_k_moe_ffn_decode_1tok_top4"] = {
        "graph_us": round(us_dec, 2), "expert_weight_GB/s": round(wdec / us_dec / 1e3, 1)}
    torch.cuda.synchronize()
    if int(st.cpu()[0]) != 0:
        raise RuntimeError("routed decode FFN reported invalid expert ids")
    del sets
    torch.cuda.empty_cache()
    return out


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(host_w, x, n, k, B, seconds):
    """The CPU oracle on the headline step (quantize the 4 rows, the LM-head
    GEMV at batch 1 and batch 4): whole steps repeated for about `seconds` on
    every core this process may run on, then a bounded sample on one core
    (the first 4096 rows of the matrix, scaled to GB/s).  GB/s of weights
    streamed.  The oracle is a plain fp64 correctness reference, not a tuned
    CPU kernel."""
    import oracle
    import gguf_synth as gs
    cores = host_cores()
    steps = 0
    t0 = time.perf_counter()
    while True:
        xq = oracle.quantize_q8_0(x)
        oracle.matmul(gs.Q4_K, host_w, n, k, xq[:1], 1, n_threads=cores, want_s=False)
        oracle.matmul(gs.Q4_K, host_w, n, k, xq, B, n_threads=cores, want_s=False)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    rows = 4096
    t1 = time.perf_counter()
    xq = oracle.quantize_q8_0(x)
    oracle.matmul(gs.Q4_K, host_w[:rows], rows, k, xq[:1], 1, n_threads=1, want_s=False)
    oracle.matmul(gs.Q4_K, host_w[:rows], rows, k, xq, B, n_threads=1, want_s=False)
    el1 = time.perf_counter() - t1
    return {"value": round(2 * host_w.nbytes * steps / el / 1e9, 3), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{steps} whole steps (quantize 4 rows, 128256x4096 Q4_K GEMV at batch 1 "
                      f"and 4) in {el:.1f} s on {cores} threads",
            "single_core_GB/s": round(2 * host_w[:rows].nbytes / el1 / 1e9, 4),
            "single_core_sample": f"rows 0..{rows - 1} of the step on 1 thread, {el1:.2f} s",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
