"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream): the routed decode FFN
(quantize, fused gate/up + SwiGLU per pair, requantize, down per pair,
combine), the greedy arg-max of an LM-head GEMV and the router.  Each
replay is compared bitwise with the eager result, with eager work that
overwrites the same buffers between the replays."""
import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import note, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_decode_steps_graph_replays(cq, orc):
    import torch
    C = gs.CONFIGS["q4_k_moe_ffn"]
    H, F, E, K = C["hidden"], C["ffn"], C["n_experts"], C["top_k"]
    fmt = gs.Q4_K
    wg = to_dev(gs.expert_weights(fmt, E, F, H, 860, 0))
    wu = to_dev(gs.expert_weights(fmt, E, F, H, 860, 1))
    wd = to_dev(gs.expert_weights(fmt, E, H, F, 860, 2))
    n_lm = 4096
    wl = to_dev(gs.weights(fmt, n_lm, H, cfg=861))
    x = to_dev(gs.activations(1, H, cfg=862))
    logits = to_dev(np.random.default_rng(863).standard_normal((1, E)).astype(np.float32))
    xq = torch.empty((1, H // 32 * 34), dtype=torch.uint8, device="cuda")
    ids = torch.empty((1, K), dtype=torch.int32, device="cuda")
    rw = torch.empty((1, K), dtype=torch.float32, device="cuda")
    h = torch.empty((K, F), dtype=torch.float32, device="cuda")
    hq = torch.empty((K, F // 32 * 34), dtype=torch.uint8, device="cuda")
    d = torch.empty((K, H), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
    yq = torch.empty((1, H // 32 * 34), dtype=torch.uint8, device="cuda")
    lg = torch.empty((1, n_lm), dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(cq.load().cq_argmax_workspace_bytes(1, n_lm), dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        cq.cq_topk_softmax(logits, K, ids=ids, w=rw)
        cq.cq_quantize_q8_0(x, xq)
        cq.cq_moe_gemv_swiglu(fmt, wg, wu, E, F, H, xq, ids, h=h, status=st)
        cq.cq_quantize_q8_0(h, hq)
        cq.cq_moe_gemv(fmt, wd, E, H, F, hq, True, ids, y=d, status=st)
        cq.cq_moe_combine(d, rw, y=y)
        cq.cq_quantize_q8_0(y, yq)
        cq.cq_gemv(fmt, wl, n_lm, H, yq, 1, y=lg)
        cq.cq_argmax(lg, idx=tok, workspace=ws)

    note("graph: eager step")
    step()
    ref = [to_host(t).copy() for t in (ids, rw, h, d, y, lg, tok)]
    note("graph: capture")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                    # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # eager work that overwrites every buffer the graph writes
        for t in (h, d, y, lg, rw):
            t.fill_(-7.0)
        tok.fill_(-1)
        ids.fill_(0)
        cq.cq_gemv(fmt, wl, n_lm, H, yq, 1, y=lg)
        torch.cuda.synchronize()
        note("graph: replay", r)
        g.replay()
        torch.cuda.synchronize()
        got = [to_host(t) for t in (ids, rw, h, d, y, lg, tok)]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), r
    assert to_host(st)[0] == 0        # no out-of-range expert id in any call
    # and the step's result is the oracle's arg-max of its own logits
    assert ref[-1][0] == orc.argmax_rows(ref[-2])[0]
