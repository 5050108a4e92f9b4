"""Greedy arg-max over logit rows (cq_argmax) and the top-k expert router
(cq_topk_softmax) against the oracle.

Arg-max is integer work: bit-exact.  It is checked on the 128256-logit LM
head at batch 4 (the logits the Q4_K LM-head GEMV writes), on random rows
with planted ties (the first index wins), signed zeros, all-equal rows,
ragged and strided rows (n not a multiple of 4; rows not 16-byte aligned)
and the chunk boundaries of the two-launch reduction.  The router's ids are
bit-exact; its fp64-softmax weights agree with the oracle's to one fp32 ulp
(the two exp implementations may differ in the last fp64 bit)."""
import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import note, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_argmax_lm_head_logits(cq, orc):
    c = gs.CONFIGS["q4_k_gemv_lm_head"]
    n, k = c["n"], c["k"]
    w = to_dev(gs.weights(c["fmt"], n, k, cfg=c["cfg"]))
    xq = cq.cq_quantize_q8_0(to_dev(gs.activations(4, k, cfg=c["cfg"])))
    note("argmax lm head")
    y = cq.cq_gemv(c["fmt"], w, n, k, xq, 4)
    idx = to_host(cq.cq_argmax(y))
    assert np.array_equal(idx, orc.argmax_rows(to_host(y)))


@pytest.mark.parametrize("rows,n", [(1, 1), (3, 7), (2, 4096), (5, 4097), (4, 128256), (8, 50001)])
def test_argmax_random_rows(cq, orc, rows, n):
    rng = np.random.default_rng(900 + n)
    y = rng.standard_normal((rows, n)).astype(np.float32)
    if n > 10:
        y[0, n // 3] = y[0, n - 1] = 50.0            # tie: the first index wins
    if rows > 2:
        y[2, :] = 0.0
        y[2, n // 2] = np.float32(-0.0)              # -0 == +0: index 0
    if rows > 3 and n > 4096:
        y[3, 4095] = y[3, 4096] = 60.0               # tie across the chunk boundary
    note("argmax", rows, n)
    idx = to_host(cq.cq_argmax(to_dev(y)))
    assert np.array_equal(idx, orc.argmax_rows(y)), (idx, orc.argmax_rows(y))


def test_argmax_strided_unaligned(cq, orc):
    import torch
    rng = np.random.default_rng(910)
    big = rng.standard_normal((6, 9000)).astype(np.float32)
    yd = to_dev(big)
    note("argmax strided")
    # rows of 8191 values starting 1 float into each 9000-float row
    view = yd[:, 1:8192]
    ws = torch.zeros(cq.load().cq_argmax_workspace_bytes(6, 8191), dtype=torch.uint8, device="cuda")
    idx = to_host(cq.cq_argmax(view, workspace=ws))
    assert np.array_equal(idx, orc.argmax_rows(big[:, 1:8192]))


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


@pytest.mark.parametrize("rows,E,K", [(256, 32, 4), (5, 32, 1), (3, 8, 8), (40, 1000, 16), (1, 64, 4)])
def test_router(cq, orc, rows, E, K):
    rng = np.random.default_rng(920 + E + K)
    logits = rng.standard_normal((rows, E)).astype(np.float32)
    logits[0, [1, 5, E - 1]] = 4.0                   # tie at the top: smaller id first
    if rows > 1:
        logits[1, :] = 0.5                           # all equal
    note("router", rows, E, K)
    ids, w = cq.cq_topk_softmax(to_dev(logits), K)
    ids, w = to_host(ids), to_host(w)
    ids_ref, w_ref = orc.topk_softmax(logits, K)
    assert np.array_equal(ids, ids_ref)
    assert ulp_diff(w, w_ref).max() <= 1


def test_router_feeds_the_moe(cq, orc):
    """Router output drives grouping exactly as the oracle's routing."""
    rows, E, K = 64, 32, 4
    logits = np.random.default_rng(930).standard_normal((rows, E)).astype(np.float32)
    note("router -> group")
    ids, _ = cq.cq_topk_softmax(to_dev(logits), K)
    offs, pairs, st = cq.cq_moe_group(ids, E)
    offs_ref, pairs_ref = orc.moe_group(orc.topk_softmax(logits, K)[0], E)
    assert np.array_equal(to_host(offs), offs_ref) and np.array_equal(to_host(pairs), pairs_ref)
    assert to_host(st)[0] == 0
