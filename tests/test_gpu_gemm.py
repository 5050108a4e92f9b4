"""GPU parity of the prefill GEMM (cq_gemm, int8 MFMA) against the fp64
oracle: |y - y_ref| <= 2e-5 * sum|w_hat*x_hat| per output; small shapes
with ragged M and N tails for every weight type, the prefill workload at
M = 512 and M = 2048 in full, and invariants
(determinism, power-of-two scaling, GEMM rows against the GEMV)."""
import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import assert_close_to_oracle, note, to_dev, to_host

pytestmark = pytest.mark.gpu

FMTS = [gs.Q4_0, gs.Q4_1, gs.Q8_0, gs.Q4_K, gs.Q5_K, gs.Q6_K]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (37, 130, 256), (128, 128, 512), (200, 300, 1024),
                                   (5, 257, 4096), (129, 64, 768),
                                   # grids dealt to the XCDs in bands of two token
                                   # tiles (ragged m and n), with and without tail tiles
                                   (250, 1000, 512), (250, 1100, 512), (500, 2000, 256)])
def test_gemm_small_shapes(cq, orc, fmt, m, n, k):
    note("gemm", gs.NAMES[fmt], m, n, k)
    w = gs.weights(fmt, n, k, cfg=600 + m)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=600 + m))
    y = to_host(cq.cq_gemm(fmt, to_dev(w), n, k, to_dev(xq), m))
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, m)
    assert_close_to_oracle(y, y_ref, s_ref, what=f"gemm {gs.NAMES[fmt]} {m}x{n}x{k}")


def test_gemm_prefill_512_full(cq, orc):
    c = gs.CONFIGS["q4_0_gemm_prefill_512"]
    n, k, m = c["n"], c["k"], c["m"]
    w = gs.weights(c["fmt"], n, k, cfg=c["cfg"])
    x = gs.activations(m, k, cfg=c["cfg"])
    note("gemm prefill 512 quantize")
    xq_d = cq.cq_quantize_q8_0(to_dev(x))
    xq = orc.quantize_q8_0(x)
    assert np.array_equal(to_host(xq_d), xq)
    note("gemm prefill 512")
    y = to_host(cq.cq_gemm(c["fmt"], to_dev(w), n, k, xq_d, m))
    y_ref, s_ref = orc.matmul(c["fmt"], w, n, k, xq, m)
    r = assert_close_to_oracle(y, y_ref, s_ref, what="prefill 512")
    print(f"prefill 512: max |err|/S = {r:.3e}")


@pytest.mark.parametrize("name", ["q4_0_gemm_prefill_2048", "q5_k_gemm_prefill_512",
                                  "q6_k_gemm_prefill_512"])
def test_gemm_prefill_full(cq, orc, name):
    """The 2048-token Q4_0 prefill and the 512-token Q5_K / Q6_K prefills:
    every output against the oracle."""
    c = gs.CONFIGS[name]
    n, k, m = c["n"], c["k"], c["m"]
    w = gs.weights(c["fmt"], n, k, cfg=c["cfg"])
    x = gs.activations(m, k, cfg=c["cfg"])
    xq = orc.quantize_q8_0(x)
    note("gemm prefill", name)
    y = to_host(cq.cq_gemm(c["fmt"], to_dev(w), n, k, to_dev(xq), m))
    y_ref, s_ref = orc.matmul(c["fmt"], w, n, k, xq, m)
    r = assert_close_to_oracle(y, y_ref, s_ref, what=name)
    print(f"{name}: max |err|/S = {r:.3e}")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
def test_gemm_invariants(cq, orc, fmt):
    m, n, k = 70, 200, 1024
    w = gs.weights(fmt, n, k, cfg=610)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=610))
    wd, xd = to_dev(w), to_dev(xq)
    note("gemm invariants", gs.NAMES[fmt])
    y0 = to_host(cq.cq_gemm(fmt, wd, n, k, xd, m))
    y1 = to_host(cq.cq_gemm(fmt, wd, n, k, xd, m))
    assert np.array_equal(y0, y1)
    # doubling every weight scale doubles y bitwise
    w2 = w.copy().reshape(-1, gs.BLOCK_BYTES[fmt])
    offs = [208] if fmt == gs.Q6_K else [0, 2] if fmt in (gs.Q4_1, gs.Q4_K, gs.Q5_K) else [0]
    for o in offs:
        h = w2[:, o:o + 2].copy().view(np.float16)
        w2[:, o:o + 2] = (h * np.float16(2)).view(np.uint8)
    y2 = to_host(cq.cq_gemm(fmt, to_dev(w2.reshape(n, -1)), n, k, xd, m))
    assert np.array_equal(y2, 2 * y0)
    # a GEMM row agrees with the GEMV on that row (both within tolerance of
    # the oracle; different summation orders)
    yv = to_host(cq.cq_gemv(fmt, wd, n, k, xd[3:4], 1))
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq[3:4], 1)
    assert_close_to_oracle(yv, y_ref, s_ref, what="gemv row")
    assert np.all(np.abs(yv[0] - y0[3]) <= 4e-5 * s_ref[0])


def test_gemm_strided_output(cq, orc):
    import torch
    fmt, m, n, k = gs.Q4_0, 33, 100, 512
    w = gs.weights(fmt, n, k, cfg=611)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=611))
    note("gemm strided y")
    y = torch.full((m, 131), -3.0, device="cuda")
    cq.cq_gemm(fmt, to_dev(w), n, k, to_dev(xq), m, y=y, ldy=131)
    yh = to_host(y)
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, m)
    assert_close_to_oracle(yh[:, :n], y_ref, s_ref, what="strided")
    assert np.all(yh[:, n:] == -3.0)


@pytest.mark.parametrize("fmt", [gs.Q4_0, gs.Q6_K], ids=lambda f: gs.NAMES[f])
def test_gemm_max_k(cq, orc, fmt):
    """k = CQ_MAX_K (65536) with ragged m and n."""
    m, n, k = 19, 130, 65536
    w = gs.weights(fmt, n, k, cfg=620)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=620))
    note("gemm max k", gs.NAMES[fmt])
    y = to_host(cq.cq_gemm(fmt, to_dev(w), n, k, to_dev(xq), m))
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, m)
    assert_close_to_oracle(y, y_ref, s_ref, what="gemm max k")
