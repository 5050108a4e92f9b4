"""Fused decode FFN front half (cq_gemv_swiglu): h = silu(W_gate x) * (W_up x).

Checks: (1) g and u inside the fused kernel are the values cq_gemv returns
for the two matrices, so h equals the oracle's SwiGLU of the two cq_gemv
results (fp64 silu on both sides; the two exp implementations may differ in
the last fp64 bit, which can move h by one fp32 ulp); (2) h against the fp64
oracle within the bound propagated from the GEMV tolerance:
|h - h_ref| <= L*|eg|*(|u_ref| + |eu|) + |silu(g_ref)|*|eu| + 2^-23*|h_ref|,
|eg| <= 2e-5*S_g, |eu| <= 2e-5*S_u, L = 1.1 >= max|silu'|; (3) batch rows
equal single-row calls; (4) shapes without the single-pass kernel are
refused."""
import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import TOL, note, to_dev, to_host

pytestmark = pytest.mark.gpu

FMTS = [gs.Q4_0, gs.Q4_1, gs.Q8_0, gs.Q4_K, gs.Q5_K, gs.Q6_K, gs.Q1_0, gs.TQ2]


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def check_against_separate(cq, orc, fmt, wg, wu, n, k, xq, batch, h):
    g = to_host(cq.cq_gemv(fmt, wg, n, k, xq, batch))
    u = to_host(cq.cq_gemv(fmt, wu, n, k, xq, batch))
    h_sep = orc.swiglu(g, u)
    d = ulp_diff(h, h_sep)
    assert d.max() <= 1, (fmt, n, k, batch, int(d.max()))
    assert np.count_nonzero(d) <= max(2, d.size // 1000)


def check_against_oracle(orc, fmt, wg_h, wu_h, n, k, xq_h, batch, h):
    g_ref, s_g = orc.matmul(fmt, wg_h, n, k, xq_h, batch)
    u_ref, s_u = orc.matmul(fmt, wu_h, n, k, xq_h, batch)
    with np.errstate(over="ignore"):   # exp(-g) = inf for very negative g: silu -> -0
        silu = g_ref / (1.0 + np.exp(-g_ref))
    h_ref = silu * u_ref
    eg, eu = TOL * s_g, TOL * s_u
    bound = 1.1 * eg * (np.abs(u_ref) + eu) + np.abs(silu) * eu + 2.0 ** -23 * np.abs(h_ref) + 1e-30
    err = np.abs(h.astype(np.float64) - h_ref)
    assert np.all(err <= bound), float(np.max(err / bound))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
@pytest.mark.parametrize("n,k", [(1, 2048), (37, 256), (300, 1024), (1001, 2048), (257, 4096),
                                 (45, 8192), (130, 14336), (3, 16384), (1, 8192), (3, 8192),
                                 (33, 5120)])
def test_gemv_swiglu_small(cq, orc, fmt, n, k):
    if k % 256 or gs.row_bytes(fmt, k) % 16:
        pytest.skip("no single-pass kernel for this (type, k)")
    wg_h = gs.weights(fmt, n, k, cfg=800 + n, tensor=0)
    wu_h = gs.weights(fmt, n, k, cfg=800 + n, tensor=1)
    xq_h = orc.quantize_q8_0(gs.activations(8, k, cfg=800 + n))
    wg, wu, xq = to_dev(wg_h), to_dev(wu_h), to_dev(xq_h)
    for batch in (1, 3, 5, 8):
        note("gemv swiglu", gs.NAMES[fmt], n, k, batch)
        h = to_host(cq.cq_gemv_swiglu(fmt, wg, wu, n, k, xq[:batch], batch))
        check_against_separate(cq, orc, fmt, wg, wu, n, k, xq[:batch], batch, h)
        check_against_oracle(orc, fmt, wg_h, wu_h, n, k, xq_h[:batch], batch, h)


@pytest.mark.parametrize("fmt", [gs.Q4_K, gs.Q8_0], ids=lambda f: gs.NAMES[f])
def test_gemv_swiglu_ffn_shape(cq, orc, fmt):
    """8B-class FFN gate/up 14336 x 4096 at batch 1 and 5: all outputs."""
    n, k = 14336, 4096
    wg_h = gs.weights(fmt, n, k, cfg=810, tensor=0)
    wu_h = gs.weights(fmt, n, k, cfg=810, tensor=1)
    xq_h = orc.quantize_q8_0(gs.activations(5, k, cfg=810))
    wg, wu, xq = to_dev(wg_h), to_dev(wu_h), to_dev(xq_h)
    h5 = None
    for batch in (5, 1):
        note("gemv swiglu ffn", gs.NAMES[fmt], batch)
        h = to_host(cq.cq_gemv_swiglu(fmt, wg, wu, n, k, xq[:batch], batch))
        check_against_separate(cq, orc, fmt, wg, wu, n, k, xq[:batch], batch, h)
        check_against_oracle(orc, fmt, wg_h, wu_h, n, k, xq_h[:batch], batch, h)
        if batch == 5:
            h5 = h
        else:
            assert np.array_equal(h[0], h5[0])   # batch rows equal single-row calls


def test_gemv_swiglu_strided_and_refusals(cq, orc):
    import torch
    fmt, n, k = gs.Q4_0, 100, 1024
    wg_h = gs.weights(fmt, n, k, cfg=820, tensor=0)
    wu_h = gs.weights(fmt, n, k, cfg=820, tensor=1)
    xq_h = orc.quantize_q8_0(gs.activations(2, k, cfg=820))
    wg, wu, xq = to_dev(wg_h), to_dev(wu_h), to_dev(xq_h)
    note("gemv swiglu strided")
    h = torch.full((2, 130), -3.0, device="cuda")
    cq.cq_gemv_swiglu(fmt, wg, wu, n, k, xq, 2, h=h, ldh=130)
    hh = to_host(h)
    assert np.all(hh[:, n:] == -3.0)
    check_against_oracle(orc, fmt, wg_h, wu_h, n, k, xq_h, 2, hh[:, :n])
    # k = 20480 needs five waves per row (beyond the k-split form's four),
    # k = 4160 gives rows that are not whole 16-byte pieces: refused,
    # nothing launched
    for kk in (20480, 4160):
        w8 = to_dev(gs.weights(fmt, 4, kk, cfg=821))
        x8 = to_dev(orc.quantize_q8_0(gs.activations(1, kk, cfg=821)))
        with pytest.raises(RuntimeError, match="SHAPE"):
            cq.cq_gemv_swiglu(fmt, w8, w8, 4, kk, x8, 1)
