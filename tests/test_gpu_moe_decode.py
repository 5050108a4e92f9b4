"""Routed experts at decode (cq_moe_gemv, cq_moe_gemv_swiglu): one GEMV per
token-expert pair straight from the routing table, on the lfm2moe expert
shapes (32 experts, gate/up 1536 x 2048, down 2048 x 1536, top 4) for 1, 2
and 5 tokens.

Checks: each pair's output against the fp64 oracle's per-pair dots
(|y - y_ref| <= 2e-5*S); each pair bitwise equal to cq_gemv (cq_gemv_swiglu)
on that expert's matrix and activation row (the same single-pass kernel);
the fused gate/up output equal to the oracle SwiGLU of the two unfused
outputs within one fp32 ulp; ids outside [0, E) counted in the status
word with zero outputs for their pairs; and the whole
decode FFN (quantize, gate/up + SwiGLU, requantize, down, combine) against
the oracle's combine of the GPU's down outputs."""
import functools

import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import assert_close_to_oracle, note, to_dev, to_host

pytestmark = pytest.mark.gpu

C = gs.CONFIGS["q4_k_moe_ffn"]
H, F, E, K = C["hidden"], C["ffn"], C["n_experts"], C["top_k"]


@functools.lru_cache(maxsize=2)
def experts(fmt):
    cfg = 830
    return (gs.expert_weights(fmt, E, F, H, cfg, 0), gs.expert_weights(fmt, E, F, H, cfg, 1),
            gs.expert_weights(fmt, E, H, F, cfg, 2))


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


@pytest.mark.parametrize("fmt", [gs.Q4_K, gs.Q8_0, gs.Q5_K], ids=lambda f: gs.NAMES[f])
@pytest.mark.parametrize("n_tokens", [1, 2, 5])
def test_moe_gemv_decode(cq, orc, fmt, n_tokens):
    wg, wu, wd = experts(fmt)
    ids, rw = gs.routing(n_tokens, E, K, cfg=831 + n_tokens)
    x = gs.activations(n_tokens, H, cfg=831)
    xq_h = orc.quantize_q8_0(x)
    wgd, wud, wdd, xq, idd = to_dev(wg), to_dev(wu), to_dev(wd), to_dev(xq_h), to_dev(ids)
    note("moe gemv gate", gs.NAMES[fmt], n_tokens)
    g, st = cq.cq_moe_gemv(fmt, wgd, E, F, H, xq, False, idd)
    g = to_host(g)
    g_ref, sg = orc.moe_matmul(fmt, wg, E, F, H, xq_h, False, ids)
    assert_close_to_oracle(g, g_ref, sg, what="moe gemv gate")
    u = to_host(cq.cq_moe_gemv(fmt, wud, E, F, H, xq, False, idd, status=st)[0])
    # bitwise: pair p is cq_gemv on expert ids[p] and token p // K
    for p in range(n_tokens * K):
        e, t = int(ids.flat[p]), p // K
        yp = to_host(cq.cq_gemv(fmt, wgd[e * F:(e + 1) * F], F, H, xq[t:t + 1], 1))
        assert np.array_equal(yp[0], g[p]), p
    note("moe gemv swiglu", gs.NAMES[fmt], n_tokens)
    h = to_host(cq.cq_moe_gemv_swiglu(fmt, wgd, wud, E, F, H, xq, idd, status=st)[0])
    d = ulp_diff(h, orc.swiglu(g.astype(np.float32), u.astype(np.float32)))
    assert d.max() <= 1 and np.count_nonzero(d) <= max(2, d.size // 1000)
    # down: per-pair activation rows (the requantized h)
    hq_h = orc.quantize_q8_0(h)
    note("moe gemv down", gs.NAMES[fmt], n_tokens)
    dn = to_host(cq.cq_moe_gemv(fmt, wdd, E, H, F, to_dev(hq_h), True, idd, status=st)[0])
    d_ref, sd = orc.moe_matmul(fmt, wd, E, H, F, hq_h, True, ids)
    assert_close_to_oracle(dn, d_ref, sd, what="moe gemv down")
    assert to_host(st)[0] == 0


def test_moe_gemv_q6k_needs_whole_16_byte_rows(cq, orc):
    """Q6_K rows are 16-byte multiples only for k % 2048 == 0: the down
    projection (k = 1536) is refused, the gate (k = 2048) runs."""
    ids_h = np.array([[2, 0, 3, 1]], np.int32)
    ids = to_dev(ids_h)
    wd = to_dev(gs.weights(gs.Q6_K, 4 * H, F, cfg=845))
    hq = to_dev(orc.quantize_q8_0(gs.activations(K, F, cfg=845)))
    note("moe gemv q6_k refusal")
    with pytest.raises(RuntimeError, match="SHAPE"):
        cq.cq_moe_gemv(gs.Q6_K, wd, 4, H, F, hq, True, ids)
    wg_h = gs.weights(gs.Q6_K, 4 * F, H, cfg=846)
    xq_h = orc.quantize_q8_0(gs.activations(1, H, cfg=846))
    g = to_host(cq.cq_moe_gemv(gs.Q6_K, to_dev(wg_h), 4, F, H, to_dev(xq_h), False, ids)[0])
    g_ref, sg = orc.moe_matmul(gs.Q6_K, wg_h, 4, F, H, xq_h, False, ids_h)
    assert_close_to_oracle(g, g_ref, sg, what="moe gemv q6_k gate")


@pytest.mark.parametrize("fmt", [gs.Q1_0, gs.TQ2], ids=lambda f: gs.NAMES[f])
def test_moe_gemv_decode_sub_2bit(cq, orc, fmt):
    """Q1_0 and TQ2 experts on the routed decode path: the gate and the
    fused gate/up + SwiGLU (k = 2048) against the oracle and bitwise against
    cq_gemv / the SwiGLU of the two outputs; the down projection (k = 1536:
    rows of 216 / 408 bytes, not whole 16-byte pieces) is refused."""
    wg, wu, wd = experts(fmt)
    n_tokens = 3
    ids, _ = gs.routing(n_tokens, E, K, cfg=836)
    xq_h = orc.quantize_q8_0(gs.activations(n_tokens, H, cfg=836))
    wgd, wud, xq, idd = to_dev(wg), to_dev(wu), to_dev(xq_h), to_dev(ids)
    note("moe gemv sub-2-bit gate", gs.NAMES[fmt])
    g, st = cq.cq_moe_gemv(fmt, wgd, E, F, H, xq, False, idd)
    g = to_host(g)
    g_ref, sg = orc.moe_matmul(fmt, wg, E, F, H, xq_h, False, ids)
    assert_close_to_oracle(g, g_ref, sg, what=f"moe gemv {gs.NAMES[fmt]} gate")
    for p in range(n_tokens * K):
        e, t = int(ids.flat[p]), p // K
        yp = to_host(cq.cq_gemv(fmt, wgd[e * F:(e + 1) * F], F, H, xq[t:t + 1], 1))
        assert np.array_equal(yp[0], g[p]), p
    u = to_host(cq.cq_moe_gemv(fmt, wud, E, F, H, xq, False, idd, status=st)[0])
    note("moe gemv sub-2-bit swiglu", gs.NAMES[fmt])
    h = to_host(cq.cq_moe_gemv_swiglu(fmt, wgd, wud, E, F, H, xq, idd, status=st)[0])
    d = ulp_diff(h, orc.swiglu(g.astype(np.float32), u.astype(np.float32)))
    assert d.max() <= 1 and np.count_nonzero(d) <= max(2, d.size // 1000)
    assert to_host(st)[0] == 0
    hq = to_dev(orc.quantize_q8_0(h))
    with pytest.raises(RuntimeError, match="SHAPE"):
        cq.cq_moe_gemv(fmt, to_dev(wd), E, H, F, hq, True, idd)


@pytest.mark.parametrize("swiglu", [False, True])
def test_moe_gemv_invalid_ids(cq, orc, swiglu):
    """Ids outside [0, E): their pairs read no weights and give exact zeros,
    each adds 1 to the caller's status counter (which the library never
    clears), and the valid pairs are unaffected (bitwise)."""
    fmt = gs.Q4_K
    wg, wu, _ = experts(fmt)
    ids = np.array([[3, -5, 99, 31]], np.int32)
    good = np.array([[3, 3, 31, 31]], np.int32)
    xq = to_dev(orc.quantize_q8_0(gs.activations(1, H, cfg=840)))
    note("moe gemv invalid ids", swiglu)
    if swiglu:
        run = (lambda i, st: cq.cq_moe_gemv_swiglu(fmt, to_dev(wg), to_dev(wu), E, F, H, xq,
                                                   to_dev(i), status=st))
    else:
        run = (lambda i, st: cq.cq_moe_gemv(fmt, to_dev(wg), E, F, H, xq, False, to_dev(i),
                                            status=st))
    y, st = run(ids, None)
    y = to_host(y)
    assert to_host(st)[0] == 2
    ref, st2 = run(good, None)
    ref = to_host(ref)
    assert to_host(st2)[0] == 0
    assert np.array_equal(y[0], ref[0]) and np.array_equal(y[3], ref[3])
    assert not y[1].any() and not y[2].any()
    run(ids, st)                       # the counter accumulates
    assert to_host(st)[0] == 4


def test_moe_decode_ffn_end_to_end(cq, orc):
    """One token through the whole decode FFN on the GPU; the oracle combines
    the GPU's own down outputs (slot order, fp64) and checks each stage."""
    import torch
    fmt = gs.Q4_K
    wg, wu, wd = experts(fmt)
    ids, rw = gs.routing(1, E, K, cfg=850)
    x = gs.activations(1, H, cfg=850)
    note("moe decode ffn")
    xq = cq.cq_quantize_q8_0(to_dev(x))
    idd = to_dev(ids)
    h, st = cq.cq_moe_gemv_swiglu(fmt, to_dev(wg), to_dev(wu), E, F, H, xq, idd)
    hq = cq.cq_quantize_q8_0(h)
    dn, _ = cq.cq_moe_gemv(fmt, to_dev(wd), E, H, F, hq, True, idd, status=st)
    assert to_host(st)[0] == 0
    y = to_host(cq.cq_moe_combine(dn, to_dev(rw)))
    assert np.array_equal(to_host(hq), orc.quantize_q8_0(to_host(h)))
    d_ref, sd = orc.moe_matmul(fmt, wd, E, H, F, to_host(hq), True, ids)
    assert_close_to_oracle(to_host(dn), d_ref, sd, what="decode down")
    dh = to_host(dn).astype(np.float64)
    y_ref, _ = orc.moe_combine(dh, None, rw)
    # fp32 combine of K products: at most 2K roundings of magnitude <= sum|w*d|
    mag = np.abs(rw.astype(np.float64).reshape(1, K, 1) * dh.reshape(1, K, -1)).sum(axis=1)
    assert np.all(np.abs(y - y_ref) <= 2 * K * 2.0 ** -24 * mag + 1e-30)
    assert torch.cuda.is_available()
