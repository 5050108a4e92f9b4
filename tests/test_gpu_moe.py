"""GPU parity of the routed expert FFN (lfm2moe shape: 256 tokens, hidden
2048, 32 Q4_K experts with gate/up 1536 x 2048 and down 2048 x 1536, top 4).

Checked stage by stage; every stage's inputs come from the oracle (or from
the seeded generator), never from the GPU:
  gate / up   grouped GEMM on the oracle's Q8_0 rows and grouping, against
              the oracle's per-pair dots: |y - y_ref| <= 2e-5 * S;
  down        grouped GEMM on the oracle's requantized SwiGLU output;
  combine     slot-order combine of the oracle's expert outputs;
then the one-call routed projection (cq_moe_gemm: grouping, grouped product
and slot-order combine in one call on a caller workspace) per stage, the
whole GPU pipeline end to end through it against the oracle pipeline with a
bound derived from the oracle's values, its status word on out-of-range
expert ids, and the reduction to dense GEMMs when every token picks the same
experts."""
import functools

import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import assert_close_to_oracle, note, to_dev, to_host

pytestmark = pytest.mark.gpu

C = gs.CONFIGS["q4_k_moe_ffn"]
T, H, F, E, K = C["n_tokens"], C["hidden"], C["ffn"], C["n_experts"], C["top_k"]
FMT = C["fmt"]


@functools.lru_cache(maxsize=1)
def inputs():
    cfg = C["cfg"]
    wg = gs.expert_weights(FMT, E, F, H, cfg, 0)
    wu = gs.expert_weights(FMT, E, F, H, cfg, 1)
    wd = gs.expert_weights(FMT, E, H, F, cfg, 2)
    x = gs.activations(T, H, cfg)
    ids, rw = gs.routing(T, E, K, cfg)
    return wg, wu, wd, x, ids, rw


@functools.lru_cache(maxsize=1)
def oracle_pipeline():
    import oracle as orc
    wg, wu, wd, x, ids, rw = inputs()
    xq = orc.quantize_q8_0(x)
    g, sg = orc.moe_matmul(FMT, wg, E, F, H, xq, False, ids)
    u, su = orc.moe_matmul(FMT, wu, E, F, H, xq, False, ids)
    h = orc.swiglu(g.astype(np.float32), u.astype(np.float32))
    hq = orc.quantize_q8_0(h)
    d, sd = orc.moe_matmul(FMT, wd, E, H, F, hq, True, ids)
    y, sy = orc.moe_combine(d, sd, rw)
    offs, pairs = orc.moe_group(ids, E)
    return dict(xq=xq, g=g, sg=sg, u=u, su=su, h=h, hq=hq, d=d, sd=sd, y=y, sy=sy,
                offs=offs, pairs=pairs)


def test_moe_gate_up(cq):
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    offs, pairs = to_dev(ref["offs"]), to_dev(ref["pairs"])
    xq = to_dev(ref["xq"])
    for name, w, yr, sr in (("gate", wg, ref["g"], ref["sg"]), ("up", wu, ref["u"], ref["su"])):
        note("moe", name)
        y = to_host(cq.cq_moe_gemm_grouped(FMT, to_dev(w), E, F, H, xq, False, offs, pairs, T, K))
        r = assert_close_to_oracle(y, yr, sr, what=name)
        print(f"{name}: max |err|/S = {r:.3e}")


def test_moe_gate_up_one_call(cq):
    """Gate and up in one call (one split of each expert's rows for both
    matrices): each output within 2e-5 * S of the oracle and bitwise equal to
    the separate grouped call."""
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    offs, pairs = to_dev(ref["offs"]), to_dev(ref["pairs"])
    xq = to_dev(ref["xq"])
    note("moe gate+up one call")
    wgd, wud = to_dev(wg), to_dev(wu)
    ya, yb = cq.cq_moe_gemm_grouped2(FMT, wgd, wud, E, F, H, xq, False, offs, pairs, T, K)
    ya, yb = to_host(ya), to_host(yb)
    assert_close_to_oracle(ya, ref["g"], ref["sg"], what="gate (one call)")
    assert_close_to_oracle(yb, ref["u"], ref["su"], what="up (one call)")
    assert np.array_equal(ya, to_host(cq.cq_moe_gemm_grouped(FMT, wgd, E, F, H, xq, False, offs,
                                                             pairs, T, K)))
    assert np.array_equal(yb, to_host(cq.cq_moe_gemm_grouped(FMT, wud, E, F, H, xq, False, offs,
                                                             pairs, T, K)))


@pytest.mark.parametrize("fmt,n_tokens,n_experts,top_k,n,k,x_per_pair",
                         [(gs.Q4_K, 70, 8, 2, 200, 1536, True), (gs.Q4_K, 300, 4, 2, 2000, 2048, False),
                          (gs.Q4_K, 40, 6, 2, 200, 512, False), (gs.Q8_0, 40, 6, 2, 200, 512, True)],
                         ids=["q4_k-k1536", "q4_k-k2048-ragged", "q4_k-k512", "q8_0"])
def test_moe_gemm_grouped2_shapes(cq, orc, fmt, n_tokens, n_experts, top_k, n, k, x_per_pair):
    """Two projections in one call: one launch for Q4_K at k = 1536 / 2048
    (ragged n, several passes per expert, two row groups per wave), two
    launches otherwise; both outputs within tolerance of the oracle and
    bitwise equal to separate calls."""
    wa = gs.expert_weights(fmt, n_experts, n, k, cfg=750 + n_tokens, which=0)
    wb = gs.expert_weights(fmt, n_experts, n, k, cfg=750 + n_tokens, which=1)
    ids, _ = gs.routing(n_tokens, n_experts, top_k, cfg=750 + n_tokens)
    offs, pairs = orc.moe_group(ids, n_experts)
    rows = n_tokens * top_k if x_per_pair else n_tokens
    xq = orc.quantize_q8_0(gs.activations(rows, k, cfg=751))
    note("moe gemm grouped2", gs.NAMES[fmt], n_tokens, n_experts, top_k, n, k, x_per_pair)
    args = (n_experts, n, k, to_dev(xq), x_per_pair, to_dev(offs), to_dev(pairs), n_tokens, top_k)
    wad, wbd = to_dev(wa), to_dev(wb)
    ya, yb = cq.cq_moe_gemm_grouped2(fmt, wad, wbd, *args)
    ya, yb = to_host(ya), to_host(yb)
    for y, w, name in ((ya, wa, "first"), (yb, wb, "second")):
        y_ref, s_ref = orc.moe_matmul(fmt, w, n_experts, n, k, xq, x_per_pair, ids)
        assert_close_to_oracle(y, y_ref, s_ref, what=f"grouped2 {name}")
    assert np.array_equal(ya, to_host(cq.cq_moe_gemm_grouped(fmt, wad, *args)))
    assert np.array_equal(yb, to_host(cq.cq_moe_gemm_grouped(fmt, wbd, *args)))


def test_moe_down(cq):
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    note("moe down")
    y = to_host(cq.cq_moe_gemm_grouped(FMT, to_dev(wd), E, H, F, to_dev(ref["hq"]), True,
                                       to_dev(ref["offs"]), to_dev(ref["pairs"]), T, K))
    r = assert_close_to_oracle(y, ref["d"], ref["sd"], what="down")
    print(f"down: max |err|/S = {r:.3e}")


def test_moe_combine_stage(cq, orc):
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    d32 = ref["d"].astype(np.float32)
    note("moe combine stage")
    y = to_host(cq.cq_moe_combine(to_dev(d32), to_dev(rw)))
    y_ref, _ = orc.moe_combine(d32.astype(np.float64), None, rw)
    mag, _ = orc.moe_combine(np.abs(d32).astype(np.float64), None, np.abs(rw))
    assert np.all(np.abs(y - y_ref) <= 4 * 2.0 ** -24 * mag + 1e-30)


def one_call(cq, w, n, k, xq, flags, ids, rw=None):
    """cq_moe_gemm on a workspace of exactly the size it asks for; returns
    (y, status) on the host."""
    import torch
    n_tokens, top_k = ids.shape
    need = cq.cq_moe_workspace_bytes(n_tokens, top_k, E, n, flags)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y, st = cq.cq_moe_gemm(FMT, w, E, n, k, xq, flags, ids, route_w=rw, workspace=ws)
    return y, int(to_host(st)[0])


def run_gpu_pipeline(cq, wg, wu, wd, x, ids, rw):
    """The routed FFN through the one-call entry point: gate and up per pair,
    SwiGLU + requantization, down combined over each token's slots."""
    idd = to_dev(ids)
    xq = cq.cq_quantize_q8_0(to_dev(x))
    g, s1 = one_call(cq, to_dev(wg), F, H, xq, cq.MOE_X_PER_TOKEN | cq.MOE_OUT_PER_PAIR, idd)
    u, s2 = one_call(cq, to_dev(wu), F, H, xq, cq.MOE_X_PER_TOKEN | cq.MOE_OUT_PER_PAIR, idd)
    _, hq = cq.cq_swiglu_quantize_q8_0(g, u)
    y, s3 = one_call(cq, to_dev(wd), H, F, hq, cq.MOE_X_PER_PAIR | cq.MOE_OUT_COMBINE, idd,
                     to_dev(rw))
    assert (s1, s2, s3) == (0, 0, 0)
    return to_host(y)


def test_moe_one_call_stages(cq, orc):
    """cq_moe_gemm per stage on the oracle's inputs: the gate projection per
    pair (2e-5 * S), and the down projection combined over slots: each
    product within 2e-5 * S_down of the oracle, then four fp32 FMAs in slot
    order, so |y - y_ref| <= 2e-5 * sum_s |w| S_down + 4 ulp of sum_s |w D|."""
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    idd = to_dev(ids)
    note("moe one-call gate")
    g, st = one_call(cq, to_dev(wg), F, H, to_dev(ref["xq"]),
                     cq.MOE_X_PER_TOKEN | cq.MOE_OUT_PER_PAIR, idd)
    assert st == 0
    r = assert_close_to_oracle(to_host(g), ref["g"], ref["sg"], what="one-call gate")
    print(f"one-call gate: max |err|/S = {r:.3e}")
    note("moe one-call down + combine")
    y, st = one_call(cq, to_dev(wd), H, F, to_dev(ref["hq"]),
                     cq.MOE_X_PER_PAIR | cq.MOE_OUT_COMBINE, idd, to_dev(rw))
    assert st == 0
    mag, _ = orc.moe_combine(np.abs(ref["d"]), None, np.abs(rw))
    err = np.abs(to_host(y) - ref["y"])
    assert np.all(err <= 2e-5 * ref["sy"] + 4 * 2.0 ** -24 * mag + 1e-30)
    print(f"one-call down + combine: max |err|/S = {(err / ref['sy']).max():.3e}")


def test_moe_one_call_invalid_ids(cq, orc):
    """Expert ids outside [0, E) are counted in the workspace status word;
    combined rows leave those slots out, and every other output is right."""
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    bad = ids[:16].copy()
    bad[3, 1] = -1
    bad[9, 3] = E
    bad[9, 0] = 1 << 30
    note("moe one-call invalid ids")
    y, st = one_call(cq, to_dev(wd), H, F, to_dev(ref["hq"][:16 * K]),
                     cq.MOE_X_PER_PAIR | cq.MOE_OUT_COMBINE, to_dev(bad), to_dev(rw[:16]))
    assert st == 3
    d = ref["d"][:16 * K].copy()
    sd = ref["sd"][:16 * K].copy()
    for t, s in ((3, 1), (9, 3), (9, 0)):
        d[t * K + s] = 0.0
        sd[t * K + s] = 0.0
    y_ref, s_ref = orc.moe_combine(d, sd, rw[:16])
    mag, _ = orc.moe_combine(np.abs(d), None, np.abs(rw[:16]))
    assert np.all(np.abs(to_host(y) - y_ref) <= 2e-5 * s_ref + 4 * 2.0 ** -24 * mag + 1e-30)
    note("moe one-call per pair, valid ids")
    yp, st = one_call(cq, to_dev(wd), H, F, to_dev(ref["hq"][:16 * K]),
                      cq.MOE_X_PER_PAIR | cq.MOE_OUT_PER_PAIR, to_dev(ids[:16]))
    assert st == 0
    assert_close_to_oracle(to_host(yp), ref["d"][:16 * K], ref["sd"][:16 * K], what="per pair")


def test_moe_end_to_end(cq):
    """The whole GPU pipeline against the oracle pipeline.  Requantizing h can
    move a quant by one step where the GPU's h and the oracle's h straddle a
    rounding boundary, so the bound adds, per pair, one quantization step of
    every element of h (oracle scales) weighted by |W_down| -- a bound derived
    from the oracle's values alone -- to the 2e-5 * S tolerance."""
    import oracle as orc
    wg, wu, wd, x, ids, rw = inputs()
    ref = oracle_pipeline()
    note("moe end to end")
    y = run_gpu_pipeline(cq, wg, wu, wd, x, ids, rw)
    # |W_down| * (one quant step of h per element) via the oracle's own dots:
    # quantization step of each h block = its fp16 scale d
    hq = ref["hq"].reshape(T * K, F // 32, 34)
    dh = orc.half_to_double(hq[:, :, :2].copy().view(np.uint16)).reshape(T * K, F // 32)
    # per element of h: |h_gpu - h_ref| is at most the propagated gate/up
    # error (|dh/dg| <= 1.1|u|, |dh/du| = |silu(g)|) plus fp32 rounding; the two
    # requantizations then differ by at most that plus one quant step
    g, u = ref["g"], ref["u"]
    silu = g / (1.0 + np.exp(-np.clip(g, -700.0, 700.0)))
    dh_in = 1.1 * np.abs(u) * 2e-5 * ref["sg"] + np.abs(silu) * 2e-5 * ref["su"] \
        + 2.0 ** -22 * np.abs(ref["h"].astype(np.float64))
    step = 1.01 * np.repeat(dh, 32, axis=1) + dh_in                       # [pairs][F]
    wabs = np.stack([np.abs(orc.dequantize(FMT, wd[r], F)) for r in range(E * H)]).reshape(E, H, F)
    flip = np.zeros((T * K, H))
    e_of = ids.reshape(-1)
    for p in range(T * K):
        flip[p] = wabs[e_of[p]] @ step[p]
    flip_tok = (np.abs(rw.astype(np.float64)).reshape(T, K, 1) * flip.reshape(T, K, H)).sum(axis=1)
    err = np.abs(y - ref["y"])
    bound = 2e-5 * ref["sy"] + flip_tok
    ratio = err / np.maximum(bound, 1e-300)
    print(f"end to end: max err/bound = {ratio.max():.3e}, max err/S = {(err / ref['sy']).max():.3e}")
    assert np.all(err <= bound)


def test_moe_reduces_to_dense(cq, orc):
    """Every token routed to the same experts: each grouped projection equals
    the dense GEMM with that expert's weights (both within 2e-5 * S of the
    oracle; the grouped Q4_K kernel applies the two block scales in the other
    order, so the two agree to within twice the tolerance, not bitwise)."""
    wg, wu, wd, x, ids, rw = inputs()
    tok = 100
    ids2 = np.tile(np.array([[5, 17, 2, 31]], np.int32), (tok, 1))
    xq = cq.cq_quantize_q8_0(to_dev(x[:tok]))
    note("moe dense reduction")
    offs, pairs, _ = cq.cq_moe_group(to_dev(ids2), E)
    g = to_host(cq.cq_moe_gemm_grouped(FMT, to_dev(wg), E, F, H, xq, False, offs, pairs, tok, K))
    xq_h = to_host(xq)
    for s, e in enumerate([5, 17, 2, 31]):
        we = wg[e * F:(e + 1) * F]
        yd = to_host(cq.cq_gemm(FMT, to_dev(we), F, H, xq, tok))
        y_ref, s_ref = orc.matmul(FMT, we, F, H, xq_h, tok)
        assert_close_to_oracle(g[s::K], y_ref, s_ref, what=f"grouped, expert {e}")
        assert_close_to_oracle(yd, y_ref, s_ref, what=f"dense, expert {e}")
        assert np.all(np.abs(g[s::K] - yd) <= 4e-5 * s_ref)


@pytest.mark.parametrize("n_tokens,n_experts,top_k,n,k", [(1, 8, 2, 128, 256), (300, 4, 2, 200, 512),
                                                          (64, 64, 1, 100, 256)])
def test_moe_gemm_shapes(cq, orc, n_tokens, n_experts, top_k, n, k):
    """Empty experts, experts with more than one 64-row tile, n not a
    multiple of 128, per-pair and per-token activation rows."""
    w = gs.expert_weights(FMT, n_experts, n, k, cfg=700 + n_tokens, which=0)
    ids, _ = gs.routing(n_tokens, n_experts, top_k, cfg=700 + n_tokens)
    for x_per_pair in (False, True):
        rows = n_tokens * top_k if x_per_pair else n_tokens
        xq = orc.quantize_q8_0(gs.activations(rows, k, cfg=701))
        offs, pairs = orc.moe_group(ids, n_experts)
        note("moe gemm shape", n_tokens, n_experts, top_k, n, k, x_per_pair)
        y = to_host(cq.cq_moe_gemm_grouped(FMT, to_dev(w), n_experts, n, k, to_dev(xq),
                                           x_per_pair, to_dev(offs), to_dev(pairs), n_tokens,
                                           top_k))
        y_ref, s_ref = orc.moe_matmul(FMT, w, n_experts, n, k, xq, x_per_pair, ids)
        assert_close_to_oracle(y, y_ref, s_ref, what="moe shape")


@pytest.mark.parametrize("n_tokens,n_experts,top_k,n,k", [(70, 8, 2, 200, 2048), (300, 4, 2, 2000, 1536),
                                                          (64, 300, 1, 100, 2048), (1, 32, 4, 1536, 2048),
                                                          (20, 3, 2, 8, 1536)])
def test_moe_gemm_whole_k_shapes(cq, orc, n_tokens, n_experts, top_k, n, k):
    """The whole-k Q4_K kernel (k of 8 or 6 super-blocks): n not a multiple
    of 16, several passes per expert (up to 150 tokens), two row groups per
    wave with a ragged last workgroup (n = 2000 at k = 1536), more experts
    than CUs with most of them empty, a single token, and fewer rows than
    one 16-row group (n = 8)."""
    w = gs.expert_weights(FMT, n_experts, n, k, cfg=740 + n_tokens, which=0)
    ids, _ = gs.routing(n_tokens, n_experts, top_k, cfg=740 + n_tokens)
    offs, pairs = orc.moe_group(ids, n_experts)
    for x_per_pair in (False, True):
        rows = n_tokens * top_k if x_per_pair else n_tokens
        xq = orc.quantize_q8_0(gs.activations(rows, k, cfg=741))
        note("moe gemm whole k", n_tokens, n_experts, top_k, n, k, x_per_pair)
        y = to_host(cq.cq_moe_gemm_grouped(FMT, to_dev(w), n_experts, n, k, to_dev(xq),
                                           x_per_pair, to_dev(offs), to_dev(pairs), n_tokens,
                                           top_k))
        y_ref, s_ref = orc.moe_matmul(FMT, w, n_experts, n, k, xq, x_per_pair, ids)
        assert_close_to_oracle(y, y_ref, s_ref, what="moe whole k")


@pytest.mark.parametrize("fmt", [gs.Q4_0, gs.Q4_1, gs.Q8_0, gs.Q5_K, gs.Q6_K], ids=lambda f: gs.NAMES[f])
@pytest.mark.parametrize("n_tokens,n_experts,top_k,n,k", [(40, 6, 2, 200, 512), (130, 3, 3, 70, 256)])
def test_moe_gemm_other_formats(cq, orc, fmt, n_tokens, n_experts, top_k, n, k):
    """Grouped GEMM over the 32-value formats (the dense tile engine over
    gathered rows): experts with more than one 64-token tile, n not a
    multiple of 128, per-token and per-pair activation rows."""
    w = gs.expert_weights(fmt, n_experts, n, k, cfg=720 + n_tokens, which=0)
    ids, _ = gs.routing(n_tokens, n_experts, top_k, cfg=720 + n_tokens)
    offs, pairs = orc.moe_group(ids, n_experts)
    for x_per_pair in (False, True):
        rows = n_tokens * top_k if x_per_pair else n_tokens
        xq = orc.quantize_q8_0(gs.activations(rows, k, cfg=721))
        note("moe gemm", gs.NAMES[fmt], n_tokens, n_experts, top_k, n, k, x_per_pair)
        y = to_host(cq.cq_moe_gemm_grouped(fmt, to_dev(w), n_experts, n, k, to_dev(xq),
                                           x_per_pair, to_dev(offs), to_dev(pairs), n_tokens,
                                           top_k))
        y_ref, s_ref = orc.moe_matmul(fmt, w, n_experts, n, k, xq, x_per_pair, ids)
        assert_close_to_oracle(y, y_ref, s_ref, what=f"moe {gs.NAMES[fmt]}")


@pytest.mark.parametrize("fmt", [gs.Q4_K, gs.Q8_0], ids=lambda f: gs.NAMES[f])
def test_moe_gemm_max_k(cq, orc, fmt):
    """k = CQ_MAX_K (65536): the streaming Q4_K kernel and the tile engine at
    their longest rows, per-token and per-pair activation rows."""
    n_tokens, n_experts, top_k, n, k = 9, 4, 2, 70, 65536
    w = gs.expert_weights(fmt, n_experts, n, k, cfg=730, which=0)
    ids, _ = gs.routing(n_tokens, n_experts, top_k, cfg=730)
    offs, pairs = orc.moe_group(ids, n_experts)
    for x_per_pair in (False, True):
        rows = n_tokens * top_k if x_per_pair else n_tokens
        xq = orc.quantize_q8_0(gs.activations(rows, k, cfg=731))
        note("moe gemm max k", gs.NAMES[fmt], x_per_pair)
        y = to_host(cq.cq_moe_gemm_grouped(fmt, to_dev(w), n_experts, n, k, to_dev(xq),
                                           x_per_pair, to_dev(offs), to_dev(pairs), n_tokens,
                                           top_k))
        y_ref, s_ref = orc.moe_matmul(fmt, w, n_experts, n, k, xq, x_per_pair, ids)
        assert_close_to_oracle(y, y_ref, s_ref, what=f"moe max k {gs.NAMES[fmt]}")
