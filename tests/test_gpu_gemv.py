"""GPU parity of the decode GEMV (cq_gemv) against the fp64 oracle:
|y - y_ref| <= 2e-5 * sum|w_hat*x_hat| per output, on small shapes that span
several row tiles with ragged tails, on the full workload shapes, and on the
invariants batch rows == single rows, determinism, power-of-two scaling and
row permutation (all bitwise)."""
import functools

import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import assert_close_to_oracle, note, to_dev, to_host

pytestmark = pytest.mark.gpu

FMTS = [gs.Q4_0, gs.Q4_1, gs.Q8_0, gs.Q4_K, gs.Q5_K, gs.Q6_K, gs.Q1_0, gs.TQ2]


def run_gemv(cq, fmt, w, n, k, xq, batch):
    return to_host(cq.cq_gemv(fmt, to_dev(w), n, k, to_dev(xq), batch))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
@pytest.mark.parametrize("n,k", [(1, 256), (37, 256), (130, 2048), (67, 4096), (9, 8192),
                                 (21, 352), (45, 1056), (11, 4160), (13, 5120), (70, 14336),
                                 (5, 16384), (3, 16416), (1, 8192), (3, 8192), (70, 8192)])
def test_gemv_small_shapes(cq, orc, fmt, n, k):
    if k % gs.BLOCK_ELEMS[fmt]:
        pytest.skip("k not a whole number of blocks for this type")
    w = gs.weights(fmt, n, k, cfg=200 + n)
    x = gs.activations(8, k, cfg=200 + n)
    xq = orc.quantize_q8_0(x)
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, 8)
    for batch in (1, 2, 5, 8):
        note("gemv", gs.NAMES[fmt], n, k, batch)
        y = run_gemv(cq, fmt, w, n, k, xq[:batch], batch)
        assert_close_to_oracle(y, y_ref[:batch], s_ref[:batch], what=f"{gs.NAMES[fmt]} b{batch}")


@functools.lru_cache(maxsize=2)
def config_inputs(name):
    c = gs.CONFIGS[name]
    w = gs.weights(c["fmt"], c["n"], c["k"], cfg=c["cfg"])
    x = gs.activations(max(c["batches"]), c["k"], cfg=c["cfg"])
    return c, w, x


@pytest.mark.parametrize("name", ["q4_0_gemv_2048", "q8_0_gemv_ffn_up", "q4_1_gemv_ffn_up",
                                  "q5_k_gemv_ffn_up", "q1_0_gemv_qkv", "tq2_gemv_70b_gate"])
def test_gemv_config_full(cq, orc, name):
    c, w, x = config_inputs(name)
    xq = orc.quantize_q8_0(x)
    B = max(c["batches"])
    y_ref, s_ref = orc.matmul(c["fmt"], w, c["n"], c["k"], xq, B)
    wd, xd = to_dev(w), to_dev(xq)
    for batch in c["batches"]:
        note("gemv config", name, batch)
        y = to_host(cq.cq_gemv(c["fmt"], wd, c["n"], c["k"], xd, batch))
        r = assert_close_to_oracle(y, y_ref[:batch], s_ref[:batch], what=f"{name} b{batch}")
        print(f"{name} batch {batch}: max |err|/S = {r:.3e}")


@pytest.mark.parametrize("name", ["q4_k_gemv_lm_head", "q6_k_gemv_lm_head"])
def test_gemv_lm_head_full(cq, orc, name):
    """LM head 128256 x 4096 (Q4_K; Q6_K, the tied-embedding type) at batch 1
    and 4: every output of both calls against the oracle, and each batch-4
    row equals the batch-1 call on that row bitwise."""
    c, w, x = config_inputs(name)
    n, k = c["n"], c["k"]
    xq = orc.quantize_q8_0(x)
    wd, xd = to_dev(w), to_dev(xq)
    note("gemv lm head b4", name)
    y4 = to_host(cq.cq_gemv(c["fmt"], wd, n, k, xd, 4))
    note("gemv lm head b1", name)
    y1 = to_host(cq.cq_gemv(c["fmt"], wd, n, k, xd, 1))
    y_ref, s_ref = orc.matmul(c["fmt"], w, n, k, xq, 4)
    r4 = assert_close_to_oracle(y4, y_ref, s_ref, what=f"{name} b4")
    r1 = assert_close_to_oracle(y1, y_ref[:1], s_ref[:1], what=f"{name} b1")
    print(f"{name}: max |err|/S = {r1:.3e} (batch 1), {r4:.3e} (batch 4)")
    assert np.array_equal(y4[0], y1[0])
    for b in range(1, 4):
        yb = to_host(cq.cq_gemv(c["fmt"], wd, n, k, xd[b:b + 1], 1))
        assert np.array_equal(yb[0], y4[b])


@pytest.mark.parametrize("k", [1024, 2048, 4096, 8192, 14336])
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
def test_gemv_batch_rows_equal_single_rows(cq, orc, fmt, k):
    """Row b of a verify batch is bitwise the batch-1 result on that row, for
    every batch size (the column split depends only on the type and k)."""
    if k % gs.BLOCK_ELEMS[fmt]:
        pytest.skip("k not a whole number of blocks for this type")
    n = 300
    w = gs.weights(fmt, n, k, cfg=300)
    xq = orc.quantize_q8_0(gs.activations(8, k, cfg=300))
    wd = to_dev(w)
    note("gemv batch invariance", gs.NAMES[fmt], k)
    y1 = [to_host(cq.cq_gemv(fmt, wd, n, k, to_dev(xq[b:b + 1]), 1))[0] for b in range(8)]
    for batch in (2, 3, 5, 8):
        yb = to_host(cq.cq_gemv(fmt, wd, n, k, to_dev(xq[:batch]), batch))
        for b in range(batch):
            assert np.array_equal(yb[b], y1[b]), (batch, b)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
def test_gemv_deterministic_and_scaling(cq, orc, fmt):
    n, k = 257, 2048
    w = gs.weights(fmt, n, k, cfg=301)
    xq = orc.quantize_q8_0(gs.activations(3, k, cfg=301))
    note("gemv determinism", gs.NAMES[fmt])
    y0 = run_gemv(cq, fmt, w, n, k, xq, 3)
    y1 = run_gemv(cq, fmt, w, n, k, xq, 3)
    assert np.array_equal(y0, y1)
    # doubling every weight scale (d, and m or dmin) doubles y bitwise
    w2 = w.copy().reshape(-1, gs.BLOCK_BYTES[fmt])
    offs = [208] if fmt == gs.Q6_K else [0, 2] if fmt in (gs.Q4_1, gs.Q4_K, gs.Q5_K) else [0]
    for o in offs:
        h = w2[:, o:o + 2].copy().view(np.float16)
        w2[:, o:o + 2] = (h * np.float16(2)).view(np.uint8)
    y2 = run_gemv(cq, fmt, w2.reshape(n, -1), n, k, xq, 3)
    assert np.array_equal(y2, 2 * y0)
    # permuting weight rows permutes y
    perm = np.random.default_rng(1).permutation(n)
    yp = run_gemv(cq, fmt, w[perm], n, k, xq, 3)
    assert np.array_equal(yp, y0[:, perm])


def test_gemv_strided_output(cq, orc):
    import torch
    fmt, n, k = gs.Q8_0, 100, 512
    w = gs.weights(fmt, n, k, cfg=302)
    xq = orc.quantize_q8_0(gs.activations(3, k, cfg=302))
    note("gemv strided y")
    y = torch.full((3, 160), -7.0, device="cuda")
    cq.cq_gemv(fmt, to_dev(w), n, k, to_dev(xq), 3, y=y, ldy=160)
    yh = to_host(y)
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, 3)
    assert_close_to_oracle(yh[:, :n], y_ref, s_ref, what="strided")
    assert np.all(yh[:, n:] == -7.0)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: gs.NAMES[f])
def test_gemv_long_rows_unaligned_and_strided(cq, orc, fmt):
    """Rows longer than one wave covers (k = 14336: the k-split streaming
    path) with the activations 2 bytes past a 16-byte boundary and a strided
    output: same values as the aligned call, bitwise, and within the oracle's
    bound; the columns past n keep their contents."""
    import torch
    n, k, B = 77, 14336, 3
    w = gs.weights(fmt, n, k, cfg=304)
    xq = orc.quantize_q8_0(gs.activations(B, k, cfg=304))
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, B)
    wd = to_dev(w)
    note("gemv long rows aligned", gs.NAMES[fmt])
    y0 = to_host(cq.cq_gemv(fmt, wd, n, k, to_dev(xq), B))
    assert_close_to_oracle(y0, y_ref, s_ref, what="long rows")
    buf = torch.zeros(xq.size + 16, dtype=torch.uint8, device="cuda")
    buf[2:2 + xq.size] = to_dev(xq.reshape(-1))
    xu = buf[2:2 + xq.size].view(B, -1)
    y = torch.full((B, 100), -7.0, device="cuda")
    note("gemv long rows unaligned strided", gs.NAMES[fmt])
    cq.cq_gemv(fmt, wd, n, k, xu, B, y=y, ldy=100)
    yh = to_host(y)
    assert np.array_equal(yh[:, :n], y0)
    assert np.all(yh[:, n:] == -7.0)


def test_gemv_zero_weights_exact(cq, orc):
    k = 1024
    w = gs.weights(gs.Q4_0, 64, k, cfg=303)
    w.reshape(-1, 18)[:, 2:] = 0x88
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=303))
    note("gemv zero weights")
    y = run_gemv(cq, gs.Q4_0, w, 64, k, xq, 2)
    assert not y.any()


@pytest.mark.parametrize("fmt", [gs.Q8_0, gs.Q4_K, gs.Q6_K, gs.Q1_0, gs.TQ2],
                         ids=lambda f: gs.NAMES[f])
def test_gemv_max_k(cq, orc, fmt):
    """k = CQ_GEMV_MAX_K (32768): the multi-wave kernel at its largest row
    (8 waves), with a ragged row count, at batch 1 and 8; one block more per
    row is refused."""
    n, k = 33, 32768
    w = gs.weights(fmt, n, k, cfg=310)
    xq = orc.quantize_q8_0(gs.activations(8, k, cfg=310))
    y_ref, s_ref = orc.matmul(fmt, w, n, k, xq, 8)
    wd, xd = to_dev(w), to_dev(xq)
    for batch in (1, 8):
        note("gemv max k", gs.NAMES[fmt], batch)
        y = to_host(cq.cq_gemv(fmt, wd, n, k, xd[:batch], batch))
        assert_close_to_oracle(y, y_ref[:batch], s_ref[:batch], what=f"max k b{batch}")
    k2 = k + gs.BLOCK_ELEMS[fmt] * (256 // gs.BLOCK_ELEMS[fmt] if gs.BLOCK_ELEMS[fmt] < 256 else 1)
    w2 = to_dev(gs.weights(fmt, 2, k2, cfg=311))
    x2 = to_dev(orc.quantize_q8_0(gs.activations(1, k2, cfg=311)))
    with pytest.raises(RuntimeError, match="SHAPE"):
        cq.cq_gemv(fmt, w2, 2, k2, x2, 1)


# Q4_K matrices with 4096-value rows and at least this many rows take the
# matrix-core kernel (integer dots on 4x4x4 int8 MFMA blocks)
MFMA_MIN_ROWS = 32768


@pytest.mark.parametrize("n", [MFMA_MIN_ROWS - 1, MFMA_MIN_ROWS, MFMA_MIN_ROWS + 3])
def test_gemv_q4k_matrix_core_path(cq, orc, n):
    """Every output against the oracle at batch 1 (each of 8 rows) and at
    batch 2, 3, 4, 5 and 8 (5..8: two 4-row launches), each batch row bitwise
    the batch-1 result; ragged row counts (not a multiple of the 4-row step),
    and the row count just below the switch (the streaming kernel)."""
    k = 4096
    w = gs.weights(gs.Q4_K, n, k, cfg=310 + n % 7)
    xq = orc.quantize_q8_0(gs.activations(8, k, cfg=310))
    y_ref, s_ref = orc.matmul(gs.Q4_K, w, n, k, xq, 8)
    wd = to_dev(w)
    note("gemv q4_k matrix-core path", n)
    y1 = [to_host(cq.cq_gemv(gs.Q4_K, wd, n, k, to_dev(xq[b:b + 1]), 1))[0] for b in range(8)]
    assert_close_to_oracle(np.stack(y1), y_ref, s_ref, what=f"q4_k n{n} b1")
    for batch in (2, 3, 4, 5, 8):
        yb = to_host(cq.cq_gemv(gs.Q4_K, wd, n, k, to_dev(xq[:batch]), batch))
        assert_close_to_oracle(yb, y_ref[:batch], s_ref[:batch], what=f"q4_k n{n} b{batch}")
        for b in range(batch):
            assert np.array_equal(yb[b], y1[b]), (batch, b)


def test_gemv_q4k_matrix_core_invariants(cq, orc):
    """On the matrix-core kernel: two runs bitwise equal, doubling every d and
    dmin doubles y bitwise, permuting weight rows permutes y, and a strided
    output leaves the columns past n alone."""
    import torch
    n, k = MFMA_MIN_ROWS + 6, 4096
    w = gs.weights(gs.Q4_K, n, k, cfg=311)
    xq = orc.quantize_q8_0(gs.activations(3, k, cfg=311))
    note("gemv q4_k matrix-core invariants")
    y0 = run_gemv(cq, gs.Q4_K, w, n, k, xq, 3)
    assert np.array_equal(y0, run_gemv(cq, gs.Q4_K, w, n, k, xq, 3))
    w2 = w.copy().reshape(-1, gs.BLOCK_BYTES[gs.Q4_K])
    for o in (0, 2):
        h = w2[:, o:o + 2].copy().view(np.float16)
        w2[:, o:o + 2] = (h * np.float16(2)).view(np.uint8)
    assert np.array_equal(run_gemv(cq, gs.Q4_K, w2.reshape(n, -1), n, k, xq, 3), 2 * y0)
    perm = np.random.default_rng(2).permutation(n)
    assert np.array_equal(run_gemv(cq, gs.Q4_K, w[perm], n, k, xq, 3), y0[:, perm])
    y = torch.full((3, n + 40), -7.0, device="cuda")
    cq.cq_gemv(gs.Q4_K, to_dev(w), n, k, to_dev(xq), 3, y=y, ldy=n + 40)
    yh = to_host(y)
    assert np.array_equal(yh[:, :n], y0)
    assert np.all(yh[:, n:] == -7.0)


def test_gemv_q4k_tall_unaligned_activations(cq, orc):
    """A tall Q4_K matrix with the activations 2 bytes past a 16-byte
    boundary (the streaming kernel): within the oracle's bound, and each batch
    row bitwise the batch-1 call on that row at the same alignment."""
    import torch
    n, k, B = MFMA_MIN_ROWS + 2, 4096, 4
    w = gs.weights(gs.Q4_K, n, k, cfg=312)
    xq = orc.quantize_q8_0(gs.activations(B, k, cfg=312))
    y_ref, s_ref = orc.matmul(gs.Q4_K, w, n, k, xq, B)
    wd = to_dev(w)
    buf = torch.zeros(xq.size + 16, dtype=torch.uint8, device="cuda")
    buf[2:2 + xq.size] = to_dev(xq.reshape(-1))
    xu = buf[2:2 + xq.size].view(B, -1)
    note("gemv q4_k tall unaligned")
    yb = to_host(cq.cq_gemv(gs.Q4_K, wd, n, k, xu, B))
    assert_close_to_oracle(yb, y_ref, s_ref, what="q4_k tall unaligned")
    for b in range(B):
        y1 = to_host(cq.cq_gemv(gs.Q4_K, wd, n, k, xu[b:b + 1], 1))
        assert np.array_equal(y1[0], yb[b]), b


def test_gemv_q4k_matrix_core_zeros_exact(cq, orc):
    """On the matrix-core kernel: weights whose 6-bit scales and mins are all
    zero (every weight exactly 0), and all-zero activations, give outputs
    that are exactly zero."""
    n, k = MFMA_MIN_ROWS + 1, 4096
    w = gs.weights(gs.Q4_K, n, k, cfg=313)
    wz = w.copy()
    wz.reshape(-1, gs.BLOCK_BYTES[gs.Q4_K])[:, 4:16] = 0
    xq = orc.quantize_q8_0(gs.activations(3, k, cfg=313))
    note("gemv q4_k matrix-core zero weights")
    assert not run_gemv(cq, gs.Q4_K, wz, n, k, xq, 3).any()
    x0 = orc.quantize_q8_0(np.zeros((3, k), dtype=np.float32))
    note("gemv q4_k matrix-core zero activations")
    assert not run_gemv(cq, gs.Q4_K, w, n, k, x0, 3).any()
