"""GPU parity of the Q8_0 activation quantizer and the SwiGLU requantizer:
bytes bit-exact against the oracle."""
import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import note, to_dev, to_host

pytestmark = pytest.mark.gpu


def q8(cq, x):
    return to_host(cq.cq_quantize_q8_0(to_dev(x)))


@pytest.mark.parametrize("rows,k", [(1, 2048), (5, 4096), (4, 4096), (3, 32), (7, 96),
                                    (512, 4096), (2048, 4096), (256, 2048), (2, 65536)])
def test_quantize_bit_exact(cq, orc, rows, k):
    note("quantize", rows, k)
    x = gs.activations(rows, k, cfg=100 + rows)
    assert np.array_equal(q8(cq, x), orc.quantize_q8_0(x))


def test_quantize_special_values(cq, orc):
    note("quantize special values")
    x = np.zeros((6, 64), np.float32)
    x[0, 0] = 127.0
    x[0, 1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5]     # exact ties
    x[1, 3], x[1, 9] = 1e-39, -5e-40                               # 127/amax overflows
    x[2] = np.float32(1e-30) * np.arange(64)                       # fp16 scale underflows
    x[3] = np.float32(3e4) * np.sin(np.arange(64))                 # large magnitudes
    x[4, 40] = -0.0                                                # negative zero
    x[5] = 1.0                                                     # constant row
    assert np.array_equal(q8(cq, x), orc.quantize_q8_0(x))


def test_quantize_scaled_grid(cq, orc):
    note("quantize scaled grid")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 1024)) * np.exp(rng.uniform(-30, 30, (64, 1)))).astype(np.float32)
    assert np.array_equal(q8(cq, x), orc.quantize_q8_0(x))


def test_quantize_strided_rows(cq, orc):
    import torch
    note("quantize strided rows")
    x = gs.activations(9, 320, cfg=7)
    xd = to_dev(x)[:, :256]          # row stride 320, k 256
    out = to_host(cq.cq_quantize_q8_0(xd))
    assert np.array_equal(out, orc.quantize_q8_0(x[:, :256]))
    torch.cuda.synchronize()


def test_swiglu_quantize(cq, orc):
    note("swiglu quantize")
    rows, k = 1024, 1536
    g = gs.activations(rows, k, cfg=40, tensor=5) * np.float32(3)
    u = gs.activations(rows, k, cfg=40, tensor=6)
    h, hq = cq.cq_swiglu_quantize_q8_0(to_dev(g), to_dev(u), want_h=True)
    h, hq = to_host(h), to_host(hq)
    h_ref = orc.swiglu(g, u)
    diff = h.view(np.int32).astype(np.int64) - h_ref.view(np.int32).astype(np.int64)
    # fp64 exp may differ in its last bit between the GPU and libm; after the
    # single rounding to fp32 that shows up (rarely) as a 1-ulp difference
    assert np.abs(diff).max() <= 1
    assert np.count_nonzero(diff) <= max(2, h.size // 100000)
    # the quantized bytes equal the oracle's wherever h matched bitwise; in a
    # block holding a 1-ulp difference each quant may move by at most one
    same_blocks = (diff.reshape(rows, k // 32, 32) == 0).all(axis=2)
    ref_q = orc.quantize_q8_0(h_ref).reshape(rows, k // 32, 34)
    got_q = hq.reshape(rows, k // 32, 34)
    assert np.array_equal(got_q[same_blocks], ref_q[same_blocks])
    qa = got_q[~same_blocks][:, 2:].view(np.int8).astype(np.int32)
    qb = ref_q[~same_blocks][:, 2:].view(np.int8).astype(np.int32)
    assert np.all(np.abs(qa - qb) <= 1)
    # without the optional h output the bytes are the same
    _, hq2 = cq.cq_swiglu_quantize_q8_0(to_dev(g), to_dev(u))
    assert np.array_equal(to_host(hq2), hq)
