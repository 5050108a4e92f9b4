"""Pins of the CPU oracle against things other than itself: hand-decoded
blocks, the block sizes the pages print, library fp16 conversions, closed
forms, invariants, exact rational brute force and a second, independent
formulation of the dot product.  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import gguf_synth as gs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")


def golden_blocks():
    with open(GOLDEN) as f:
        return json.load(f)["blocks"]


def q4k_golden_bytes(b):
    qs = bytearray(128)
    for c in range(4):
        for i in range(32):
            qs[32 * c + i] = (i % 16) | ((15 - i % 16) << 4)
    return bytes.fromhex(b["hex_header"]) + bytes.fromhex(b["scale_bytes_hex"]) + bytes(qs)


# --------------------------------------------------------------- block sizes
def test_block_sizes_match_pages(orc):
    # alice-llm 2.0.0 README, Quantization Block Specs: Q8_0 32 values / 34 B,
    # Q4_K 256 values / 144 B.  Q4_0 and Q4_1 sizes follow from the layout
    # reading (2 or 4 scale bytes + 16 nibble bytes).
    assert (orc.block_elems(orc.Q8_0), orc.block_bytes(orc.Q8_0)) == (32, 34)
    assert (orc.block_elems(orc.Q4_K), orc.block_bytes(orc.Q4_K)) == (256, 144)
    assert (orc.block_elems(orc.Q4_0), orc.block_bytes(orc.Q4_0)) == (32, 18)
    assert (orc.block_elems(orc.Q4_1), orc.block_bytes(orc.Q4_1)) == (32, 20)
    # bits per weight printed on the same table: 8.5 (Q8_0), 4.5 (Q4_K)
    assert 34 * 8 / 32 == 8.5 and 144 * 8 / 256 == 4.5
    # Q6_K: 256 values in 210 bytes (ql[128] + qh[64] + scales[16] + fp16 d),
    # 6.5625 bits per weight, same table
    assert (orc.block_elems(orc.Q6_K), orc.block_bytes(orc.Q6_K)) == (256, 210)
    assert 128 + 64 + 16 + 2 == 210 and 210 * 8 / 256 == 6.5625
    # Q5_K: 256 values in 176 bytes (d + dmin + scales[12] + qh[32] + qs[128]),
    # 5.5 bits per weight, same table
    assert (orc.block_elems(orc.Q5_K), orc.block_bytes(orc.Q5_K)) == (256, 176)
    assert 2 + 2 + 12 + 32 + 128 == 176 and 176 * 8 / 256 == 5.5
    # Q1_0 (Bonsai notes): 128 values in 18 bytes, 1.125 bits per weight
    assert (orc.block_elems(orc.Q1_0), orc.block_bytes(orc.Q1_0)) == (128, 18)
    assert 18 * 8 / 128 == 1.125
    assert orc.block_bytes(99) == -1


# ---------------------------------------------------------------------- fp16
def test_half_decode_exhaustive_vs_numpy(orc):
    h = np.arange(65536, dtype=np.uint16)
    ours = orc.half_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zeros
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_half_encode_sampled_vs_numpy(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.float_to_half(f), ref)
    # dense sweep of the range the quantizer uses (fp16 subnormal..normal)
    g = np.float32(np.linspace(0, 70000, 1_000_003, dtype=np.float64))
    g = np.concatenate([g, -g, np.float32(np.geomspace(1e-9, 1e-3, 200_000))])
    with np.errstate(over="ignore"):
        assert np.array_equal(orc.float_to_half(g), g.astype(np.float16).view(np.uint16))


def test_half_encode_closed_forms(orc):
    f2h = orc.lib().oracle_float_to_half
    assert f2h(1.0) == 0x3C00
    assert f2h(65504.0) == 0x7BFF
    assert f2h(65519.99) == 0x7BFF
    assert f2h(65520.0) == 0x7C00          # halfway, ties to even -> overflow
    assert f2h(2.0 ** -24) == 0x0001
    assert f2h(2.0 ** -25) == 0x0000       # halfway between 0 and 2^-24 -> even (0)
    assert f2h(3 * 2.0 ** -25) == 0x0002   # halfway between 1 and 2 quanta -> 2
    assert f2h(1.0 + 2.0 ** -11) == 0x3C00  # halfway -> even
    assert f2h(1.0 + 3 * 2.0 ** -11) == 0x3C02
    assert f2h(-0.0) == 0x8000


@pytest.mark.timeout(300)
def test_half_encode_exhaustive_vs_f16c(orc, tmp_path):
    """All 2^32 fp32 encodings against the host's F16C conversion."""
    src = os.path.join(os.path.dirname(__file__), "native", "fp16_exhaustive.cpp")
    exe = tmp_path / "fp16_exhaustive"
    from oracle import build
    import subprocess
    subprocess.run(["g++", "-O2", "-mf16c", "-std=c++17", "-pthread", src, "-o", str(exe),
                    "-ldl"], check=True)
    r = subprocess.run([str(exe), build.LIB], capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


# ------------------------------------------------------- hand-decoded blocks
@pytest.mark.parametrize("blk", golden_blocks(), ids=lambda b: b["name"])
def test_golden_block_decodes(orc, blk):
    t = gs.FORMATS[blk["format"]]
    if t == gs.Q4_K:
        raw = np.frombuffer(q4k_golden_bytes(blk), np.uint8)
        for j in range(8):
            assert orc.q4k_scale_min(raw[4:16], j) == (blk["sc"][j], blk["m"][j])
        exp = np.empty(256)
        for c in range(4):
            for i in range(32):
                j0, j1 = 2 * c, 2 * c + 1
                exp[64 * c + i] = blk["d"] * blk["sc"][j0] * (i % 16) - blk["dmin"] * blk["m"][j0]
                exp[64 * c + 32 + i] = (blk["d"] * blk["sc"][j1] * (15 - i % 16)
                                        - blk["dmin"] * blk["m"][j1])
        assert np.array_equal(orc.dequantize(t, raw, 256), exp)
        return
    raw = np.frombuffer(bytes.fromhex(blk["hex"]), np.uint8)
    assert raw.size == gs.BLOCK_BYTES[t]
    got = orc.dequantize(t, raw, gs.BLOCK_ELEMS[t])
    if "expected" in blk:
        assert np.array_equal(got, np.array(blk["expected"], np.float64))
    else:
        exp = blk["expected_scale"] * np.array(blk["expected_q"], np.float64)
        assert np.array_equal(got, exp)


# ------------------------------------------------------------- the quantizer
def test_quantize_zero_block(orc):
    out = orc.quantize_q8_0(np.zeros((1, 64), np.float32))
    assert not out.any()


def test_quantize_ties_round_to_even(orc):
    # amax = 127 -> 127/amax = 1 exactly, so each q is rint(x) and d = 1.0
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5]
    out = orc.quantize_q8_0(x)[0]
    assert int(out[0]) | (int(out[1]) << 8) == 0x3C00
    q = out[2:].view(np.int8)
    assert list(q[:9]) == [127, 2, 4, -2, -4, 0, 2, 0, 126]
    assert not q[9:].any()


def test_quantize_exact_grid(orc):
    # x = i (integers), amax 127 -> q = x exactly; d = 1
    x = np.arange(-15, 17, dtype=np.float32)
    x[0] = -127.0
    out = orc.quantize_q8_0(x)[0]
    assert list(out[2:].view(np.int8)) == list(x.astype(np.int64))


def test_quantize_power_of_two_scaling(orc):
    x = gs.activations(4, 256, cfg=900)
    base = orc.quantize_q8_0(x)
    for j in (-6, -1, 1, 5):
        sc = orc.quantize_q8_0(x * np.float32(2.0 ** j))
        bq = base.reshape(-1, 34)
        sq = sc.reshape(-1, 34)
        assert np.array_equal(sq[:, 2:], bq[:, 2:])
        d0 = orc.half_to_double(bq[:, :2].copy().view(np.uint16).ravel())
        d1 = orc.half_to_double(sq[:, :2].copy().view(np.uint16).ravel())
        assert np.array_equal(d1, d0 * 2.0 ** j)


def test_quantize_sign_symmetry(orc):
    x = gs.activations(3, 128, cfg=901)
    a = orc.quantize_q8_0(x).reshape(-1, 34)
    b = orc.quantize_q8_0(-x).reshape(-1, 34)
    assert np.array_equal(a[:, :2], b[:, :2])
    assert np.array_equal(a[:, 2:].view(np.int8), -(b[:, 2:].view(np.int8)))


def test_quantize_scale_closed_form(orc):
    # amax = 127 * 2^j gives d = 2^j exactly
    for j in (-20, -3, 0, 4):
        x = np.full(32, 0.25 * 2.0 ** j, np.float32)
        x[7] = -127.0 * 2.0 ** j
        out = orc.quantize_q8_0(x)[0]
        d = orc.half_to_double(out[:2].copy().view(np.uint16))[0]
        assert d == 2.0 ** j
        assert out[2 + 7].view(np.int8) == -127


def test_quantize_spike(orc):
    x = np.full(32, 1e-3, np.float32)
    x[5] = 1000.0
    q = orc.quantize_q8_0(x)[0][2:].view(np.int8)
    assert q[5] == 127 and not np.delete(q, 5).any()


def test_quantize_tiny_amax_overflowing_reciprocal(orc):
    # 127/amax overflows fp32 -> zeros stay 0, others saturate, d rounds to 0
    x = np.zeros(32, np.float32)
    x[3] = 1e-39
    x[9] = -5e-40
    out = orc.quantize_q8_0(x)[0]
    q = out[2:].view(np.int8)
    assert out[0] == 0 and out[1] == 0
    assert q[3] == 127 and q[9] == -127
    assert not np.delete(q, [3, 9]).any()


def test_quantize_dequant_error_bound(orc):
    # |x - d*q| <= d/2 * (1 + tiny) for every element (round to nearest)
    x = gs.activations(8, 1024, cfg=902)
    out = orc.quantize_q8_0(x)
    xh = np.stack([orc.dequantize(gs.Q8_0, out[i], 1024) for i in range(8)])
    d = orc.half_to_double(out.reshape(-1, 34)[:, :2].copy().view(np.uint16).ravel())
    dd = np.repeat(d, 32).reshape(8, 1024)
    # the fp16 scale is within 2^-11 relative of amax/127; quants within 0.5
    amax = np.abs(x.reshape(-1, 32)).max(axis=1).repeat(32).reshape(8, 1024)
    assert np.all(np.abs(xh - x) <= 0.5 * dd + 127 * np.abs(dd - amax / 127) + 1e-12)


def _f32(r):
    """The fp32 value nearest to the rational r (ties to even), normal range:
    the rounding of one IEEE single-precision operation."""
    if r == 0:
        return Fraction(0)
    sign, a = (-1, -r) if r < 0 else (1, r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def _rne_q(v):
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return max(-127, min(127, fl))


def test_quantize_fp32_reciprocal_multiply(orc):
    # The page's recipe (alice-llm 2.0.0 README, "The CPU Optimization
    # Journey", Phase 4) takes scale = 127/amax as one fp32 value and then
    # one fp32 multiply per element before rounding.  Near a half-integer
    # that differs from dividing by the fp32 amax/127 and from the exact
    # x*127/amax; elements placed there (found here with exact rationals,
    # every step rounded to fp32 as the page's code does) must quantize to
    # the page's value.
    rng = np.random.default_rng(20261203)
    cases, diff_div, diff_exact = [], 0, 0
    while len(cases) < 96 or diff_div < 8 or diff_exact < 8:
        amax = np.float32(rng.uniform(0.5, 8.0))
        A = Fraction(float(amax))
        inv = _f32(Fraction(127) / A)
        q = int(rng.integers(-126, 126))
        x = np.float32(float((Fraction(q) + Fraction(1, 2)) / inv))
        x = x if rng.integers(2) else np.nextafter(x, np.float32(np.inf))
        if not abs(x) < amax:
            continue
        X = Fraction(float(x))
        page = _rne_q(_f32(X * inv))
        div = _rne_q(_f32(X / _f32(A / 127)))
        exact = _rne_q(X * 127 / A)
        if page != div or page != exact:
            cases.append((amax, x, page))
            diff_div += page != div
            diff_exact += page != exact
    blocks = np.zeros((len(cases), 32), np.float32)
    for i, (amax, x, _) in enumerate(cases):
        blocks[i, 0] = amax
        blocks[i, 1 + i % 31] = x
    out = orc.quantize_q8_0(blocks.reshape(1, -1)).reshape(-1, 34)
    for i, (amax, x, page) in enumerate(cases):
        q = out[i, 2:].view(np.int8)
        assert q[0] == 127
        assert int(q[1 + i % 31]) == page, (float(amax), float(x), page, int(q[1 + i % 31]))
        d16 = int(out[i, 0]) | (int(out[i, 1]) << 8)
        assert d16 == int(np.float16(np.float32(amax) / np.float32(127)).view(np.uint16))


# ------------------------------------------------------- matmul formulations
def one_hot_rows(k, cols, value=3.0):
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = value if i % 2 == 0 else -value
    return x


@pytest.mark.parametrize("fmt", [gs.Q4_0, gs.Q4_1, gs.Q8_0, gs.Q4_K])
def test_column_extraction(orc, fmt):
    """One-hot x quantizes to a single +-127 with d = fp16(|c|/127), so y
    reads one dequantized weight column times 127*d."""
    n, k = 5, 512
    w = gs.weights(fmt, n, k, cfg=910)
    cols = list(range(0, k, 37))
    x = one_hot_rows(k, cols)
    xq = orc.quantize_q8_0(x)
    y, s = orc.matmul(fmt, w, n, k, xq, len(cols))
    wd = np.stack([orc.dequantize(fmt, w[r], k) for r in range(n)])
    d = orc.half_to_double(np.array([orc.lib().oracle_float_to_half(np.float32(3.0) / np.float32(127.0))], np.uint16))[0]
    for i, c in enumerate(cols):
        sign = 1.0 if i % 2 == 0 else -1.0
        assert np.array_equal(y[i], sign * 127 * d * wd[:, c])
        assert np.array_equal(s[i], np.abs(127 * d * wd[:, c]))


def test_zero_weights_give_zero(orc):
    k = 256
    x = gs.activations(3, k, cfg=911)
    xq = orc.quantize_q8_0(x)
    w0 = gs.weights(gs.Q4_0, 4, k, cfg=911)
    w0.reshape(-1, 18)[:, 2:] = 0x88                  # every q = 8
    y, _ = orc.matmul(gs.Q4_0, w0, 4, k, xq, 3)
    assert not y.any()
    wk = gs.weights(gs.Q4_K, 4, k, cfg=911)
    wk.reshape(-1, 144)[:, 4:16] = 0                 # all scales and mins 0
    y, _ = orc.matmul(gs.Q4_K, wk, 4, k, xq, 3)
    assert not y.any()


def test_constant_q8_0_closed_form(orc):
    k = 1024
    w = np.zeros((2, k // 32, 34), np.uint8)
    w[:, :, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    w[:, :, 2:] = 1
    xq = orc.quantize_q8_0(np.ones((1, k), np.float32))
    y, s = orc.matmul(gs.Q8_0, w.reshape(2, -1), 2, k, xq, 1)
    d = float(np.float16(np.float32(1.0) / np.float32(127.0)))
    assert np.all(y == k * 127 * d) and np.all(s == k * 127 * d)


def test_cross_format_identities(orc):
    """Q4_0(d, q) == Q8_0(d, q-8) == Q4_1(d, -8d, q) exactly."""
    n, k = 6, 512
    w40 = gs.weights(gs.Q4_0, n, k, cfg=912).reshape(-1, 18)
    nb = w40.shape[0]
    w80 = np.zeros((nb, 34), np.uint8)
    w41 = np.zeros((nb, 20), np.uint8)
    w80[:, :2] = w40[:, :2]
    lo = (w40[:, 2:] & 0x0F).astype(np.int16) - 8
    hi = (w40[:, 2:] >> 4).astype(np.int16) - 8
    w80[:, 2:18] = lo.astype(np.int8).view(np.uint8)
    w80[:, 18:34] = hi.astype(np.int8).view(np.uint8)
    d = w40[:, :2].copy().view(np.float16).ravel()
    w41[:, :2] = w40[:, :2]
    w41[:, 2:4] = (-8 * d.astype(np.float32)).astype(np.float16).view(np.uint8).reshape(-1, 2)
    w41[:, 4:] = w40[:, 2:]
    xq = orc.quantize_q8_0(gs.activations(3, k, cfg=912))
    y0, _ = orc.matmul(gs.Q4_0, w40.reshape(n, -1), n, k, xq, 3)
    y8, _ = orc.matmul(gs.Q8_0, w80.reshape(n, -1), n, k, xq, 3)
    y1, _ = orc.matmul(gs.Q4_1, w41.reshape(n, -1), n, k, xq, 3)
    assert np.array_equal(y0, y8) and np.array_equal(y0, y1)


def test_q4k_subblock_equals_q4_1(orc):
    """A Q4_K sub-block with d*sc and dmin*m exact in fp16 equals the Q4_1
    block (d*sc, -dmin*m) over the same nibbles."""
    k = 256
    wk = gs.weights(gs.Q4_K, 3, k, cfg=913).reshape(-1, 144)
    wk[:, 0:2] = np.frombuffer(np.float16(2.0 ** -8).tobytes(), np.uint8)
    wk[:, 2:4] = np.frombuffer(np.float16(2.0 ** -9).tobytes(), np.uint8)
    w41 = np.zeros((wk.shape[0] * 8, 20), np.uint8).reshape(-1, 8, 20)
    for r in range(wk.shape[0]):
        for j in range(8):
            sc, mn = orc.q4k_scale_min(wk[r, 4:16], j)
            c = j // 2
            q = (wk[r, 16 + 32 * c: 48 + 32 * c] & 0x0F) if j % 2 == 0 else (wk[r, 16 + 32 * c: 48 + 32 * c] >> 4)
            w41[r, j, 0:2] = np.frombuffer(np.float16(2.0 ** -8 * sc).tobytes(), np.uint8)
            w41[r, j, 2:4] = np.frombuffer(np.float16(-(2.0 ** -9) * mn).tobytes(), np.uint8)
            w41[r, j, 4:] = q[:16] | (q[16:] << 4)
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=913))
    yk, _ = orc.matmul(gs.Q4_K, wk.reshape(3, -1), 3, k, xq, 2)
    y1, _ = orc.matmul(gs.Q4_1, w41.reshape(3, -1), 3, k, xq, 2)
    assert np.array_equal(yk, y1)


@pytest.mark.parametrize("fmt", [gs.Q4_0, gs.Q4_1, gs.Q8_0, gs.Q4_K, gs.Q5_K, gs.Q6_K, gs.Q1_0,
                                 gs.TQ2])
def test_two_formulations_agree(orc, fmt):
    n, m, k = 33, 5, 1024
    w = gs.weights(fmt, n, k, cfg=914)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=914))
    y, s = orc.matmul(fmt, w, n, k, xq, m)
    yf = orc.matmul_factored(fmt, w, n, k, xq, m)
    assert np.all(np.abs(y - yf) <= 1e-14 * s)
    # sampled variant agrees exactly with the full product
    ai = np.array([0, 4, 2, 1, 3]); ri = np.array([0, 32, 17, 5, 31])
    ys, ss = orc.matmul_sampled(fmt, w, n, k, xq, m, ai, ri)
    assert np.array_equal(ys, y[ai, ri]) and np.array_equal(ss, s[ai, ri])


@pytest.mark.parametrize("fmt,k", [(gs.Q4_0, 32), (gs.Q4_1, 64), (gs.Q8_0, 96), (gs.Q4_K, 256),
                                   (gs.Q4_K, 512), (gs.Q5_K, 256), (gs.Q6_K, 256),
                                   (gs.Q1_0, 128), (gs.Q1_0, 384), (gs.TQ2, 128), (gs.TQ2, 384)])
def test_exact_rational_brute_force(orc, fmt, k):
    """Tiny shapes in exact rational arithmetic: the fp64 sums must agree
    with the exact value to within the fp64 summation bound."""
    n, m = 3, 2
    w = gs.weights(fmt, n, k, cfg=915)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=915))
    y, s = orc.matmul(fmt, w, n, k, xq, m)
    wd = [[Fraction(v) for v in orc.dequantize(fmt, w[r], k)] for r in range(n)]
    xd = [[Fraction(v) for v in orc.dequantize(gs.Q8_0, xq[i], k)] for i in range(m)]
    for i in range(m):
        for r in range(n):
            exact = sum(a * b for a, b in zip(wd[r], xd[i]))
            mag = sum(abs(a * b) for a, b in zip(wd[r], xd[i]))
            assert abs(Fraction(y[i, r]) - exact) <= Fraction(k) * Fraction(2.0 ** -53) * mag
            assert Fraction(s[i, r]) == pytest.approx(mag, rel=1e-15) or abs(Fraction(s[i, r]) - mag) <= Fraction(k) * Fraction(2.0 ** -53) * mag


def test_dequantize_matches_library_matmul(orc):
    """y = W_hat @ X_hat^T computed with numpy's matmul on the decoded values."""
    fmt, n, m, k = gs.Q4_K, 7, 3, 512
    w = gs.weights(fmt, n, k, cfg=916)
    xq = orc.quantize_q8_0(gs.activations(m, k, cfg=916))
    y, s = orc.matmul(fmt, w, n, k, xq, m)
    wd = np.stack([orc.dequantize(fmt, w[r], k) for r in range(n)])
    xd = np.stack([orc.dequantize(gs.Q8_0, xq[i], k) for i in range(m)])
    assert np.allclose(y, xd @ wd.T, rtol=0, atol=1e-13 * s.max())
    assert np.allclose(s, np.abs(xd) @ np.abs(wd).T, rtol=1e-13)


# ------------------------------------------------------------------- SwiGLU
def test_swiglu_closed_forms(orc):
    g = np.array([0.0, 100.0, -100.0, math.log(3.0), 1.0], np.float32)
    u = np.array([5.0, 0.5, 2.0, 1.0, -3.0], np.float32)
    h = orc.swiglu(g, u)
    assert h[0] == 0.0
    assert h[1] == np.float32(50.0)
    assert abs(h[2]) < 1e-40
    z = float(np.float32(math.log(3.0)))
    assert h[3] == np.float32(z / (1 + math.exp(-z)))
    assert abs(float(h[3]) - 0.75 * math.log(3.0)) < 1e-6
    sig1 = 1.0 / (1.0 + math.exp(-1.0))
    assert h[4] == np.float32(-3.0 * sig1)


def test_swiglu_odd_part_identity(orc):
    """silu(z) - silu(-z) = z."""
    g = gs.activations(1, 4096, cfg=917).ravel() * np.float32(4)
    one = np.ones_like(g)
    d = orc.swiglu(g, one).astype(np.float64) - orc.swiglu(-g, one).astype(np.float64)
    assert np.all(np.abs(d - g) <= 2 * np.abs(g) * 2.0 ** -23 + 1e-30)


# ---------------------------------------------------------------------- MoE
def test_moe_group_vs_stable_argsort(orc):
    ids, _ = gs.routing(256, 32, 4, cfg=920)
    offs, pairs = orc.moe_group(ids, 32)
    flat = ids.ravel()
    assert np.array_equal(pairs, np.argsort(flat, kind="stable"))
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=32))]))


def test_moe_group_rejects_bad_id(orc):
    ids = np.zeros((2, 2), np.int32)
    ids[1, 1] = 32
    with pytest.raises(ValueError):
        orc.moe_group(ids, 32)


def test_moe_reduces_to_dense(orc):
    """All tokens routed to the same experts: each slot is a dense matmul."""
    fmt, E, n, k, T, K = gs.Q4_K, 4, 16, 256, 5, 2
    w = gs.expert_weights(fmt, E, n, k, cfg=921, which=0)
    xq = orc.quantize_q8_0(gs.activations(T, k, cfg=921))
    ids = np.tile(np.array([[2, 0]], np.int32), (T, 1))
    y, s = orc.moe_matmul(fmt, w, E, n, k, xq, False, ids)
    rb = k // 256 * 144
    for slot, e in enumerate([2, 0]):
        yd, sd = orc.matmul(fmt, w[e * n:(e + 1) * n], n, k, xq, T)
        assert np.array_equal(y[slot::K], yd) and np.array_equal(s[slot::K], sd)
    assert rb == w.shape[1]


def test_moe_combine_vs_numpy(orc):
    rng = np.random.default_rng(3)
    T, K, n = 6, 4, 10
    d = rng.standard_normal((T * K, n))
    _, rw = gs.routing(T, 32, K, cfg=922)
    y, s = orc.moe_combine(d, np.abs(d), rw)
    ref = np.einsum("tk,tkn->tn", rw.astype(np.float64), d.reshape(T, K, n))
    assert np.allclose(y, ref, rtol=1e-15, atol=1e-15)
    assert np.allclose(s, np.einsum("tk,tkn->tn", np.abs(rw.astype(np.float64)),
                                    np.abs(d).reshape(T, K, n)), rtol=1e-15)


# ------------------------------------------------------------------- Q6_K
# alice-llm 2.0.0 README, Quantization Block Specs: Q6_K = ql[128] + qh[64]
# + scales[16] + d(f16), 210 bytes for 256 values.  NEON matvec design notes:
# the four quadrants take their high bits from qh through (qh<<4)&0x30,
# (qh<<2)&0x30, qh&0x30 and (qh>>2)&0x30.  Reading (GGUF): in half h, element
# l + 32g (l < 32) takes a nibble of ql[64h + l] (g = 0, 2: low, high) or
# ql[64h + 32 + l] (g = 1, 3), scale byte 8h + 2g + l/16 (signed), value
# d*scale*(q-32).

def _q6k_block(d=1.0, ql=None, qh=None, scales=None):
    b = np.zeros(210, np.uint8)
    if ql is not None:
        b[0:128] = ql
    if qh is not None:
        b[128:192] = qh
    if scales is not None:
        b[192:208] = np.asarray(scales, np.int8).view(np.uint8)
    b[208:210] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    return b


def test_q6k_field_offsets(orc):
    """d sits in the last two bytes, the signed scales in bytes 192..207:
    with all quants 33 (ql low nibbles 1, qh bit pairs 2 -> q-32 = 1 in
    quadrants 0 and 1), each element equals d times its group's scale."""
    ql = np.full(128, 0x01, np.uint8)          # low nibble 1, high nibble 0
    qh = np.full(64, 0b0000_1010, np.uint8)    # quadrants 0, 1: high bits 2 -> q = 33
    scales = np.arange(-8, 8)
    v = orc.dequantize(gs.Q6_K, _q6k_block(0.5, ql, qh, scales), 256)
    for h in range(2):
        for g in range(2):                     # quadrants with q = 33
            for l in range(32):
                assert v[128 * h + 32 * g + l] == 0.5 * scales[8 * h + 2 * g + l // 16]
        for g in range(2, 4):                  # high nibble 0, high bits 0: q = 0
            for l in range(32):
                assert v[128 * h + 32 * g + l] == 0.5 * scales[8 * h + 2 * g + l // 16] * -32


@pytest.mark.parametrize("quad", range(4))
def test_q6k_high_bits_follow_the_page_shift_masks(orc, quad):
    """qh byte l carries quadrant 0..3's high bit pairs in bits 0-1, 2-3,
    4-5, 6-7: the page's four shift-masks place them at bits 4-5 of q."""
    shift_mask = [lambda x: (x << 4) & 0x30, lambda x: (x << 2) & 0x30,
                  lambda x: x & 0x30, lambda x: (x >> 2) & 0x30][quad]
    qh = np.zeros(64, np.uint8)
    qh[5] = 0b11 << (2 * quad)                 # half 0, l = 5: high bits 3
    ql = np.zeros(128, np.uint8)
    v = orc.dequantize(gs.Q6_K, _q6k_block(1.0, ql, qh, np.ones(16)), 256)
    q = v + 32                                 # d = 1, every scale 1
    assert shift_mask(int(qh[5])) == 0x30
    assert q[32 * quad + 5] == 0x30            # bits 4-5 set, nibble 0
    q[32 * quad + 5] = 0
    assert not q.any()                         # no other element moved


def test_q6k_nibble_quadrants(orc):
    """ql[l] low/high nibble -> quadrants 0/2, ql[32 + l] -> quadrants 1/3, in
    each half; qh all zero, d = 1, scales 1."""
    ql = np.zeros(128, np.uint8)
    ql[3] = 0x5A           # half 0: l = 3, quadrant 0 gets 0xA, quadrant 2 gets 0x5
    ql[32 + 7] = 0xC3      # half 0: l = 7, quadrant 1 gets 0x3, quadrant 3 gets 0xC
    ql[64 + 31] = 0x1F     # half 1: l = 31, quadrant 0 gets 0xF, quadrant 2 gets 0x1
    v = orc.dequantize(gs.Q6_K, _q6k_block(1.0, ql, None, np.ones(16)), 256) + 32
    exp = np.zeros(256)
    exp[0 + 3], exp[64 + 3] = 0xA, 0x5
    exp[32 + 7], exp[96 + 7] = 0x3, 0xC
    exp[128 + 31], exp[128 + 64 + 31] = 0xF, 0x1
    assert np.array_equal(v, exp)


def test_q6k_equals_q8_0(orc):
    """A Q6_K row whose d*scale is exact in fp16 equals the Q8_0 row with
    block scale d*scale per 16-value group (each Q8_0 block split in two
    groups of equal scale) and quants q-32: built here from the bit fields
    directly, not through the decoder."""
    k, n = 512, 3
    w6 = gs.weights(gs.Q6_K, n, k, cfg=915).reshape(-1, 210)
    # equal scales within each 32-value quadrant (both 16-groups), d = 2^-10
    sc = w6[:, 192:208].view(np.int8).copy()
    sc[:, 1::2] = sc[:, 0::2]
    w6[:, 192:208] = sc.view(np.uint8)
    w6[:, 208:210] = np.frombuffer(np.float16(2.0 ** -10).tobytes(), np.uint8)
    w8 = np.zeros((w6.shape[0], 8, 34), np.uint8)
    for r in range(w6.shape[0]):
        ql, qh = w6[r, 0:128].astype(np.int32), w6[r, 128:192].astype(np.int32)
        for h in range(2):
            for g in range(4):
                lb = ql[64 * h + (32 if g % 2 else 0): 64 * h + (32 if g % 2 else 0) + 32]
                low = (lb & 0x0F) if g < 2 else (lb >> 4)
                high = (qh[32 * h: 32 * h + 32] >> (2 * g)) & 3
                q = (low | (high << 4)) - 32
                s_ = int(sc[r, 8 * h + 2 * g])
                w8[r, 4 * h + g, 0:2] = np.frombuffer(np.float16(2.0 ** -10 * s_).tobytes(), np.uint8)
                w8[r, 4 * h + g, 2:] = q.astype(np.int8).view(np.uint8)
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=915))
    y6, _ = orc.matmul(gs.Q6_K, w6.reshape(n, -1), n, k, xq, 2)
    y8, _ = orc.matmul(gs.Q8_0, w8.reshape(n, -1), n, k, xq, 2)
    assert np.array_equal(y6, y8)


def test_q6k_scale_sign_and_d(orc):
    """Negating every scale byte negates the row; doubling d doubles it."""
    k, n = 512, 4
    w = gs.weights(gs.Q6_K, n, k, cfg=916).reshape(-1, 210)
    sc = w[:, 192:208].view(np.int8)
    keep = sc != -128                       # -(-128) does not fit in int8
    sc[~keep] = 0
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=916))
    y0, _ = orc.matmul(gs.Q6_K, w.reshape(n, -1), n, k, xq, 2)
    wn = w.copy(); wn[:, 192:208] = (-sc).view(np.uint8)
    yn, _ = orc.matmul(gs.Q6_K, wn.reshape(n, -1), n, k, xq, 2)
    assert np.array_equal(yn, -y0)
    w2 = w.copy()
    d = w2[:, 208:210].copy().view(np.float16)
    w2[:, 208:210] = (d * np.float16(2)).view(np.uint8)
    y2, _ = orc.matmul(gs.Q6_K, w2.reshape(n, -1), n, k, xq, 2)
    assert np.array_equal(y2, 2 * y0)


# ------------------------------------------------------------------- Q5_K
# alice-llm 2.0.0 README, Quantization Block Specs: Q5_K = d (fp16) + dmin
# (fp16) + scales[12] + qh[32] + qs[128], 176 bytes for 256 values.  Reading:
# d, dmin, scales and the qs nibbles as in Q4_K; bit j of qh[l] is bit 4 of
# element l of sub-block j; value d*sc*q - dmin*m with q in 0..31.

def _q5k_from_q4k(wk, qh=None):
    """Q5_K blocks carrying the fields of Q4_K blocks wk ([nb][144]) and the
    given qh bytes ([nb][32], default zeros)."""
    nb = wk.shape[0]
    w5 = np.zeros((nb, 176), np.uint8)
    w5[:, 0:16] = wk[:, 0:16]
    w5[:, 16:48] = 0 if qh is None else qh
    w5[:, 48:176] = wk[:, 16:144]
    return w5


def test_q5k_without_high_bits_is_q4k(orc):
    """With qh all zero every element decodes exactly as the Q4_K block with
    the same d, dmin, scales and qs: pins the offsets of d, dmin, the scale
    bytes and qs (byte 48) against the pinned Q4_K decode."""
    wk = gs.weights(gs.Q4_K, 1, 2048, cfg=920).reshape(-1, 144)
    w5 = _q5k_from_q4k(wk)
    for b in range(wk.shape[0]):
        assert np.array_equal(orc.dequantize(gs.Q5_K, w5[b], 256), orc.dequantize(gs.Q4_K, wk[b], 256))


@pytest.mark.parametrize("j", range(8))
def test_q5k_high_bit_one_hot(orc, j):
    """Setting bit j of qh[l] raises exactly element 32*j + l, by 16*d*sc_j
    (the fifth bit of that quant), and nothing else."""
    wk = gs.weights(gs.Q4_K, 1, 256, cfg=921 + j).reshape(-1, 144)
    d = float(np.frombuffer(wk[0, 0:2].tobytes(), np.float16)[0])
    sc, _ = orc.q4k_scale_min(wk[0, 4:16], j)
    base = orc.dequantize(gs.Q5_K, _q5k_from_q4k(wk)[0], 256)
    for l in (0, 1, 7, 16, 30, 31):
        qh = np.zeros((1, 32), np.uint8)
        qh[0, l] = 1 << j
        v = orc.dequantize(gs.Q5_K, _q5k_from_q4k(wk, qh)[0], 256)
        diff = v - base
        assert np.count_nonzero(diff) == (1 if sc else 0)
        assert diff[32 * j + l] == 16 * d * sc


def test_q5k_high_bits_add(orc):
    """The high bits of all elements act independently: with every qh bit
    set, each element is its Q4_K value plus 16*d*sc of its sub-block."""
    wk = gs.weights(gs.Q4_K, 1, 512, cfg=930).reshape(-1, 144)
    for b in range(wk.shape[0]):
        d = float(np.frombuffer(wk[b, 0:2].tobytes(), np.float16)[0])
        v4 = orc.dequantize(gs.Q4_K, wk[b], 256)
        v5 = orc.dequantize(gs.Q5_K, _q5k_from_q4k(wk[b:b + 1], np.full((1, 32), 255, np.uint8))[0], 256)
        for j in range(8):
            sc, _ = orc.q4k_scale_min(wk[b, 4:16], j)
            assert np.array_equal(v5[32 * j: 32 * j + 32], v4[32 * j: 32 * j + 32] + 16 * d * sc)


def test_q5k_matmul_equals_q4k_plus_high_part(orc):
    """y over a Q5_K row = y over its Q4_K part + y over the Q8_0 row whose
    quants are 16 at the set qh bits, scale d*sc (exact: d = 2^-8, dmin
    any), built block by block from the qh bits alone."""
    n, k = 3, 512
    wk = gs.weights(gs.Q4_K, n, k, cfg=931).reshape(-1, 144)
    wk[:, 0:2] = np.frombuffer(np.float16(2.0 ** -8).tobytes(), np.uint8)
    qh = gs.rng(931, 5).integers(0, 256, size=(wk.shape[0], 32), dtype=np.uint8)
    w5 = _q5k_from_q4k(wk, qh)
    w8 = np.zeros((wk.shape[0] * 8, 34), np.uint8)
    for b in range(wk.shape[0]):
        for j in range(8):
            sc, _ = orc.q4k_scale_min(wk[b, 4:16], j)
            w8[8 * b + j, 0:2] = np.frombuffer(np.float16(2.0 ** -8 * sc).tobytes(), np.uint8)
            w8[8 * b + j, 2:34] = ((qh[b] >> j) & 1) * 16
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=931))
    y5, _ = orc.matmul(gs.Q5_K, w5.reshape(n, -1), n, k, xq, 2)
    y4, _ = orc.matmul(gs.Q4_K, wk.reshape(n, -1), n, k, xq, 2)
    y8, _ = orc.matmul(gs.Q8_0, w8.reshape(n, -1), n, k, xq, 2)
    assert np.allclose(y5, y4 + y8, rtol=0, atol=1e-12 * np.abs(y5).max())


# --------------------------------------------------------- greedy arg-max
# cera 0.5.3 README, "Speculative decoding": greedy verification compares
# arg-max tokens.  Reading: the first index of the largest value.

def test_argmax_rows_matches_numpy(orc):
    rng = np.random.default_rng(60)
    y = rng.standard_normal((7, 1000)).astype(np.float32)
    y[1, 10] = y[1, 900] = 9.0          # a tie: the first index wins
    y[2, :] = 0.0
    y[2, 5] = np.float32(-0.0)          # -0 and +0 compare equal
    y[3, :] = -np.inf
    y[3, 17] = -1e30
    assert np.array_equal(orc.argmax_rows(y), np.argmax(y, axis=1))
    assert orc.argmax_rows(y)[1] == 10 and orc.argmax_rows(y)[2] == 0


# ------------------------------------------------------------------ router
# Cera README, "Supported models": each token picks its own 4 of 32 experts.
# Reading: the top_k largest logits, descending (equal logits: smaller id
# first), softmax over those top_k in fp64, rounded to fp32.

def test_router_topk_matches_stable_argsort(orc):
    rng = np.random.default_rng(61)
    logits = rng.standard_normal((50, 32)).astype(np.float32)
    ids, w = orc.topk_softmax(logits, 4)
    assert np.array_equal(ids, np.argsort(-logits, axis=1, kind="stable")[:, :4])
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref = e / e.sum(axis=1, keepdims=True)
    assert np.allclose(w, ref, rtol=1e-6, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)                     # descending logits -> weights
    assert np.allclose(w.sum(axis=1), 1.0, atol=4 * 2.0 ** -24)


def test_router_closed_forms(orc):
    logits = np.zeros((3, 8), np.float32)
    logits[1, [2, 5, 6]] = 3.0                                 # three-way tie at the top
    logits[2] = np.arange(8, dtype=np.float32)
    ids, w = orc.topk_softmax(logits, 4)
    assert ids[0].tolist() == [0, 1, 2, 3] and np.all(w[0] == np.float32(0.25))
    assert ids[1].tolist() == [2, 5, 6, 0]
    assert ids[2].tolist() == [7, 6, 5, 4]
    # exact shift invariance (integer logits, shift by 16)
    ids2, w2 = orc.topk_softmax(logits + np.float32(16), 4)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    # top_k = n_experts: the full softmax
    idsf, wf = orc.topk_softmax(logits[2:3], 8)
    e = np.exp(np.arange(8)[::-1] - 7.0)
    assert np.allclose(wf[0], e / e.sum(), rtol=1e-7)


# ------------------------------------------------------------------- Q1_0
# alice-llm 2.0.0 README, Bonsai notes: 128-value blocks of 18 bytes, fp16 d
# then 16 bytes of 1-bit weights, value +d or -d.  Reading: value i is bit
# i % 8 of byte 2 + i/8 (LSB first), set = +d.

def _q10_block(d, bits):
    b = np.zeros(18, np.uint8)
    b[0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    b[2:18] = bits
    return b


def test_q1_0_all_set_and_clear(orc):
    assert np.all(orc.dequantize(gs.Q1_0, _q10_block(0.5, np.full(16, 255, np.uint8)), 128) == 0.5)
    assert np.all(orc.dequantize(gs.Q1_0, _q10_block(0.5, np.zeros(16, np.uint8)), 128) == -0.5)


def test_q1_0_one_hot_bits(orc):
    """Setting bit b of sign byte m turns exactly value 8m + b from -d to +d."""
    base = orc.dequantize(gs.Q1_0, _q10_block(2.0, np.zeros(16, np.uint8)), 128)
    for m, b in [(0, 0), (0, 7), (3, 1), (8, 4), (15, 7)]:
        bits = np.zeros(16, np.uint8)
        bits[m] = 1 << b
        v = orc.dequantize(gs.Q1_0, _q10_block(2.0, bits), 128)
        diff = np.flatnonzero(v != base)
        assert diff.tolist() == [8 * m + b] and v[8 * m + b] == 2.0


def test_q1_0_equals_q8_0_of_signs(orc):
    """A Q1_0 row equals the Q8_0 row with the same d and quants +-1, built
    in the test from the sign bits (exact in fp64)."""
    n, k = 3, 512
    w1 = gs.weights(gs.Q1_0, n, k, cfg=940).reshape(-1, 18)
    w8 = np.zeros((w1.shape[0] * 4, 34), np.uint8)
    for b in range(w1.shape[0]):
        signs = np.unpackbits(w1[b, 2:18], bitorder="little").astype(np.int8) * 2 - 1
        for j in range(4):
            w8[4 * b + j, 0:2] = w1[b, 0:2]
            w8[4 * b + j, 2:34] = signs[32 * j: 32 * j + 32].view(np.uint8)
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=940))
    y1, _ = orc.matmul(gs.Q1_0, w1.reshape(n, -1), n, k, xq, 2)
    y8, _ = orc.matmul(gs.Q8_0, w8.reshape(n, -1), n, k, xq, 2)
    assert np.array_equal(y1, y8)


# ------------------------------------------------ TQ2 (2-bit sparse ternary)
def _tq2_block(d, codes):
    """fp16 d, then the 128 2-bit codes four per byte, lowest pair first."""
    codes = np.asarray(codes, np.uint8).reshape(32, 4)
    packed = codes[:, 0] | (codes[:, 1] << 2) | (codes[:, 2] << 4) | (codes[:, 3] << 6)
    return np.concatenate([np.array([d], np.float16).view(np.uint8), packed.astype(np.uint8)])


def test_tq2_block_size(orc):
    # four weights per byte (alice-llm 2.0.0 README, "Sparse Ternary
    # Quantization"): 128 codes in 32 bytes after the 2-byte scale
    assert orc.block_elems(gs.TQ2) == 128 and orc.block_bytes(gs.TQ2) == 34
    assert orc.block_bytes(gs.TQ2) * 8 / orc.block_elems(gs.TQ2) == 2.125


@pytest.mark.parametrize("code,value", [(0, 0.0), (1, 1.0), (3, -1.0), (2, 0.0)])
def test_tq2_codes(orc, code, value):
    # 00 = 0, 01 = +1, 11 = -1 (the page's encoding); 10 expands to 0 through
    # the page's table [0, +1, 0, -1]
    v = orc.dequantize(gs.TQ2, _tq2_block(0.75, np.full(128, code)), 128)
    assert np.all(v == 0.75 * value)


def test_tq2_code_order(orc):
    """Code i sits in bits 2*(i%4) of byte 2 + i/4: a single 01 at position i
    makes exactly value i equal to +d, a single 11 makes it -d."""
    for i in [0, 1, 2, 3, 4, 31, 64, 126, 127]:
        for code, sign in ((1, 1.0), (3, -1.0)):
            c = np.zeros(128, np.uint8)
            c[i] = code
            blk = _tq2_block(2.0, c)
            assert blk[2 + i // 4] == code << (2 * (i % 4))
            v = orc.dequantize(gs.TQ2, blk, 128)
            assert np.flatnonzero(v).tolist() == [i] and v[i] == 2.0 * sign


def test_tq2_equals_q8_0_of_codes(orc):
    """A TQ2 row equals the Q8_0 row with the same d and quants 0 / +1 / -1,
    built in the test from the codes with numpy (exact in fp64)."""
    n, k = 3, 1024
    wt = gs.weights(gs.TQ2, n, k, cfg=950).reshape(-1, 34)
    bits = np.unpackbits(wt[:, 2:34], axis=1, bitorder="little").reshape(-1, 128, 2)
    codes = bits[:, :, 0] + 2 * bits[:, :, 1]
    vals = np.array([0, 1, 0, -1], np.int8)[codes]
    w8 = np.zeros((wt.shape[0] * 4, 34), np.uint8)
    for j in range(4):
        w8[j::4, 0:2] = wt[:, 0:2]
        w8[j::4, 2:34] = vals[:, 32 * j: 32 * j + 32].view(np.uint8)
    xq = orc.quantize_q8_0(gs.activations(2, k, cfg=950))
    yt, _ = orc.matmul(gs.TQ2, wt.reshape(n, -1), n, k, xq, 2)
    y8, _ = orc.matmul(gs.Q8_0, w8.reshape(n, -1), n, k, xq, 2)
    assert np.array_equal(yt, y8)


def test_tq2_generator_is_8_of_16_sparse():
    """The synthetic TQ2 weights keep the pages' 8:16 structure: exactly 8
    non-zero codes in every 16 consecutive values, only codes 00/01/11."""
    w = gs.weights(gs.TQ2, 17, 2048, cfg=951).reshape(-1, 34)
    bits = np.unpackbits(w[:, 2:34], axis=1, bitorder="little").reshape(-1, 128, 2)
    codes = (bits[:, :, 0] + 2 * bits[:, :, 1]).reshape(-1, 16)
    assert not (codes == 2).any()
    assert np.all((codes != 0).sum(axis=1) == 8)
