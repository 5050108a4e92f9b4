/*
 * oracle.cpp -- plain CPU reference for the block-quantized GGUF matmul.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h for who may call it and for the
 * sources and readings it follows).  Built with g++ -O2 -ffp-contract=off,
 * no fast-math, no SIMD intrinsics: every floating-point operation below is
 * the IEEE operation written in the source.
 */
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

/* ---- fp16 (IEEE-754 binary16) ------------------------------------------ */

/* Value of a binary16 encoding: sign, 5-bit biased exponent (bias 15), 10-bit
 * fraction.  Exponent 0 = subnormal (fraction * 2^-24), 31 = inf / NaN. */
double half_value(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1F;
    const int frac = h & 0x3FF;
    double v;
    if (expo == 0) {
        v = std::ldexp(static_cast<double>(frac), -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = std::ldexp(static_cast<double>(1024 + frac), expo - 25);
    }
    return sign ? -v : v;
}

/* fp32 -> binary16 with round-to-nearest-even.  The fp32 value is exact in
 * fp64; scaling by a power of two is exact, so nearbyint() (default rounding
 * mode: nearest, ties to even) performs the single rounding. */
uint16_t half_from_float(float f) {
    uint32_t bits;
    std::memcpy(&bits, &f, 4);
    const uint16_t sign = static_cast<uint16_t>((bits >> 16) & 0x8000u);
    if (std::isnan(f)) {
        /* quiet NaN keeping the top 9 payload bits */
        return static_cast<uint16_t>(sign | 0x7E00u | ((bits >> 13) & 0x3FFu));
    }
    const double a = std::fabs(static_cast<double>(f));
    if (std::isinf(f) || a >= 65520.0) {  /* 65520 = halfway past 65504 -> inf */
        return static_cast<uint16_t>(sign | 0x7C00u);
    }
    if (a == 0.0) return sign;
    int e;                       /* a = mant * 2^e with mant in [0.5, 1) */
    std::frexp(a, &e);
    int unbiased = e - 1;        /* a in [2^unbiased, 2^(unbiased+1)) */
    if (unbiased < -14) {
        /* subnormal range: quantum 2^-24 */
        const double n = std::nearbyint(std::ldexp(a, 24));
        /* n == 1024 rounds up into the smallest normal, whose encoding is
         * the same integer */
        return static_cast<uint16_t>(sign | static_cast<uint16_t>(n));
    }
    double n = std::nearbyint(std::ldexp(a, 10 - unbiased)); /* in [1024, 2048] */
    if (n == 2048.0) {
        n = 1024.0;
        unbiased += 1;
    }
    if (unbiased > 15) return static_cast<uint16_t>(sign | 0x7C00u);
    return static_cast<uint16_t>(sign | ((unbiased + 15) << 10) |
                                 (static_cast<int>(n) - 1024));
}

uint16_t rd16(const uint8_t* p) {   /* little-endian 16-bit field */
    return static_cast<uint16_t>(p[0] | (p[1] << 8));
}

/* ---- block formats ------------------------------------------------------ */

int64_t elems_of(int type) {
    switch (type) {
        case ORACLE_Q4_0: case ORACLE_Q4_1: case ORACLE_Q8_0: return 32;
        case ORACLE_Q4_K: case ORACLE_Q5_K: case ORACLE_Q6_K: return 256;
        case ORACLE_Q1_0: case ORACLE_TQ2: return 128;
        default: return -1;
    }
}

int64_t bytes_of(int type) {
    switch (type) {
        case ORACLE_Q4_0: return 18;   /* fp16 d + 16 nibble bytes        */
        case ORACLE_Q4_1: return 20;   /* fp16 d + fp16 m + 16 bytes      */
        case ORACLE_Q8_0: return 34;   /* fp16 d + 32 int8 [alice-QBS]    */
        case ORACLE_Q4_K: return 144;  /* 2 + 2 + 12 + 128 [alice-QBS]    */
        case ORACLE_Q5_K: return 176;  /* 2 + 2 + 12 + 32 + 128 [alice-Q5K] */
        case ORACLE_Q1_0: return 18;   /* 2 + 16 [alice-Q10]              */
        case ORACLE_Q6_K: return 210;  /* 128 + 64 + 16 + 2 [alice-Q6K]   */
        case ORACLE_TQ2: return 34;    /* 2 + 32 (2 bits x 128) [alice-TQ] */
        default: return -1;
    }
}

/* Q4_K six-bit scale/min of sub-block j from the 12 packed bytes S.
 * Sub-blocks 0..3: low six bits of S[j] (scale) and S[j+4] (min).
 * Sub-blocks 4..7: low nibble of S[j+4] plus the top two bits of S[j-4]
 * (scale); high nibble of S[j+4] plus the top two bits of S[j] (min). */
void q4k_scale_min(const uint8_t* S, int j, int* sc, int* mn) {
    if (j < 4) {
        *sc = S[j] & 63;
        *mn = S[j + 4] & 63;
    } else {
        *sc = (S[j + 4] & 0x0F) | ((S[j - 4] >> 6) << 4);
        *mn = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
}

/* Q5_K: 5-bit quant (0..31) of element e (0..255) of the super-block at b,
 * per the reading in oracle.h: low four bits from the qs nibble, bit 4 from
 * bit (sub-block) of qh[e % 32]. */
int q5k_quant(const uint8_t* b, int e) {
    const uint8_t* qh = b + 16;
    const uint8_t* qs = b + 48;
    const int j = e / 32, l = e % 32, c = j / 2;
    const uint8_t byte = qs[32 * c + l];
    const int low = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return low | (((qh[l] >> j) & 1) << 4);
}

/* Q6_K: 6-bit quant (0..63) and signed scale of element e (0..255) of the
 * super-block at b, per the reading in oracle.h. */
void q6k_element(const uint8_t* b, int e, int* q, int* scale) {
    const uint8_t* ql = b;
    const uint8_t* qh = b + 128;
    const int8_t* sc = reinterpret_cast<const int8_t*>(b + 192);
    const int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
    const uint8_t lbyte = ql[64 * h + l + (g % 2 == 1 ? 32 : 0)];
    const int low = (g < 2) ? (lbyte & 0x0F) : (lbyte >> 4);
    const int high = (qh[32 * h + l] >> (2 * g)) & 3;
    *q = low | (high << 4);
    *scale = sc[8 * h + 2 * g + l / 16];
}

/* TQ2: the value (0, +1 or -1) of 2-bit code i of the block at b, through
 * the expansion table [0, +1, 0, -1] [alice-TQ]. */
int tq2_value(const uint8_t* b, int i) {
    static const int table[4] = {0, 1, 0, -1};
    return table[(b[2 + i / 4] >> (2 * (i % 4))) & 3];
}

/* Decode one block to its elems_of(type) exact fp64 values. */
void decode_block(int type, const uint8_t* b, double* out) {
    switch (type) {
        case ORACLE_Q4_0: {
            const double d = half_value(rd16(b));
            for (int i = 0; i < 16; ++i) {
                out[i]      = d * ((b[2 + i] & 0x0F) - 8);
                out[i + 16] = d * ((b[2 + i] >> 4) - 8);
            }
            break;
        }
        case ORACLE_Q4_1: {
            const double d = half_value(rd16(b));
            const double m = half_value(rd16(b + 2));
            for (int i = 0; i < 16; ++i) {
                out[i]      = d * (b[4 + i] & 0x0F) + m;
                out[i + 16] = d * (b[4 + i] >> 4) + m;
            }
            break;
        }
        case ORACLE_Q1_0: {
            const double d = half_value(rd16(b));
            for (int i = 0; i < 128; ++i) out[i] = ((b[2 + i / 8] >> (i % 8)) & 1) ? d : -d;
            break;
        }
        case ORACLE_Q8_0: {
            const double d = half_value(rd16(b));
            for (int i = 0; i < 32; ++i) out[i] = d * static_cast<int8_t>(b[2 + i]);
            break;
        }
        case ORACLE_TQ2: {
            const double d = half_value(rd16(b));
            for (int i = 0; i < 128; ++i) out[i] = d * tq2_value(b, i);
            break;
        }
        case ORACLE_Q4_K: {
            const double d = half_value(rd16(b));
            const double dmin = half_value(rd16(b + 2));
            const uint8_t* S = b + 4;
            const uint8_t* Q = b + 16;
            for (int c = 0; c < 4; ++c) {
                int sc_lo, m_lo, sc_hi, m_hi;
                q4k_scale_min(S, 2 * c, &sc_lo, &m_lo);
                q4k_scale_min(S, 2 * c + 1, &sc_hi, &m_hi);
                for (int i = 0; i < 32; ++i) {
                    out[64 * c + i]      = d * sc_lo * (Q[32 * c + i] & 0x0F) - dmin * m_lo;
                    out[64 * c + 32 + i] = d * sc_hi * (Q[32 * c + i] >> 4) - dmin * m_hi;
                }
            }
            break;
        }
        case ORACLE_Q5_K: {
            const double d = half_value(rd16(b));
            const double dmin = half_value(rd16(b + 2));
            for (int e = 0; e < 256; ++e) {
                int sc, mn;
                q4k_scale_min(b + 4, e / 32, &sc, &mn);
                out[e] = d * sc * q5k_quant(b, e) - dmin * mn;
            }
            break;
        }
        case ORACLE_Q6_K: {
            const double d = half_value(rd16(b + 208));
            for (int e = 0; e < 256; ++e) {
                int q, sc;
                q6k_element(b, e, &q, &sc);
                out[e] = d * sc * (q - 32);
            }
            break;
        }
        default: break;
    }
}

void decode_row(int type, const uint8_t* row, int64_t k, double* out) {
    const int64_t qk = elems_of(type), bs = bytes_of(type);
    for (int64_t b = 0; b < k / qk; ++b) decode_block(type, row + b * bs, out + b * qk);
}

bool shape_ok(int type, int64_t k) {
    const int64_t qk = elems_of(type);
    return qk > 0 && k > 0 && k % qk == 0 && k % 32 == 0;
}

/* Run f(i) for i in [0, count) over up to n_threads threads, static blocks. */
template <class F>
void parallel_for(int64_t count, int n_threads, F f) {
    if (n_threads <= 1 || count < 2) {
        for (int64_t i = 0; i < count; ++i) f(i);
        return;
    }
    const int64_t nt = std::min<int64_t>(n_threads, count);
    std::vector<std::thread> th;
    for (int64_t t = 0; t < nt; ++t) {
        const int64_t lo = count * t / nt, hi = count * (t + 1) / nt;
        th.emplace_back([=] { for (int64_t i = lo; i < hi; ++i) f(i); });
    }
    for (auto& x : th) x.join();
}

/* ---- Q8_0 quantization of one 32-value block ---------------------------- */
/* [alice-P4]: amax over the block, scale 127/amax, multiply, round to
 * nearest with ties to even, saturate.  Stored scale d = amax/127 rounded to
 * fp16.  Readings: all arithmetic in fp32 (one division for 127/amax, one
 * per-element multiply, one division for amax/127 then one rounding to
 * fp16); amax == 0 gives d = 0 and all quants 0; a zero element quantizes to
 * 0 even when 127/amax overflows to infinity (then the other elements
 * saturate to +-127 and d rounds to 0). */
void quantize_block_q8_0(const float* x, uint8_t* out) {
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        const float a = std::fabs(x[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        std::memset(out, 0, 34);
        return;
    }
    const float id = 127.0f / amax;
    const float d = amax / 127.0f;
    const uint16_t d16 = half_from_float(d);
    out[0] = static_cast<uint8_t>(d16 & 0xFF);
    out[1] = static_cast<uint8_t>(d16 >> 8);
    for (int i = 0; i < 32; ++i) {
        const float v = x[i] * id;
        int q;
        if (std::isnan(v)) {
            q = 0;                        /* 0 * inf */
        } else {
            float r = std::nearbyint(v);  /* ties to even */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q = static_cast<int>(r);
        }
        out[2 + i] = static_cast<uint8_t>(static_cast<int8_t>(q));
    }
}

/* ---- integer block dots for the factored formulation -------------------- */

/* Exact integer sum of wq[i]*xq[i] over 32 values. */
int64_t idot32(const int* wq, const int8_t* xq) {
    int64_t s = 0;
    for (int i = 0; i < 32; ++i) s += static_cast<int64_t>(wq[i]) * xq[i];
    return s;
}

int64_t isum32(const int8_t* xq) {
    int64_t s = 0;
    for (int i = 0; i < 32; ++i) s += xq[i];
    return s;
}

/* y = sum over blocks of the factored per-block contributions for one
 * weight row and one activation row. */
double factored_dot(int type, const uint8_t* wrow, const uint8_t* xrow, int64_t k) {
    double acc = 0.0;
    const int64_t nb32 = k / 32;
    if (type == ORACLE_Q4_K) {
        for (int64_t sb = 0; sb < k / 256; ++sb) {
            const uint8_t* b = wrow + sb * 144;
            const double d = half_value(rd16(b)), dmin = half_value(rd16(b + 2));
            for (int j = 0; j < 8; ++j) {
                int sc, mn;
                q4k_scale_min(b + 4, j, &sc, &mn);
                int q[32];
                const int c = j / 2;
                for (int i = 0; i < 32; ++i) {
                    const uint8_t byte = b[16 + 32 * c + i];
                    q[i] = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                }
                const uint8_t* xb = xrow + (sb * 8 + j) * 34;
                const double dx = half_value(rd16(xb));
                const int8_t* xq = reinterpret_cast<const int8_t*>(xb + 2);
                /* d*dx*sc*sum(q*qx) - dmin*dx*m*sum(qx) [alice-Q4K] */
                acc += d * dx * sc * static_cast<double>(idot32(q, xq)) -
                       dmin * dx * mn * static_cast<double>(isum32(xq));
            }
        }
        return acc;
    }
    if (type == ORACLE_Q1_0) {
        /* per 32-value activation block: d*dx*sum(s*qx), s = +-1 [alice-Q10] */
        for (int64_t blk = 0; blk < k / 128; ++blk) {
            const uint8_t* b = wrow + blk * 18;
            const double d = half_value(rd16(b));
            for (int j = 0; j < 4; ++j) {
                int s[32];
                for (int i = 0; i < 32; ++i) {
                    const int e = 32 * j + i;
                    s[i] = ((b[2 + e / 8] >> (e % 8)) & 1) ? 1 : -1;
                }
                const uint8_t* xb = xrow + (blk * 4 + j) * 34;
                const double dx = half_value(rd16(xb));
                acc += d * dx * static_cast<double>(idot32(s, reinterpret_cast<const int8_t*>(xb + 2)));
            }
        }
        return acc;
    }
    if (type == ORACLE_TQ2) {
        /* per 32-value activation block: d*dx*sum(t*qx), t in {0, +1, -1} */
        for (int64_t blk = 0; blk < k / 128; ++blk) {
            const uint8_t* b = wrow + blk * 34;
            const double d = half_value(rd16(b));
            for (int j = 0; j < 4; ++j) {
                int t[32];
                for (int i = 0; i < 32; ++i) t[i] = tq2_value(b, 32 * j + i);
                const uint8_t* xb = xrow + (blk * 4 + j) * 34;
                const double dx = half_value(rd16(xb));
                acc += d * dx * static_cast<double>(idot32(t, reinterpret_cast<const int8_t*>(xb + 2)));
            }
        }
        return acc;
    }
    if (type == ORACLE_Q5_K) {
        /* as Q4_K per 32-element sub-block, with 5-bit quants [alice-Q5K] */
        for (int64_t sb = 0; sb < k / 256; ++sb) {
            const uint8_t* b = wrow + sb * 176;
            const double d = half_value(rd16(b)), dmin = half_value(rd16(b + 2));
            for (int j = 0; j < 8; ++j) {
                int sc, mn;
                q4k_scale_min(b + 4, j, &sc, &mn);
                int q[32];
                for (int i = 0; i < 32; ++i) q[i] = q5k_quant(b, 32 * j + i);
                const uint8_t* xb = xrow + (sb * 8 + j) * 34;
                const double dx = half_value(rd16(xb));
                const int8_t* xq = reinterpret_cast<const int8_t*>(xb + 2);
                acc += d * dx * sc * static_cast<double>(idot32(q, xq)) -
                       dmin * dx * mn * static_cast<double>(isum32(xq));
            }
        }
        return acc;
    }
    if (type == ORACLE_Q6_K) {
        /* per 16-element scale group: d*dx*scale*(sum q*qx - 32*sum qx) */
        for (int64_t sb = 0; sb < k / 256; ++sb) {
            const uint8_t* b = wrow + sb * 210;
            const double d = half_value(rd16(b + 208));
            for (int grp = 0; grp < 16; ++grp) {
                const int e0 = 16 * grp;
                const uint8_t* xb = xrow + (sb * 8 + e0 / 32) * 34;
                const double dx = half_value(rd16(xb));
                const int8_t* xq = reinterpret_cast<const int8_t*>(xb + 2) + e0 % 32;
                int64_t sq = 0, sx = 0;
                int sc = 0;
                for (int i = 0; i < 16; ++i) {
                    int q;
                    q6k_element(b, e0 + i, &q, &sc);  /* one scale per group */
                    sq += static_cast<int64_t>(q) * xq[i];
                    sx += xq[i];
                }
                acc += d * dx * sc * static_cast<double>(sq - 32 * sx);
            }
        }
        return acc;
    }
    const int64_t bs = bytes_of(type);
    for (int64_t blk = 0; blk < nb32; ++blk) {
        const uint8_t* b = wrow + blk * bs;
        const uint8_t* xb = xrow + blk * 34;
        const double dx = half_value(rd16(xb));
        const int8_t* xq = reinterpret_cast<const int8_t*>(xb + 2);
        int q[32];
        if (type == ORACLE_Q4_0) {
            for (int i = 0; i < 16; ++i) {
                q[i] = (b[2 + i] & 0x0F) - 8;
                q[i + 16] = (b[2 + i] >> 4) - 8;
            }
            acc += half_value(rd16(b)) * dx * static_cast<double>(idot32(q, xq));
        } else if (type == ORACLE_Q4_1) {
            for (int i = 0; i < 16; ++i) {
                q[i] = b[4 + i] & 0x0F;
                q[i + 16] = b[4 + i] >> 4;
            }
            const double d = half_value(rd16(b)), m = half_value(rd16(b + 2));
            acc += dx * (d * static_cast<double>(idot32(q, xq)) +
                         m * static_cast<double>(isum32(xq)));
        } else { /* Q8_0 */
            for (int i = 0; i < 32; ++i) q[i] = static_cast<int8_t>(b[2 + i]);
            acc += half_value(rd16(b)) * dx * static_cast<double>(idot32(q, xq));
        }
    }
    return acc;
}

}  // namespace

extern "C" {

int oracle_abi_version(void) { return 1; }

int64_t oracle_block_elems(int type) { return elems_of(type); }
int64_t oracle_block_bytes(int type) { return bytes_of(type); }

double oracle_half_to_double(uint16_t h) { return half_value(h); }
uint16_t oracle_float_to_half(float f) { return half_from_float(f); }

void oracle_half_to_double_n(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = half_value(h[i]);
}

void oracle_float_to_half_n(const float* f, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = half_from_float(f[i]);
}

void oracle_q4k_scale_min(const uint8_t* scales12, int j, int* sc, int* mn) {
    q4k_scale_min(scales12, j, sc, mn);
}

int oracle_dequantize(int type, const uint8_t* blocks, int64_t n_elems, double* out) {
    if (elems_of(type) < 0) return -2;
    if (!blocks || !out || n_elems < 0) return -1;
    if (n_elems % elems_of(type) != 0) return -3;
    decode_row(type, blocks, n_elems, out);
    return 0;
}

int oracle_quantize_q8_0(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* out) {
    if (!x || !out || rows < 0 || k <= 0 || ldx < k) return -1;
    if (k % 32 != 0) return -3;
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            quantize_block_q8_0(x + r * ldx + b * 32, out + (r * nb + b) * 34);
    return 0;
}

int oracle_matmul(int type, const uint8_t* w, int64_t n, int64_t k,
                  const uint8_t* xq, int64_t m, double* y, double* s, int n_threads) {
    if (elems_of(type) < 0) return -2;
    if (!w || !xq || n < 0 || m < 0) return -1;
    if (!shape_ok(type, k)) return -3;
    const int64_t wrow_bytes = k / elems_of(type) * bytes_of(type);
    const int64_t xrow_bytes = k / 32 * 34;
    /* dequantized activations, all rows */
    std::vector<double> xd(static_cast<size_t>(m * k));
    for (int64_t i = 0; i < m; ++i) decode_row(ORACLE_Q8_0, xq + i * xrow_bytes, k, &xd[i * k]);
    parallel_for(n, n_threads, [&](int64_t r) {
        std::vector<double> wd(static_cast<size_t>(k));
        decode_row(type, w + r * wrow_bytes, k, wd.data());
        for (int64_t i = 0; i < m; ++i) {
            double acc = 0.0, mag = 0.0;
            const double* xr = &xd[i * k];
            for (int64_t j = 0; j < k; ++j) {
                const double p = wd[j] * xr[j];   /* exact: <= 21 x 19 bits */
                acc += p;
                mag += std::fabs(p);
            }
            if (y) y[i * n + r] = acc;
            if (s) s[i * n + r] = mag;
        }
    });
    return 0;
}

int oracle_matmul_sampled(int type, const uint8_t* w, int64_t n, int64_t k,
                          const uint8_t* xq, int64_t m,
                          const int64_t* act_rows, const int64_t* w_rows, int64_t count,
                          double* y, double* s, int n_threads) {
    if (elems_of(type) < 0) return -2;
    if (!w || !xq || !act_rows || !w_rows || count < 0) return -1;
    if (!shape_ok(type, k)) return -3;
    for (int64_t c = 0; c < count; ++c)
        if (act_rows[c] < 0 || act_rows[c] >= m || w_rows[c] < 0 || w_rows[c] >= n) return -1;
    const int64_t wrow_bytes = k / elems_of(type) * bytes_of(type);
    const int64_t xrow_bytes = k / 32 * 34;
    parallel_for(count, n_threads, [&](int64_t c) {
        std::vector<double> wd(static_cast<size_t>(k)), xd(static_cast<size_t>(k));
        decode_row(type, w + w_rows[c] * wrow_bytes, k, wd.data());
        decode_row(ORACLE_Q8_0, xq + act_rows[c] * xrow_bytes, k, xd.data());
        double acc = 0.0, mag = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            const double p = wd[j] * xd[j];
            acc += p;
            mag += std::fabs(p);
        }
        if (y) y[c] = acc;
        if (s) s[c] = mag;
    });
    return 0;
}

int oracle_matmul_factored(int type, const uint8_t* w, int64_t n, int64_t k,
                           const uint8_t* xq, int64_t m, double* y, int n_threads) {
    if (elems_of(type) < 0) return -2;
    if (!w || !xq || !y || n < 0 || m < 0) return -1;
    if (!shape_ok(type, k)) return -3;
    const int64_t wrow_bytes = k / elems_of(type) * bytes_of(type);
    const int64_t xrow_bytes = k / 32 * 34;
    parallel_for(n, n_threads, [&](int64_t r) {
        for (int64_t i = 0; i < m; ++i)
            y[i * n + r] = factored_dot(type, w + r * wrow_bytes, xq + i * xrow_bytes, k);
    });
    return 0;
}

void oracle_swiglu(const float* g, const float* u, int64_t n, float* h) {
    for (int64_t i = 0; i < n; ++i) {
        const double z = static_cast<double>(g[i]);
        const double silu = z / (1.0 + std::exp(-z));
        h[i] = static_cast<float>(silu * static_cast<double>(u[i]));
    }
}

int oracle_moe_group(const int32_t* ids, int64_t n_tokens, int64_t top_k,
                     int64_t n_experts, int32_t* offsets, int32_t* pairs) {
    if (!ids || !offsets || !pairs || n_tokens < 0 || top_k <= 0 || n_experts <= 0) return -1;
    const int64_t np = n_tokens * top_k;
    std::vector<int64_t> count(static_cast<size_t>(n_experts), 0);
    for (int64_t p = 0; p < np; ++p) {
        if (ids[p] < 0 || ids[p] >= n_experts) return -1;
        count[ids[p]]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < n_experts; ++e)
        offsets[e + 1] = static_cast<int32_t>(offsets[e] + count[e]);
    std::vector<int64_t> fill(offsets, offsets + n_experts);
    for (int64_t p = 0; p < np; ++p)          /* ascending p: stable */
        pairs[fill[ids[p]]++] = static_cast<int32_t>(p);
    return 0;
}

int oracle_moe_matmul(int type, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                      const uint8_t* xq, int x_per_pair, const int32_t* ids,
                      int64_t n_tokens, int64_t top_k, double* y, double* s, int n_threads) {
    if (elems_of(type) < 0) return -2;
    if (!w || !xq || !ids || n_experts <= 0 || n < 0 || n_tokens < 0 || top_k <= 0) return -1;
    if (!shape_ok(type, k)) return -3;
    const int64_t wrow_bytes = k / elems_of(type) * bytes_of(type);
    const int64_t xrow_bytes = k / 32 * 34;
    const int64_t np = n_tokens * top_k;
    for (int64_t p = 0; p < np; ++p)
        if (ids[p] < 0 || ids[p] >= n_experts) return -1;
    parallel_for(np, n_threads, [&](int64_t p) {
        const int64_t e = ids[p];
        const int64_t row = x_per_pair ? p : p / top_k;
        std::vector<double> xd(static_cast<size_t>(k)), wd(static_cast<size_t>(k));
        decode_row(ORACLE_Q8_0, xq + row * xrow_bytes, k, xd.data());
        for (int64_t r = 0; r < n; ++r) {
            decode_row(type, w + (e * n + r) * wrow_bytes, k, wd.data());
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                const double prod = wd[j] * xd[j];
                acc += prod;
                mag += std::fabs(prod);
            }
            if (y) y[p * n + r] = acc;
            if (s) s[p * n + r] = mag;
        }
    });
    return 0;
}

int oracle_moe_combine(const double* d, const double* s_in, const float* route_w,
                       int64_t n_tokens, int64_t top_k, int64_t n,
                       double* y, double* s_out) {
    if (!d || !route_w || n_tokens < 0 || top_k <= 0 || n < 0) return -1;
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t sl = 0; sl < top_k; ++sl) {
                const double wt = static_cast<double>(route_w[t * top_k + sl]);
                const int64_t p = t * top_k + sl;
                acc += wt * d[p * n + j];
                if (s_in) mag += std::fabs(wt) * s_in[p * n + j];
            }
            if (y) y[t * n + j] = acc;
            if (s_out) s_out[t * n + j] = mag;
        }
    }
    return 0;
}

}  // extern "C"

/* ---- greedy arg-max and router ------------------------------------------ */

void oracle_argmax_rows(const float* y, int64_t rows, int64_t n, int64_t ldy, int32_t* idx) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* row = y + r * ldy;
        int64_t best = 0;
        for (int64_t i = 1; i < n; ++i)
            if (row[i] > row[best]) best = i;   /* strict: the first maximum wins */
        idx[r] = static_cast<int32_t>(best);
    }
}

int oracle_topk_softmax(const float* logits, int64_t rows, int64_t n_experts, int64_t ld,
                        int64_t top_k, int32_t* ids, float* w) {
    if (rows < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts || ld < n_experts) return -1;
    std::vector<int64_t> order(static_cast<size_t>(n_experts));
    for (int64_t t = 0; t < rows; ++t) {
        const float* l = logits + t * ld;
        for (int64_t e = 0; e < n_experts; ++e) order[static_cast<size_t>(e)] = e;
        /* descending logit, then ascending id */
        std::stable_sort(order.begin(), order.end(),
                         [&](int64_t a, int64_t b) { return l[a] > l[b]; });
        const double l0 = static_cast<double>(l[order[0]]);
        double sum = 0.0;
        for (int64_t s = 0; s < top_k; ++s) sum += std::exp(static_cast<double>(l[order[s]]) - l0);
        for (int64_t s = 0; s < top_k; ++s) {
            ids[t * top_k + s] = static_cast<int32_t>(order[static_cast<size_t>(s)]);
            w[t * top_k + s] = static_cast<float>(std::exp(static_cast<double>(l[order[s]]) - l0) / sum);
        }
    }
    return 0;
}
