// gemm.hip -- prefill GEMM over GGUF blocks with int8 MFMA on gfx950.
//
//   y[m][n] = sum over 32-value blocks b of dx[m,b] * dw[n,b] * I[m,n,b],
//   I[m,n,b] = sum_i wq[n, 32b+i] * xq[m, 32b+i]   (exact int32)
//
// (alice-llm 2.0.0 README, "Computation Path (Q4_K)": integer dot inside
// each 32-value block, scales applied once per block.)
//
// Tiling: a 256-thread workgroup owns 128 tokens x 128 weight rows and walks
// k in steps of 4 blocks (128 values).  Per step the weight blocks are
// decoded once into signed int8 rows in LDS (Q4_0: q-8, Q4_1 / Q4_K: q) and
// the Q8_0 activation blocks are split into int8 rows plus fp32 scales.
// Each wave computes 64 x 64 outputs as 2 x 2 tiles of
// v_mfma_i32_32x32x32_i8: one MFMA is exactly one 32-value block.
//
// Scale application: the MFMA accumulator starts from the bit pattern of
// 1.5*2^23 (12582912.0f), so the int32 result read as a float is exactly
// 12582912 + I (|I| < 2^22).  Then t = fma(D, dx, -12582912*dx) = round(I*dx)
// (the subtrahend is exact: dx has 11 significant bits) and
// acc = fma(t, dw, acc): two VALU FMAs per output and block, no convert.
// With packed-FP32 instructions disabled this VALU work, not the MFMA, is
// the bound: 2 lane-FMAs per output per block against 1/128 of a CU-clock
// of MFMA time, i.e. at most a quarter of the int8 MFMA peak.
//
// Q4_1 and Q4_K also carry an additive term per block, sum_b (dx*sum(xq))[m,b]
// * c[n,b] with c = m (Q4_1) or -dmin*min (Q4_K).  That is itself a matrix
// product over blocks; it is accumulated with fp32 MFMA
// (v_mfma_f32_32x32x2_f32, two blocks per instruction) into the same
// accumulators, so it costs MFMA time, not VALU time.
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {
namespace {

enum { T_Q4_0 = 2, T_Q4_1 = 3, T_Q8_0 = 8, T_Q4_K = 12 };

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128;          // tokens per workgroup tile
constexpr int BN = 128;          // weight rows per workgroup tile
constexpr int KB = 4;            // 32-value blocks per k step
constexpr int ROW = KB * 32 + 16;  // LDS row stride of the int8 tiles (16 B pad)
constexpr int kThreads = 256;
constexpr int kBias = 0x4B400000;
constexpr float kBiasF = 12582912.0f;

template <int FMT> constexpr bool kHasOffset = (FMT == T_Q4_1 || FMT == T_Q4_K);

struct Smem {
    int8_t w[BN * ROW];       // decoded weight quants, row n, k within the step
    int8_t x[BM * ROW];       // activation quants
    float dw[KB][BN];         // weight block scale (Q4_K: d*sc)
    float dx[KB][BM];         // activation block scale
    float cw[KB][BN];         // Q4_1: m; Q4_K: -dmin*min  (additive weight term)
    float sx[KB][BM];         // dx * sum of the block's activation quants
};

__device__ __forceinline__ uint32_t nib_lo_s8(uint32_t v) {   // low nibbles as q-8
    return ((v & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t nib_hi_s8(uint32_t v) {
    return (((v >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t nib_lo(uint32_t v) { return v & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t v) { return (v >> 4) & 0x0F0F0F0Fu; }

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Bytes [off, off+4*N) of a little-endian byte stream held in dwords
// w[0..] (off even, known at compile time after unrolling).
template <int N>
__device__ __forceinline__ void extract(const uint32_t* w, int off, uint32_t* out) {
#pragma unroll
    for (int t = 0; t < N; ++t) {
        const int o = off + 4 * t;
        out[t] = (o & 2) ? __builtin_amdgcn_alignbit(w[(o >> 2) + 1], w[o >> 2], 16) : w[o >> 2];
    }
}
__device__ __forceinline__ uint32_t half_at(const uint32_t* w, int off) {
    return (w[off >> 2] >> ((off & 2) * 8)) & 0xFFFFu;
}

// ---- staging of one k step --------------------------------------------------
// Two threads per row: thread t stages row t/2, blocks 2*(t%2) and
// 2*(t%2)+1 of the step.  All global loads are 4-byte loads.
template <int FMT>
__device__ __forceinline__ void stage_weights(Smem& s, const uint8_t* __restrict__ w, int64_t n,
                                              int64_t rb, int64_t n0, int kstep) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    const int64_t gn = n0 + row;
    if constexpr (FMT == T_Q4_K) {
        // a 256-value super-block spans two k steps; this step holds nibble
        // chunks 2*(kstep&1) and +1, this thread chunk c (sub-blocks 2c, 2c+1)
        const int c = 2 * (kstep & 1) + half;
        uint32_t hdr[4], q[8];
        if (gn < n) {
            const uint8_t* p = w + gn * rb + static_cast<int64_t>(kstep >> 1) * 144;
            const uint4 hv = *reinterpret_cast<const uint4*>(p);
            hdr[0] = hv.x; hdr[1] = hv.y; hdr[2] = hv.z; hdr[3] = hv.w;
            const uint4 v0 = *reinterpret_cast<const uint4*>(p + 16 + 32 * c);
            const uint4 v1 = *reinterpret_cast<const uint4*>(p + 32 + 32 * c);
            q[0] = v0.x; q[1] = v0.y; q[2] = v0.z; q[3] = v0.w;
            q[4] = v1.x; q[5] = v1.y; q[6] = v1.z; q[7] = v1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) hdr[i] = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = 0;
        }
        const float d = h2f(hdr[0] & 0xFFFFu), dmin = h2f(hdr[0] >> 16);
        const uint32_t S0 = hdr[1], S1 = hdr[2], S2 = hdr[3];
#pragma unroll
        for (int e = 0; e < 2; ++e) {             // sub-block j = 2c + e -> local block 2*half + e
            const int j = 2 * c + e;
            int sc, mn;
            if (j < 4) {
                sc = (S0 >> (8 * j)) & 63;
                mn = (S1 >> (8 * j)) & 63;
            } else {
                const int sh = 8 * (j - 4);
                sc = ((S2 >> sh) & 0xF) | ((((S0 >> sh) >> 6) & 3) << 4);
                mn = (((S2 >> sh) >> 4) & 0xF) | ((((S1 >> sh) >> 6) & 3) << 4);
            }
            const int b = 2 * half + e;
            s.dw[b][row] = d * static_cast<float>(sc);
            s.cw[b][row] = -(dmin * static_cast<float>(mn));
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = e ? nib_hi(q[i]) : nib_lo(q[i]);
            uint4* d4 = reinterpret_cast<uint4*>(s.w + row * ROW + 32 * b);
            d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    } else {
        constexpr int BS = (FMT == T_Q4_0) ? 18 : (FMT == T_Q4_1) ? 20 : 34;
        constexpr int NW = (2 * BS) / 4;          // dwords of 2 blocks
        uint32_t v[NW];
        if (gn < n) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(
                w + gn * rb + (static_cast<int64_t>(kstep) * KB + 2 * half) * BS);
#pragma unroll
            for (int i = 0; i < NW; ++i) v[i] = p[i];
        } else {
#pragma unroll
            for (int i = 0; i < NW; ++i) v[i] = 0;
        }
#pragma unroll
        for (int bl = 0; bl < 2; ++bl) {
            const int b = 2 * half + bl;
            uint32_t o[8];
            s.dw[b][row] = h2f(half_at(v, bl * BS));
            if constexpr (FMT == T_Q8_0) {
                extract<8>(v, bl * BS + 2, o);
            } else {
                uint32_t q[4];
                extract<4>(v, bl * BS + (FMT == T_Q4_0 ? 2 : 4), q);
                if constexpr (FMT == T_Q4_1) s.cw[b][row] = h2f(half_at(v, bl * BS + 2));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = (FMT == T_Q4_0) ? nib_lo_s8(q[i]) : nib_lo(q[i]);
                    o[4 + i] = (FMT == T_Q4_0) ? nib_hi_s8(q[i]) : nib_hi(q[i]);
                }
            }
            uint4* d4 = reinterpret_cast<uint4*>(s.w + row * ROW + 32 * b);
            d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

template <int FMT>
__device__ __forceinline__ void stage_acts(Smem& s, const uint8_t* __restrict__ xq, int64_t m,
                                           int64_t xrb, int64_t m0, int kstep) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    const int64_t gm = m0 + row;
    uint32_t v[17];  // 2 blocks x 34 bytes
    if (gm < m) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(
            xq + gm * xrb + (static_cast<int64_t>(kstep) * KB + 2 * half) * 34);
#pragma unroll
        for (int i = 0; i < 17; ++i) v[i] = p[i];
    } else {
#pragma unroll
        for (int i = 0; i < 17; ++i) v[i] = 0;
    }
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
        const int b = 2 * half + bl;
        uint32_t o[8];
        extract<8>(v, bl * 34 + 2, o);
        const float dx = h2f(half_at(v, bl * 34));
        s.dx[b][row] = dx;
        if constexpr (kHasOffset<FMT>) {
            int sum = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum = sdot4(o[i], 0x01010101u, sum);
            s.sx[b][row] = dx * static_cast<float>(sum);
        }
        uint4* d4 = reinterpret_cast<uint4*>(s.x + row * ROW + 32 * b);
        d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
        d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t k, int64_t rb,
        const uint8_t* __restrict__ xq, int64_t m, float* __restrict__ y, int64_t ldy,
        int tiles_m, int tiles_total) {
    __shared__ __align__(16) Smem s;
    // XCD-aware tile order: workgroups are dealt to the 8 XCDs round-robin,
    // so give each XCD a contiguous run of tiles (the M tiles of one weight
    // tile share that XCD's L2).
    const int G = gridDim.x, g = blockIdx.x;
    const int per_xcd = G / 8, rem = G % 8;
    int tile;
    if (g < 8 * per_xcd) tile = (g % 8) * per_xcd + g / 8;
    else tile = 8 * per_xcd + (g - 8 * per_xcd);
    (void)rem;
    if (tile >= tiles_total) return;
    const int64_t m0 = static_cast<int64_t>(tile % tiles_m) * BM;
    const int64_t n0 = static_cast<int64_t>(tile / tiles_m) * BN;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;       // wave tile: tokens 64*wm.., rows 64*wn..
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t xrb = k / 32 * 34;

    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = kBias;

    const int ksteps = static_cast<int>(k / (32 * KB));
    for (int ks = 0; ks < ksteps; ++ks) {
        __syncthreads();
        stage_weights<FMT>(s, w, n, rb, n0, ks);
        stage_acts<FMT>(s, xq, m, xrb, m0, ks);
        __syncthreads();
#pragma unroll 2
        for (int b = 0; b < KB; ++b) {
            v4i A[2], Bv[2];
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                A[ni] = *reinterpret_cast<const v4i*>(s.w + (64 * wn + 32 * ni + l32) * ROW + 32 * b + 16 * h);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                Bv[mi] = *reinterpret_cast<const v4i*>(s.x + (64 * wm + 32 * mi + l32) * ROW + 32 * b + 16 * h);
            float dx[2], ndx[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                dx[mi] = s.dx[b][64 * wm + 32 * mi + l32];
                ndx[mi] = -kBiasF * dx[mi];
            }
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                float dwv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 d4 = *reinterpret_cast<const float4*>(&s.dw[b][64 * wn + 32 * ni + 8 * q + 4 * h]);
                    dwv[4 * q] = d4.x; dwv[4 * q + 1] = d4.y; dwv[4 * q + 2] = d4.z; dwv[4 * q + 3] = d4.w;
                }
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) {
                    const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ni], Bv[mi], bias, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float tq = fmaf(__int_as_float(D[r]), dx[mi], ndx[mi]);
                        acc[mi][ni][r] = fmaf(tq, dwv[r], acc[mi][ni][r]);
                    }
                }
            }
        }
        if constexpr (kHasOffset<FMT>) {
            // additive term: acc[n][m] += sum_b cw[b][n] * sx[b][m], two blocks
            // per fp32 MFMA (A: rows n, k = block; B: columns m)
#pragma unroll
            for (int b2 = 0; b2 < KB; b2 += 2) {
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const float a = s.cw[b2 + h][64 * wn + 32 * ni + l32];
#pragma unroll
                    for (int mi = 0; mi < 2; ++mi) {
                        const float bx = s.sx[b2 + h][64 * wm + 32 * mi + l32];
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bx, acc[mi][ni], 0, 0, 0);
                    }
                }
            }
        }
    }

    // epilogue: lane holds token m = m0 + 64wm + 32mi + l32 and weight rows
    // n = n0 + 64wn + 32ni + 8q + 4h + s (register r = 4q + s)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int64_t gm = m0 + 64 * wm + 32 * mi + l32;
        if (gm >= m) continue;
        float* yr = y + gm * ldy;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t gn = n0 + 64 * wn + 32 * ni + 8 * q + 4 * h;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gn + e < n) yr[gn + e] = acc[mi][ni][4 * q + e];
            }
        }
    }
}

}  // namespace

int gemm_shape_ok(int wt, int64_t k) {
    (void)wt;
    return (k % 256 == 0) ? 0 : -3;
}

int launch_gemm(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t m, float* y,
                int64_t ldy, hipStream_t stream) {
    const int64_t bs = wt == T_Q4_0 ? 18 : wt == T_Q4_1 ? 20 : wt == T_Q8_0 ? 34 : 144;
    const int64_t qk = wt == T_Q4_K ? 256 : 32;
    const int64_t rb = k / qk * bs;
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    if (tiles > 0x7FFFFFFF) return -3;
    const dim3 g(static_cast<unsigned>(tiles)), b(kThreads);
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int tm = static_cast<int>(tiles_m), tt = static_cast<int>(tiles);
    switch (wt) {
        case T_Q4_0: hipLaunchKernelGGL(gemm_kernel<T_Q4_0>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q4_1: hipLaunchKernelGGL(gemm_kernel<T_Q4_1>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q8_0: hipLaunchKernelGGL(gemm_kernel<T_Q8_0>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q4_K: hipLaunchKernelGGL(gemm_kernel<T_Q4_K>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        default: return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace cq
