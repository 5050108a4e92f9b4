// gemv_mfma.hip -- Q4_K decode GEMV for tall matrices with 4096-value rows
// (the 128K-vocabulary LM head), for 1..4 Q8_0 activation rows, with the
// integer dots on the matrix cores.
//
// The streaming kernel of gemv.hip spends 64 of its ~140 VALU instructions
// per row and batch of 4 on v_dot4 (one per 4 values and activation row);
// at 4 activation rows that VALU work, not HBM, sets its duration.  Here the
// dots run on v_mfma_i32_4x4x4_16b_i8 instead: 16 independent 4x4x4 blocks
// per instruction, block b taking activation rows (tokens) 0..3 as its A
// rows and 4 weight rows as its B columns.  What is left on the VALU is the
// nibble split, the per-sub-block scales and the rescale of each integer
// sub-block dot, the same arithmetic (and the same exact int -> fp32 steps)
// as the dot path:
//  * a wave streams 4 consecutive weight rows per step (9216 contiguous
//    bytes, nine 16-byte loads per lane, each load covering 256 bytes of
//    each row) through a register ring into a wave-private LDS buffer;
//  * lane 4b + j takes super-block b (values 256 b .. 256 b + 255) of row j
//    of the step, so block b of each MFMA is super-block b of the 4 rows,
//    and holds that super-block's Q8_0 activations of token j (the A rows of
//    its block) in registers for the whole kernel;
//  * per 32-value sub-block s: 8 MFMAs give the integer dots of the 4 rows
//    with the 4 tokens (lane 4b + j: row j, tokens 0..3); then per token
//    t = float(dot) * dx (exact product rounded once) and acc += t * d*sc_s
//    (Cera README, "Supported models", Q4_K: w = d*sc*q - dmin*m per
//    32-value sub-block; activation Q8_0 blocks of 32, alice-llm 2.0.0
//    README, "Computation Path (Q4_K)");
//  * the min terms -dmin*m_s * dx*sum(q) are a rank-1 update per block and
//    sub-block: one v_mfma_f32_4x4x1_16b_f32 each (A: the lane's token's
//    dx*sum(q), B: the lane's row's -dmin*m_s), into a second accumulator;
//  * the 16 super-block partial sums of each row and token are added across
//    lanes (DPP row rotations, then permlane swaps), one store per step.
// Every token's sums are formed by the same instructions whatever the number
// of activation rows, so row t of a batch is bitwise the batch-1 result for
// that row (the MFMA integer dots are exact, and the f32 rank-1 MFMA forms
// each element independently).
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

constexpr int kSbBytes = 144;                    // Q4_K super-block
constexpr int kRowSb = 16;                       // super-blocks per 4096-value row
constexpr int kRowBytes = kRowSb * kSbBytes;     // 2304
constexpr int kStepRows = 4;
constexpr int kStepBytes = kStepRows * kRowBytes;
constexpr int kLoads = kRowBytes / 256;          // 16-byte loads per lane and step
// LDS row stride: 2304 + 64 bytes makes the 64 lanes' 16-byte reads at
// j * stride + 144 b + 16 u hit all 64 banks once per 16 lanes
constexpr int kRowStride = kRowBytes + 64;
constexpr int kStage = kStepRows * kRowStride;   // bytes per wave
constexpr int kWaves = 4;                        // waves per workgroup
constexpr int kXRow = 4096 / 32 * 34;            // Q8_0 bytes of one activation row
// LDS stride of the activation rows: 4352 + 64 bytes makes the lanes'
// 16-byte reads at j * stride + 272 b + 16 u hit all 64 banks once per 16 lanes
constexpr int kXStride = kXRow + 64;
constexpr int kRing = 2;                         // steps in flight per wave
constexpr int kPar = 2;                          // nibble chunks per MFMA pass

constexpr int kBufWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kBufWord3);
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <bool V> struct Flag { static constexpr bool value = V; };

// Rows [rbeg, rend) of wave g: whole steps of 4 rows, steps_q each and one
// more for the first steps_r waves.
template <int B>
__global__ __launch_bounds__(kWave * kWaves, 1) void gemv_q4k_mfma_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t steps_q, int steps_r,
        const uint8_t* __restrict__ xq, int64_t xrb, float* __restrict__ y, int64_t ldy) {
    static_assert(B >= 1 && B <= 4, "one 4-token MFMA block set");
    __shared__ __align__(16) uint8_t lds[kWaves * kStage];   // per-wave stage buffers
    __shared__ __align__(16) uint8_t xlds[4 * kXStride];       // activation rows
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kWaves + wv;
    const int64_t sbeg = g * steps_q + (g < steps_r ? g : steps_r);
    const int64_t nsteps = steps_q + (g < steps_r ? 1 : 0);
    const int64_t rbeg = kStepRows * sbeg;
    const int64_t rend = rbeg + kStepRows * nsteps < n ? rbeg + kStepRows * nsteps : n;
    uint8_t* stage = lds + wv * kStage;

    // this lane's part of each step's loads: row lane / 16, bytes
    // 256 u + 16 (lane % 16) of it
    const int lrow = lane >> 4;
    const int ld_off = lrow * kRowBytes + 16 * (lane & 15);
    const int st_off = lrow * kRowStride + 16 * (lane & 15);
    // this lane's super-block in the staged step: row j, super-block b
    const int j = lane & 3, b = lane >> 2;
    const int rd_off = j * kRowStride + kSbBytes * b;

    auto load_step = [&](int64_t s, u32x4m* d) {
        const int64_t r0 = rbeg + kStepRows * s;
        const int64_t left = rend - r0;   // rows of the step that exist (may be <= 0)
        const int bytes = left <= 0 ? 0 : (left >= kStepRows ? kStepBytes : static_cast<int>(left) * kRowBytes);
        const __amdgpu_buffer_rsrc_t rs = rsrc(w + (left > 0 ? r0 : 0) * kRowBytes, bytes);
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            d[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, ld_off + 256 * u, 0, kNonTemporal);
    };

    // Activation rows: copied into LDS (rows kXStride apart) with coalesced
    // 16-byte loads issued ahead of the first steps' weight loads, so the
    // wait for the copy does not wait for those.
    constexpr int kPieces = kXRow / 16;                  // 272 per row
    constexpr int XPT = (B * kPieces + kWave * kWaves - 1) / (kWave * kWaves);
    u32x4m xv[XPT];
#pragma unroll
    for (int t = 0; t < XPT; ++t) {
        const int pc = threadIdx.x + t * kWave * kWaves;
        xv[t] = *reinterpret_cast<const u32x4m*>(xq + (pc < B * kPieces ? 16 * pc : 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4m buf[kRing][kLoads];
#pragma unroll
    for (int s = 0; s < kRing; ++s) load_step(s, buf[s]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < XPT; ++t) {
        const int pc = threadIdx.x + t * kWave * kWaves;
        if (pc < B * kPieces) {
            const int row = pc / kPieces;
            *reinterpret_cast<u32x4m*>(xlds + row * kXStride + 16 * (pc - row * kPieces)) = xv[t];
        }
    }
    __syncthreads();
    // This lane's activations, token j's Q8_0 blocks 8 b .. 8 b + 7: the 272
    // bytes at j * kXStride + 272 b (zeros past the batch).
    uint32_t xw[68];
#pragma unroll
    for (int u = 0; u < 17; ++u) {
        u32x4m v = u32x4m{0, 0, 0, 0};
        if (j < B) v = *reinterpret_cast<const u32x4m*>(xlds + j * kXStride + 272 * b + 16 * u);
        xw[4 * u] = v.x; xw[4 * u + 1] = v.y; xw[4 * u + 2] = v.z; xw[4 * u + 3] = v.w;
    }
    // The blocks as MFMA A words, their scales and integer sums.
    uint32_t act[8][8];
    float sxo[8];          // dx * sum(q) (rank-1 A operand of the min terms)
    float dxs[8];          // dx, odd sub-blocks dx / 16 (rank-1 A operand of the scales)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        // block s: fp16 dx at byte 34 s, quants from byte 34 s + 2
        const float dx = h2f((s & 1) ? xw[(34 * s) >> 2] >> 16 : xw[(34 * s) >> 2] & 0xFFFFu);
        int sum = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int o = 34 * s + 2 + 4 * u;
            act[s][u] = (o & 2) ? __builtin_amdgcn_alignbit(xw[(o >> 2) + 1], xw[o >> 2], 16) : xw[o >> 2];
            sum = __builtin_amdgcn_sdot4(static_cast<int>(act[s][u]), 0x01010101, sum, false);
        }
        sxo[s] = dx * static_cast<float>(sum);
        dxs[s] = (s & 1) ? dx * 0.0625f : dx;
    }
    if (nsteps <= 0) return;

    // One step: stage the ring slot, refill it with the step kRing further
    // on (REFILL), compute the 4 rows, reduce across the 16 super-blocks and
    // store.
    auto step = [&](int64_t s, u32x4m* bs, auto refill) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            *reinterpret_cast<u32x4m*>(stage + st_off + 256 * u) = bs[u];
        if constexpr (decltype(refill)::value) {
            __builtin_amdgcn_sched_barrier(0);
            load_step(s + kRing, bs);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        u32x4m hq = *reinterpret_cast<const u32x4m*>(stage + rd_off);
        u32x4m wq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            wq[u] = *reinterpret_cast<const u32x4m*>(stage + rd_off + 16 + 16 * u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // scales and mins of the 8 sub-blocks (6-bit fields of the 12 bytes)
        const float d = h2f(hq.x & 0xFFFFu);
        const float ndmin = -h2f(hq.x >> 16);
        const uint32_t sc03 = hq.y & 0x3F3F3F3Fu, m03 = hq.z & 0x3F3F3F3Fu;
        const uint32_t sc47 = (hq.w & 0x0F0F0F0Fu) | ((hq.y >> 2) & 0x30303030u);
        const uint32_t m47 = ((hq.w >> 4) & 0x0F0F0F0Fu) | ((hq.z >> 2) & 0x30303030u);
        float ws[8], mn[8];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            ws[s2] = d * static_cast<float>((sc03 >> (8 * s2)) & 0xFFu);
            ws[4 + s2] = d * static_cast<float>((sc47 >> (8 * s2)) & 0xFFu);
            mn[s2] = ndmin * static_cast<float>((m03 >> (8 * s2)) & 0xFFu);
            mn[4 + s2] = ndmin * static_cast<float>((m47 >> (8 * s2)) & 0xFFu);
        }
        // odd sub-blocks take the high nibbles h as the signed bytes
        // 16 (h - 8): w = d*sc*(h - 8) + (8 d*sc - dmin*m), so their min term
        // carries 8 d*sc as well
#pragma unroll
        for (int s2 = 1; s2 < 8; s2 += 2) mn[s2] = fmaf(8.0f, ws[s2], mn[s2]);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        v4f accm = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        const v4f zero = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        // kPar nibble chunks at a time, their 2 kPar MFMA chains interleaved
#pragma unroll
        for (int c0 = 0; c0 < 4; c0 += kPar) {
            v4i dlo[kPar], dhi[kPar];
#pragma unroll
            for (int p = 0; p < kPar; ++p) dlo[p] = dhi[p] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int p = 0; p < kPar; ++p) {
                    const int c = c0 + p;
                    const uint32_t wd = wq[2 * c + (u >> 2)][u & 3];
                    const int lo = static_cast<int>(wd & 0x0F0F0F0Fu);
                    const int hi = static_cast<int>((wd & 0xF0F0F0F0u) ^ 0x80808080u);  // 16 (h - 8)
                    dlo[p] = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(act[2 * c][u]), lo, dlo[p], 0, 0, 0);
                    dhi[p] = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(act[2 * c + 1][u]), hi, dhi[p], 0, 0, 0);
                }
#pragma unroll
            for (int p = 0; p < kPar; ++p) {
                const int c = c0 + p;
                // per-element scales dx_t * d*sc_s of the block (rank-1), and
                // the min terms dx_t*sum_t * (-dmin*m_s ...) into accm
                const v4f slo = __builtin_amdgcn_mfma_f32_4x4x1f32(dxs[2 * c], ws[2 * c], zero, 0, 0, 0);
                const v4f shi = __builtin_amdgcn_mfma_f32_4x4x1f32(dxs[2 * c + 1], ws[2 * c + 1], zero, 0, 0, 0);
                accm = __builtin_amdgcn_mfma_f32_4x4x1f32(sxo[2 * c], mn[2 * c], accm, 0, 0, 0);
                accm = __builtin_amdgcn_mfma_f32_4x4x1f32(sxo[2 * c + 1], mn[2 * c + 1], accm, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < B; ++t) {
                    acc[t] = fmaf(static_cast<float>(dlo[p][t]), slo[t], acc[t]);
                    acc[t] = fmaf(static_cast<float>(dhi[p][t]), shi[t], acc[t]);
                }
            }
        }
        // sum over the 16 super-blocks (lanes 4 b + j, b = 0..15): within each
        // row of 16 lanes by DPP rotations, then across the rows; the result
        // for token t sits in row {0, 2, 1, 3}[t], in its lanes 0..3 (j)
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float x = t < B ? acc[t] + accm[t] : 0.0f;
            x += __int_as_float(dpp_i<0x124>(__float_as_int(x)));   // row_ror:4
            x += __int_as_float(dpp_i<0x128>(__float_as_int(x)));   // row_ror:8
            v[t] = x;
        }
        const auto ab = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[1]), false, false);
        const auto cd = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2]), __float_as_uint(v[3]), false, false);
        const float s01 = __uint_as_float(ab[0]) + __uint_as_float(ab[1]);
        const float s23 = __uint_as_float(cd[0]) + __uint_as_float(cd[1]);
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
        const float tot = __uint_as_float(q[0]) + __uint_as_float(q[1]);
        const int rowg = lane >> 4;
        const int tok = rowg == 1 ? 2 : (rowg == 2 ? 1 : rowg);
        const int64_t r = rbeg + kStepRows * s + (lane & 3);
        if ((lane & 15) < 4 && tok < B && r < rend) y[tok * ldy + r] = tot;
    };

    int64_t s = 0;
    for (; s + kRing < nsteps; s += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) step(s + i, buf[i], Flag<true>{});
    }
#pragma unroll
    for (int i = 0; i < kRing; ++i)
        if (s + i < nsteps) step(s + i, buf[i], Flag<false>{});
}

template <int B>
int launch_b(const uint8_t* w, int64_t n, const uint8_t* xq, int64_t xrb, float* y, int64_t ldy,
             hipStream_t stream) {
    // one workgroup (one wave per SIMD) per CU: two per CU (the register
    // budget allows it) took 47.2 against 46.8 us for the 128256 x 4096
    // matrix at batch 1
    auto kern = gemv_q4k_mfma_kernel<B>;
    const int64_t steps = (n + kStepRows - 1) / kStepRows;
    int64_t waves = static_cast<int64_t>(device_cu_count()) * kWaves;
    if (waves > steps) waves = steps;
    // as few waves as keep the most steps per wave: nearly all of them then
    // run that many steps and end together (128256 rows: 1004 waves, 940 of
    // them with 32 steps, instead of 1024 waves, 320 with 32)
    const int64_t spw = (steps + waves - 1) / waves;
    waves = (steps + spw - 1) / spw;
    const int64_t wgs = (waves + kWaves - 1) / kWaves, nw = wgs * kWaves;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(wgs)), dim3(kWave * kWaves), 0, stream, w, n,
                       steps / nw, static_cast<int>(steps % nw), xq, xrb, y, ldy);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace

bool gemv_q4k_mfma_ok(int64_t n, int64_t k, int64_t batch, const void* xq) {
    return k == 4096 && n >= kMfmaMinRows && batch >= 1 && batch <= 8 &&
           (reinterpret_cast<uintptr_t>(xq) & 15) == 0;
}

// Batches of 5..8 rows run as two launches (rows 0..3, then the rest), so
// every row still takes the 4-token kernel.
int launch_gemv_q4k_mfma(const void* w, int64_t n, const void* xq, int64_t batch, float* y,
                         int64_t ldy, hipStream_t stream) {
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int64_t xrb = kXRow;
    int rc = 0;
    for (int64_t t0 = 0; t0 < batch && rc == 0; t0 += 4) {
        const int64_t bt = batch - t0 < 4 ? batch - t0 : 4;
        const uint8_t* xt = xp + t0 * xrb;
        float* yt = y + t0 * ldy;
        switch (bt) {
            case 1: rc = launch_b<1>(wp, n, xt, xrb, yt, ldy, stream); break;
            case 2: rc = launch_b<2>(wp, n, xt, xrb, yt, ldy, stream); break;
            case 3: rc = launch_b<3>(wp, n, xt, xrb, yt, ldy, stream); break;
            default: rc = launch_b<4>(wp, n, xt, xrb, yt, ldy, stream); break;
        }
    }
    return rc;
}

}  // namespace cq
