// cq_device.h -- gfx950 device helpers shared by the libcq kernels:
// fp16 field access, 2-byte-aligned LDS reads, wave64 DPP reductions and
// the Q8_0 block quantizer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cq {

constexpr int kWave = 64;

// h = fp32( silu(g) * u ) with silu(z) = z / (1 + exp(-z)) evaluated in fp64
// and rounded once.
__device__ __forceinline__ float swiglu1(float g, float u) {
    const double z = static_cast<double>(g);
    const double s = z / (1.0 + exp(-z));
    return static_cast<float>(s * static_cast<double>(u));
}

// ---- fp16 ---------------------------------------------------------------
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}
// round to nearest even, subnormals kept (v_cvt_f16_f32)
__device__ __forceinline__ uint32_t f2h_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---- LDS reads at 2-byte-aligned offsets -------------------------------
// N consecutive dwords starting at byte offset `off` (even) of an LDS byte
// array: read N+1 aligned dwords and funnel-shift by 0 or 16 bits.  The
// array must have 4 bytes of slack past the last byte read.
template <int N>
__device__ __forceinline__ void lds_dwords_a2(const uint8_t* lds, int off, uint32_t* out) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (off & ~3));
    const uint32_t sh = static_cast<uint32_t>(off & 2) << 3;
    uint32_t w[N + 1];
#pragma unroll
    for (int t = 0; t <= N; ++t) w[t] = p[t];
#pragma unroll
    for (int t = 0; t < N; ++t) out[t] = __builtin_amdgcn_alignbit(w[t + 1], w[t], sh);
}

__device__ __forceinline__ uint32_t lds_u16(const uint8_t* lds, int off) {
    return *reinterpret_cast<const uint16_t*>(lds + off);
}

// ---- wave64 reductions (DPP) -------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over all 64 lanes; the total is returned in every lane (read back
// from lane 63, where the row broadcasts accumulate it).  Every lane of the
// wave must be active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);          // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);          // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);         // row_half_mirror
    v += dpp_f<0x140>(v);         // row_mirror: every lane holds its row sum
    v += dpp_f<0x142, 0xA>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp_f<0x143, 0xC>(v);    // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Max over each aligned group of 8 lanes, result in all 8 lanes.
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    return v;
}

// ---- Q8_0 block quantization, one block per 8 lanes, 4 values per lane --
// Same single-rounding fp32 operations as the contract: amax, 127/amax,
// x*id rounded to nearest even and clamped, fp16(amax/127).  Returns the
// four packed int8 quants of this lane; *d16 gets the scale bits.
__device__ __forceinline__ uint32_t q8_0_quantize4(float x0, float x1, float x2, float x3,
                                                   uint32_t* d16) {
    float a = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
    const float amax = group8_max(a);
    const float id = 127.0f / amax;          // correctly rounded division
    *d16 = f2h_bits(amax / 127.0f);
    const float xs[4] = {x0, x1, x2, x3};
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p = xs[i] * id;
        float r = __builtin_rintf(p);        // v_rndne_f32: ties to even
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int q = (p != p) ? 0 : static_cast<int>(r);   // 0 * inf -> 0
        packed |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * i);
    }
    return packed;
}

}  // namespace cq
