// quantize.hip -- Q8_0 activation quantization and the fused SwiGLU +
// Q8_0 requantization of the routed FFN.
//
// Layout: one 32-value block per 8 lanes, each lane loads 16 bytes (4 fp32)
// so a wave reads 8 whole blocks (1 KiB) with fully coalesced 16-byte loads.
// The block amax is a 3-step DPP max inside the 8-lane group; the 34-byte
// output block is written as 2-byte stores (blocks are only 2-byte aligned).
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {

__device__ __forceinline__ void store_block_part(uint8_t* blk, int part, uint32_t packed,
                                                 uint32_t d16) {
    uint16_t* p = reinterpret_cast<uint16_t*>(blk + 2 + 4 * part);
    p[0] = static_cast<uint16_t>(packed & 0xFFFFu);
    p[1] = static_cast<uint16_t>(packed >> 16);
    if (part == 0) *reinterpret_cast<uint16_t*>(blk) = static_cast<uint16_t>(d16);
}

__global__ __launch_bounds__(256) void quantize_q8_0_kernel(
        const float* __restrict__ x, int64_t ldx, int64_t rows, int64_t nb,
        uint8_t* __restrict__ xq) {
    const int64_t total = rows * nb;
    const int part = threadIdx.x & 7;
    for (int64_t blk = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 3;
         blk < total; blk += (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 3) {
        // every lane of a group shares blk, so the group is active together
        const int64_t r = blk / nb, b = blk - r * nb;
        const float4 v = *reinterpret_cast<const float4*>(x + r * ldx + b * 32 + part * 4);
        uint32_t d16;
        const uint32_t packed = q8_0_quantize4(v.x, v.y, v.z, v.w, &d16);
        store_block_part(xq + blk * 34, part, packed, d16);
    }
}

__global__ __launch_bounds__(256) void swiglu_quantize_q8_0_kernel(
        const float* __restrict__ g, const float* __restrict__ u, int64_t ld, int64_t rows,
        int64_t nb, float* __restrict__ h, uint8_t* __restrict__ hq) {
    const int64_t total = rows * nb;
    const int part = threadIdx.x & 7;
    const int64_t k = nb * 32;
    for (int64_t blk = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 3;
         blk < total; blk += (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 3) {
        const int64_t r = blk / nb, b = blk - r * nb;
        const int64_t off = r * ld + b * 32 + part * 4;
        const float4 gv = *reinterpret_cast<const float4*>(g + off);
        const float4 uv = *reinterpret_cast<const float4*>(u + off);
        float4 hv;
        hv.x = swiglu1(gv.x, uv.x);
        hv.y = swiglu1(gv.y, uv.y);
        hv.z = swiglu1(gv.z, uv.z);
        hv.w = swiglu1(gv.w, uv.w);
        if (h) *reinterpret_cast<float4*>(h + r * k + b * 32 + part * 4) = hv;
        uint32_t d16;
        const uint32_t packed = q8_0_quantize4(hv.x, hv.y, hv.z, hv.w, &d16);
        store_block_part(hq + blk * 34, part, packed, d16);
    }
}

static int grid_for_blocks(int64_t total_blocks, int cu_count) {
    // 32 blocks per 256-thread workgroup; cap at a few waves of workgroups
    // per CU and let the grid-stride loop cover the rest.
    const int64_t want = (total_blocks + 31) / 32;
    const int64_t cap = static_cast<int64_t>(cu_count) * 16;
    return static_cast<int>(want < cap ? want : cap);
}

int launch_quantize_q8_0(const float* x, int64_t ldx, int64_t rows, int64_t k, void* xq,
                         hipStream_t stream) {
    const int64_t nb = k / 32;
    const int grid = grid_for_blocks(rows * nb, device_cu_count());
    hipLaunchKernelGGL(quantize_q8_0_kernel, dim3(grid), dim3(256), 0, stream, x, ldx, rows, nb,
                       static_cast<uint8_t*>(xq));
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_swiglu_quantize_q8_0(const float* g, const float* u, int64_t ld, int64_t rows,
                                int64_t k, float* h, void* hq, hipStream_t stream) {
    const int64_t nb = k / 32;
    const int grid = grid_for_blocks(rows * nb, device_cu_count());
    hipLaunchKernelGGL(swiglu_quantize_q8_0_kernel, dim3(grid), dim3(256), 0, stream, g, u, ld,
                       rows, nb, h, static_cast<uint8_t*>(hq));
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace cq
