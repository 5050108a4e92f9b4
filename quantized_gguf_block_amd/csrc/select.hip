// select.hip -- greedy arg-max over logit rows and the top-k expert router.
//
// Arg-max (cera 0.5.3 README, "Speculative decoding": the greedy verify
// compares arg-max tokens; Cera README, "Performance": keeping it on the
// device reads a few bytes instead of the logits).  Every value becomes a
// 64-bit key whose high word orders like the float (sign-folded bits, -0
// taken as +0) and whose low word is ~index, so the largest key is the
// largest value at its first index; the maximum of keys does not depend on
// the order of reduction, so the result is deterministic.  Two launches: each
// workgroup reduces a 4096-value chunk of a row to one key in the caller's
// workspace, then one wave per row reduces the chunk keys.
//
// Router (Cera README, "Supported models": each token picks its own 4 of 32
// experts): one wave per token; top_k rounds of a wave-wide key maximum
// (equal logits: smaller expert id first), then the softmax over the chosen
// logits in fp64, summed in slot order, rounded once to fp32.
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {
namespace {

constexpr int kChunk = 4096;          // values per arg-max workgroup
constexpr int kArgThreads = 256;      // 16 values per thread

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;     // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
    return (static_cast<uint64_t>(order_key(v)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// maximum of one key per lane over the wave (butterfly, every lane gets it)
__device__ __forceinline__ uint64_t wave_max64(uint64_t k) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(k & 0xFFFFFFFFu), m));
        const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(k >> 32), m));
        k = umax64(k, (static_cast<uint64_t>(hi) << 32) | lo);
    }
    return k;
}

// Chunk (blockIdx.x) of row blockIdx.y -> keys[row * nchunks + chunk].
// VEC: rows are 16-byte aligned, so each thread reads four float4.
template <bool VEC>
__global__ __launch_bounds__(kArgThreads) void argmax_chunk_kernel(
        const float* __restrict__ y, int64_t n, int64_t ldy, uint64_t* __restrict__ keys,
        int nchunks) {
    const float* row = y + static_cast<int64_t>(blockIdx.y) * ldy;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kChunk;
    uint64_t best = 0;                // below every real key
    if constexpr (VEC) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t e = c0 + 4 * (threadIdx.x + u * kArgThreads);
            v[u] = e + 3 < n ? *reinterpret_cast<const float4*>(row + e) : make_float4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t e = c0 + 4 * (threadIdx.x + u * kArgThreads);
            const float f[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = e + q;
                float val = f[q];
                if (e + 3 >= n) val = i < n ? row[i] : 0.0f;   // ragged tail: scalar reads
                if (i < n) best = umax64(best, make_key(val, static_cast<uint32_t>(i)));
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < kChunk / kArgThreads; ++u) {
            const int64_t i = c0 + threadIdx.x + u * kArgThreads;
            if (i < n) best = umax64(best, make_key(row[i], static_cast<uint32_t>(i)));
        }
    }
    best = wave_max64(best);
    __shared__ uint64_t part[kArgThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = part[0];
#pragma unroll
        for (int w = 1; w < kArgThreads / kWave; ++w) k = umax64(k, part[w]);
        keys[static_cast<int64_t>(blockIdx.y) * nchunks + blockIdx.x] = k;
    }
}

__global__ __launch_bounds__(kWave) void argmax_final_kernel(const uint64_t* __restrict__ keys,
                                                             int nchunks, int32_t* __restrict__ idx) {
    const uint64_t* k = keys + static_cast<int64_t>(blockIdx.x) * nchunks;
    uint64_t best = 0;
    for (int c = threadIdx.x; c < nchunks; c += kWave) best = umax64(best, k[c]);
    best = wave_max64(best);
    if (threadIdx.x == 0)
        idx[blockIdx.x] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

constexpr int kMaxExperts = 1024;
constexpr int kRouterWaves = 4;
constexpr int kMaxTopK = 16;                   // largest top_k the router takes

// One wave per token row (4 per workgroup); PL logits per lane (n_experts
// <= 64 * PL).
template <int PL>
__global__ __launch_bounds__(kWave * kRouterWaves) void topk_softmax_kernel(
        const float* __restrict__ logits, int64_t rows, int n_experts, int64_t ld, int top_k,
        int32_t* __restrict__ ids, float* __restrict__ w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouterWaves + threadIdx.x / kWave;
    if (t >= rows) return;            // the whole wave leaves together
    const float* l = logits + t * ld;
    uint64_t key[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
        const int e = lane + kWave * j;
        key[j] = e < n_experts ? make_key(l[e], static_cast<uint32_t>(e)) : 0;
    }
    // Each round every lane learns the chosen expert; lane s keeps the
    // choice of round s (rounds unrolled, so no register array is indexed
    // at run time).
    int my_sel = 0;
    float my_val = 0.0f, l0f = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
        if (s < top_k) {              // (top_k is uniform: no divergence)
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < PL; ++j) best = umax64(best, key[j]);
            best = wave_max64(best);
            const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFu));
            const float v = l[e];
            if (s == 0) l0f = v;
            if (lane == s) {
                my_sel = e;
                my_val = v;
            }
            // the owner drops the chosen logit from later rounds
#pragma unroll
            for (int j = 0; j < PL; ++j)
                if (lane + kWave * j == e) key[j] = 0;
        }
    }
    // softmax over the chosen logits: one fp64 exp per lane, the sum taken
    // in slot order
    const double l0 = static_cast<double>(l0f);
    const double ex = lane < top_k ? exp(static_cast<double>(my_val) - l0) : 0.0;
    const int lo = __double2loint(ex), hi = __double2hiint(ex);
    double sum = 0.0;
    for (int s = 0; s < top_k; ++s)
        sum += __hiloint2double(__shfl(hi, s), __shfl(lo, s));
    if (lane < top_k) {
        ids[t * top_k + lane] = my_sel;
        w[t * top_k + lane] = static_cast<float>(ex / sum);
    }
}

}  // namespace

int64_t argmax_chunks(int64_t n) { return (n + kChunk - 1) / kChunk; }

int launch_argmax(const float* y, int64_t rows, int64_t n, int64_t ldy, int32_t* idx, void* ws,
                  hipStream_t stream) {
    const int64_t nchunks = argmax_chunks(n);
    if (nchunks > 0x7FFFFFFF || rows > 65535) return -3;
    uint64_t* keys = static_cast<uint64_t*>(ws);
    const dim3 g(static_cast<unsigned>(nchunks), static_cast<unsigned>(rows));
    const bool vec = (reinterpret_cast<uintptr_t>(y) & 15) == 0 && ldy % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(argmax_chunk_kernel<true>, g, dim3(kArgThreads), 0, stream, y, n, ldy,
                           keys, static_cast<int>(nchunks));
    else
        hipLaunchKernelGGL(argmax_chunk_kernel<false>, g, dim3(kArgThreads), 0, stream, y, n, ldy,
                           keys, static_cast<int>(nchunks));
    hipLaunchKernelGGL(argmax_final_kernel, dim3(static_cast<unsigned>(rows)), dim3(kWave), 0,
                       stream, keys, static_cast<int>(nchunks), idx);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_topk_softmax(const float* logits, int64_t rows, int64_t n_experts, int64_t ld,
                        int64_t top_k, int32_t* ids, float* w, hipStream_t stream) {
    const int64_t wgs = (rows + kRouterWaves - 1) / kRouterWaves;
    if (wgs > 0x7FFFFFFF || n_experts > kMaxExperts || top_k > kMaxTopK) return -3;
    const dim3 g(static_cast<unsigned>(wgs)), b(kWave * kRouterWaves);
    const int ne = static_cast<int>(n_experts), tk = static_cast<int>(top_k);
    if (n_experts <= 64)
        hipLaunchKernelGGL(topk_softmax_kernel<1>, g, b, 0, stream, logits, rows, ne, ld, tk, ids, w);
    else if (n_experts <= 128)
        hipLaunchKernelGGL(topk_softmax_kernel<2>, g, b, 0, stream, logits, rows, ne, ld, tk, ids, w);
    else if (n_experts <= 256)
        hipLaunchKernelGGL(topk_softmax_kernel<4>, g, b, 0, stream, logits, rows, ne, ld, tk, ids, w);
    else if (n_experts <= 512)
        hipLaunchKernelGGL(topk_softmax_kernel<8>, g, b, 0, stream, logits, rows, ne, ld, tk, ids, w);
    else
        hipLaunchKernelGGL(topk_softmax_kernel<16>, g, b, 0, stream, logits, rows, ne, ld, tk, ids, w);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace cq
