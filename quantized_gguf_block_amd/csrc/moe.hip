// moe.hip -- routed expert FFN: grouping, grouped GEMM, combine.
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {

// ---- grouping: stable counting sort of (token, slot) pairs by expert ------
// One workgroup of 1024 threads (16 waves).
//  1. histogram of expert ids with LDS integer atomics (totals are order
//     independent), exclusive scan -> offsets;
//  2. pairs are placed chunk by chunk (1024 consecutive pair ids per chunk):
//     inside a wave, lanes holding the same expert find each other with a
//     ballot loop (one ballot per distinct expert); each group's size goes
//     to an LDS table [wave][expert]; a pair's slot is then
//       fill[e] + (same-expert pairs in earlier waves) + (lower lanes of its group)
//     which is its rank in ascending pair order.  No step depends on thread
//     timing, so the output is deterministic.
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(
        const int32_t* __restrict__ ids, int np, int n_experts, int32_t* __restrict__ offsets,
        int32_t* __restrict__ pairs) {
    __shared__ int fill[kMaxExperts];
    __shared__ int scan[kGroupThreads];
    __shared__ uint16_t wcnt[kGroupWaves][kMaxExperts];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

    for (int e = t; e < n_experts; e += kGroupThreads) fill[e] = 0;
    __syncthreads();
    for (int p = t; p < np; p += kGroupThreads) {
        const int e = ids[p];
        if (e >= 0 && e < n_experts) atomicAdd(&fill[e], 1);
    }
    __syncthreads();
    // inclusive Hillis-Steele scan of the counts (n_experts <= 1024 = threads)
    scan[t] = (t < n_experts) ? fill[t] : 0;
    __syncthreads();
    for (int d = 1; d < kGroupThreads; d <<= 1) {
        const int v = (t >= d) ? scan[t - d] : 0;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    if (t < n_experts) {
        const int excl = scan[t] - fill[t];
        offsets[t] = excl;
        fill[t] = excl;  // running fill pointer
    }
    if (t == 0) offsets[n_experts] = scan[n_experts - 1];
    for (int i = t; i < kGroupWaves * n_experts; i += kGroupThreads)
        wcnt[i / n_experts][i % n_experts] = 0;
    __syncthreads();

    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < np; base += kGroupThreads) {
        const int p = base + t;
        const int e = (p < np) ? ids[p] : -1;
        const bool ok = e >= 0 && e < n_experts;
        // lanes of this wave holding the same expert
        uint64_t todo = __ballot(1);
        uint64_t same = 0;
        while (todo) {
            const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
            const int le = __builtin_amdgcn_readlane(e, leader);
            const uint64_t m = __ballot(e == le);
            if (e == le) same = m;
            todo &= ~m;
        }
        const int rank_in_wave = __popcll(same & below);
        if (ok && rank_in_wave == 0) wcnt[wv][e] = static_cast<uint16_t>(__popcll(same));
        __syncthreads();
        if (ok) {
            int before = 0;
            for (int w2 = 0; w2 < wv; ++w2) before += wcnt[w2][e];
            pairs[fill[e] + before + rank_in_wave] = p;
        }
        __syncthreads();
        for (int e2 = t; e2 < n_experts; e2 += kGroupThreads) {
            int c = 0;
            for (int w2 = 0; w2 < kGroupWaves; ++w2) {
                c += wcnt[w2][e2];
                wcnt[w2][e2] = 0;
            }
            fill[e2] += c;
        }
        __syncthreads();
    }
}

int launch_moe_group(const int32_t* ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                     int32_t* offsets, int32_t* pairs, hipStream_t stream) {
    const int np = static_cast<int>(n_tokens * top_k);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, stream, ids, np,
                       static_cast<int>(n_experts), offsets, pairs);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// ---- combine: y[t] = sum_s w[t,s] * d[t*k+s] in slot order ---------------
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ d,
                                                          const float* __restrict__ rw,
                                                          int64_t n_tokens, int top_k, int64_t n,
                                                          float* __restrict__ y, int64_t ldy) {
    const int64_t total = n_tokens * n;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t t = i / n, c = i - t * n;
        float acc = 0.0f;
        for (int s = 0; s < top_k; ++s) {
            const int64_t p = t * top_k + s;
            acc = fmaf(rw[p], d[p * n + c], acc);
        }
        y[t * ldy + c] = acc;
    }
}

int launch_moe_combine(const float* d, const float* route_w, int64_t n_tokens, int64_t top_k,
                       int64_t n, float* y, int64_t ldy, hipStream_t stream) {
    const int64_t total = n_tokens * n;
    int64_t grid = (total + 255) / 256;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                       d, route_w, n_tokens, static_cast<int>(top_k), n, y, ldy);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace cq
