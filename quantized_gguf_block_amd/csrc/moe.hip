// moe.hip -- routed expert FFN: grouping, grouped GEMM, combine.
#include "cq_device.h"
#include "cq_internal.h"

#include <mutex>

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
// Pairs whose id lies outside [0, n_experts) are placed in no group; their
// count is stored to *status (0 when every id is valid), so a caller that
// reads it after the stream reaches this kernel knows whether the grouping
// is whole.
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(
        const int32_t* __restrict__ ids, int np, int n_experts, int32_t* __restrict__ offsets,
        int32_t* __restrict__ pairs, int32_t* __restrict__ status) {
    __shared__ int fill[kMaxExperts];
    __shared__ uint16_t wcnt[kGroupWaves][kMaxExperts];
    __shared__ int invalid;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

    for (int e = t; e < n_experts; e += kGroupThreads) fill[e] = 0;
    if (t == 0) invalid = 0;
    __syncthreads();
    int bad = 0;
    for (int p = t; p < np; p += kGroupThreads) {
        const int e = ids[p];
        if (e >= 0 && e < n_experts) atomicAdd(&fill[e], 1);
        else ++bad;
    }
    if (bad) atomicAdd(&invalid, bad);
    __syncthreads();
    if (t == 0) *status = invalid;
    // exclusive scan of the counts by wave 0, 64 experts at a time (a
    // wave-level inclusive scan plus the running carry)
    if (wv == 0) {
        int carry = 0;
        for (int e0 = 0; e0 < n_experts; e0 += 64) {
            const int e = e0 + lane;
            const int c = e < n_experts ? fill[e] : 0;
            int v = c;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(v, d, 64);
                if (lane >= d) v += o;
            }
            if (e < n_experts) {
                offsets[e] = carry + v - c;
                fill[e] = carry + v - c;  // running fill pointer
            }
            carry += __shfl(v, 63, 64);
        }
        if (lane == 0) offsets[n_experts] = carry;
    }
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
                     int32_t* offsets, int32_t* pairs, int32_t* status, hipStream_t stream) {
    const int np = static_cast<int>(n_tokens * top_k);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, stream, ids, np,
                       static_cast<int>(n_experts), offsets, pairs, status);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// ---- combine: y[t] = sum_s w[t,s] * d[t*k+s] in slot order ---------------
// Workgroup (column chunk, tokens blockIdx.y, + gridDim.y, ...): each thread
// four consecutive columns, with 16-byte loads and stores when d and y allow
// them; the route weights of a token are wave-uniform.  With ids given (the
// one-call routed projection), a slot whose id lies outside [0, n_experts)
// has no product row and adds nothing.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ d,
                                                          const float* __restrict__ rw,
                                                          int64_t n_tokens, int top_k, int64_t n,
                                                          float* __restrict__ y, int64_t ldy,
                                                          const int32_t* __restrict__ ids,
                                                          int n_experts) {
    const int64_t c = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (c >= n) return;
    const bool vec = (n & 3) == 0 && (ldy & 3) == 0 && (reinterpret_cast<uintptr_t>(d) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(y) & 15) == 0;
    for (int64_t t = blockIdx.y; t < n_tokens; t += gridDim.y) {
        const float* dp = d + t * top_k * n;
        if (vec) {
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int s = 0; s < top_k; ++s) {
                if (ids) {
                    const int e = ids[t * top_k + s];
                    if (e < 0 || e >= n_experts) continue;
                }
                const float wgt = rw[t * top_k + s];
                const float4 v = *reinterpret_cast<const float4*>(dp + s * n + c);
                acc.x = fmaf(wgt, v.x, acc.x);
                acc.y = fmaf(wgt, v.y, acc.y);
                acc.z = fmaf(wgt, v.z, acc.z);
                acc.w = fmaf(wgt, v.w, acc.w);
            }
            *reinterpret_cast<float4*>(y + t * ldy + c) = acc;
        } else {
            for (int64_t cc = c; cc < c + 4 && cc < n; ++cc) {
                float acc = 0.0f;
                for (int s = 0; s < top_k; ++s) {
                    if (ids) {
                        const int e = ids[t * top_k + s];
                        if (e < 0 || e >= n_experts) continue;
                    }
                    acc = fmaf(rw[t * top_k + s], dp[s * n + cc], acc);
                }
                y[t * ldy + cc] = acc;
            }
        }
    }
}

int launch_moe_combine(const float* d, const float* route_w, int64_t n_tokens, int64_t top_k,
                       int64_t n, float* y, int64_t ldy, const int32_t* ids, int64_t n_experts,
                       hipStream_t stream) {
    const int64_t gx = (n + 1023) / 1024;
    const int64_t gy = n_tokens < 4096 ? n_tokens : 4096;
    if (gx > 0x7FFFFFFF) return -3;
    hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                       dim3(256), 0, stream, d, route_w, n_tokens, static_cast<int>(top_k), n, y, ldy,
                       ids, static_cast<int>(n_experts));
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// ---- the one-call routed projection ------------------------------------------
// Workspace layout (each part 256-byte aligned): the status word, the
// offsets [n_experts + 1], the grouped pair list [n_tokens * top_k] and,
// when the per-pair products are combined, those products fp32
// [n_tokens * top_k][n].
static int64_t align256(int64_t b) { return (b + 255) & ~static_cast<int64_t>(255); }

MoeLayout moe_layout(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t n, int flags) {
    MoeLayout L;
    const int64_t np = n_tokens * top_k;
    L.status = 0;
    L.offsets = 256;
    L.pairs = L.offsets + align256(4 * (n_experts + 1));
    L.prod = L.pairs + align256(4 * (np > 0 ? np : 1));
    L.total = (flags & kMoeOutCombine) ? L.prod + align256(4 * np * n) : L.prod;
    return L;
}

int launch_moe_routed(int wt, const void* w, int64_t n_experts, int64_t n, int64_t k,
                      const void* xq, int flags, const int32_t* ids, const float* route_w,
                      int64_t n_tokens, int64_t top_k, float* y, int64_t ldy, uint8_t* ws,
                      int32_t* status, hipStream_t stream) {
    const MoeLayout L = moe_layout(n_tokens, top_k, n_experts, n, flags);
    if (!status) status = reinterpret_cast<int32_t*>(ws + L.status);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* pairs = reinterpret_cast<int32_t*>(ws + L.pairs);
    const bool combine = (flags & kMoeOutCombine) != 0;
    if (int rc = launch_moe_group(ids, n_tokens, top_k, n_experts, offsets, pairs, status, stream))
        return rc;
    float* prod = combine ? reinterpret_cast<float*>(ws + L.prod) : y;
    if (int rc = launch_moe_gemm(wt, w, n_experts, n, k, xq, (flags & kMoeXPerPair) ? 1 : 0,
                                 offsets, pairs, n_tokens, top_k, prod, combine ? n : ldy, stream))
        return rc;
    if (combine)
        return launch_moe_combine(prod, route_w, n_tokens, top_k, n, y, ldy, ids, n_experts, stream);
    return 0;
}

// ---- fixed device scratch for callers that cannot allocate ------------------
// One array per device, the size of the largest workspace the no-allocation
// routed projection accepts.  In host code its name is only a stand-in: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current and kept here.
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

int moe_scratch_address(uint8_t** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -7;
    if (dev >= kMaxScratchDevices) return -7;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -6;
        g_scratch_dev[dev] = p;
    }
    *ptr = static_cast<uint8_t*>(g_scratch_dev[dev]);
    return 0;
}

}  // namespace cq
