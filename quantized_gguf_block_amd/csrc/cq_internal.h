// cq_internal.h -- launchers behind the C ABI (host side, HIP runtime).
// Arguments reaching these functions have been validated by cq_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cq {

// Compute-unit count of the current device (cached per device id).
int device_cu_count();

int launch_quantize_q8_0(const float* x, int64_t ldx, int64_t rows, int64_t k, void* xq,
                         hipStream_t stream);
int launch_swiglu_quantize_q8_0(const float* g, const float* u, int64_t ld, int64_t rows,
                                int64_t k, float* h, void* hq, hipStream_t stream);
int launch_gemv(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t batch,
                float* y, int64_t ldy, hipStream_t stream);
// Q4_K GEMV with 4096-value rows on the 4x4x4 int8 matrix cores (gemv_mfma.hip):
// taken for matrices of at least kMfmaMinRows rows, 1..8 activation rows and a
// 16-byte aligned xq; otherwise launch_gemv uses the streaming kernel.
constexpr int64_t kMfmaMinRows = 32768;
bool gemv_q4k_mfma_ok(int64_t n, int64_t k, int64_t batch, const void* xq);
int launch_gemv_q4k_mfma(const void* w, int64_t n, const void* xq, int64_t batch, float* y,
                         int64_t ldy, hipStream_t stream);
int launch_gemv_swiglu(int wt, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                       const void* xq, int64_t batch, float* h, int64_t ldh, hipStream_t stream);
int launch_moe_gemv(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                    const void* xq, int x_per_pair, const int32_t* ids, int64_t n_tokens,
                    int64_t top_k, float* y, int64_t ldy, int32_t* status, hipStream_t stream);
int launch_moe_gemv_swiglu(int wt, const void* w_gate, const void* w_up, int64_t n_experts,
                           int64_t n, int64_t k, const void* xq, const int32_t* ids,
                           int64_t n_tokens, int64_t top_k, float* h, int64_t ldh,
                           int32_t* status, hipStream_t stream);
int64_t argmax_chunks(int64_t n);
int launch_argmax(const float* y, int64_t rows, int64_t n, int64_t ldy, int32_t* idx, void* ws,
                  hipStream_t stream);
int launch_topk_softmax(const float* logits, int64_t rows, int64_t n_experts, int64_t ld,
                        int64_t top_k, int32_t* ids, float* w, hipStream_t stream);
int launch_gemm(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t m,
                float* y, int64_t ldy, hipStream_t stream);
int launch_moe_group(const int32_t* ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                     int32_t* offsets, int32_t* pairs, int32_t* status, hipStream_t stream);
int launch_moe_gemm(int wt, const void* w, int64_t n_experts, int64_t n, int64_t k,
                    const void* xq, int x_per_pair, const int32_t* offsets,
                    const int32_t* pairs, int64_t n_tokens, int64_t top_k, float* y,
                    int64_t ldy, hipStream_t stream);
int launch_moe_gemm2(int wt, const void* w, const void* w2, int64_t n_experts, int64_t n, int64_t k,
                     const void* xq, int x_per_pair, const int32_t* offsets, const int32_t* pairs,
                     int64_t n_tokens, int64_t top_k, float* y, float* y2, int64_t ldy,
                     hipStream_t stream);
int launch_moe_combine(const float* d, const float* route_w, int64_t n_tokens, int64_t top_k,
                       int64_t n, float* y, int64_t ldy, const int32_t* ids, int64_t n_experts,
                       hipStream_t stream);

// One-call routed projection: flag bits as CQ_MOE_* in cq.h.
constexpr int kMoeXPerPair = 1;
constexpr int kMoeOutCombine = 2;
// Byte offsets of the parts of the one-call workspace, and its total size.
struct MoeLayout {
    int64_t status, offsets, pairs, prod, total;
};
MoeLayout moe_layout(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t n, int flags);
// status: where the count of invalid expert ids goes (NULL: the workspace's
// own status word).
int launch_moe_routed(int wt, const void* w, int64_t n_experts, int64_t n, int64_t k,
                      const void* xq, int flags, const int32_t* ids, const float* route_w,
                      int64_t n_tokens, int64_t top_k, float* y, int64_t ldy, uint8_t* ws,
                      int32_t* status, hipStream_t stream);

// The fixed device scratch of the no-allocation routed projection: its size,
// and its address on the current device (resolved once per device; returns
// 0, or -7 without a usable current device, -6 if HIP cannot resolve it).
constexpr int64_t kMoeScratchBytes = int64_t(16) << 20;
constexpr int kMaxScratchDevices = 64;
int moe_scratch_address(uint8_t** ptr);

}  // namespace cq
