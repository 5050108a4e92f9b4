// cq_api.cpp -- the extern "C" entry points declared in include/cq.h.
//
// Every argument is validated here, on the host, before any HIP call; an
// invalid call returns its cq_status without touching the device.  Valid
// calls go to the launchers in cq_internal.h, which enqueue kernels on the
// caller's stream and return at once.
#include "../../include/cq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "cq_internal.h"

namespace cq {

int gemv_shape_ok(int wt, int64_t k, int64_t batch);  // gemv.hip
int gemv_swiglu_shape_ok(int wt, int64_t k, int64_t batch);  // gemv.hip
int moe_gemv_shape_ok(int wt, int64_t k, int64_t npairs);     // gemv.hip
int gemm_shape_ok(int wt, int64_t n, int64_t k);       // gemm.hip
int moe_shape_ok(int wt, int64_t n, int64_t k);        // moe.hip

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int64_t elems(int t) {
    switch (t) {
        case CQ_Q4_0: case CQ_Q4_1: case CQ_Q8_0: return 32;
        case CQ_Q4_K: case CQ_Q5_K: case CQ_Q6_K: return 256;
        case CQ_Q1_0: case CQ_TQ2: return 128;
        default: return -1;
    }
}
int64_t bytes(int t) {
    switch (t) {
        case CQ_Q4_0: return 18;
        case CQ_Q4_1: return 20;
        case CQ_Q8_0: return 34;
        case CQ_Q4_K: return 144;
        case CQ_Q5_K: return 176;
        case CQ_Q1_0: return 18;
        case CQ_TQ2: return 34;
        case CQ_Q6_K: return 210;
        default: return -1;
    }
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Common checks for a weight operand: type, k, pointer alignment.
int check_weights(int wt, const void* w, int64_t n, int64_t k) {
    if (elems(wt) < 0) return CQ_ERR_UNSUPPORTED_TYPE;
    if (n < 0 || k <= 0) return CQ_ERR_INVALID_ARG;
    if (k % elems(wt) != 0 || k % 32 != 0 || k > CQ_MAX_K) return CQ_ERR_SHAPE;
    if (n > 0 && !w) return CQ_ERR_INVALID_ARG;
    if (!aligned(w, 16)) return CQ_ERR_ALIGNMENT;
    return CQ_OK;
}

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CQ_ERR_NO_DEVICE;
    return CQ_OK;
}

int status_of(int rc) { return rc == 0 ? CQ_OK : rc; }

}  // namespace

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

}  // namespace cq

using namespace cq;

extern "C" {

int cq_abi_version(void) { return CQ_ABI_VERSION; }

const char* cq_status_string(int status) {
    switch (status) {
        case CQ_OK: return "CQ_OK";
        case CQ_ERR_INVALID_ARG: return "CQ_ERR_INVALID_ARG: null pointer, negative size or bad flag";
        case CQ_ERR_UNSUPPORTED_TYPE: return "CQ_ERR_UNSUPPORTED_TYPE: weight type not supported by this call (Q4_0, Q4_1, Q8_0, Q4_K, Q5_K, Q6_K; Q1_0 and TQ2 in the GEMV entry points)";
        case CQ_ERR_SHAPE: return "CQ_ERR_SHAPE: k is not a whole number of blocks or exceeds the kernel's limit";
        case CQ_ERR_ALIGNMENT: return "CQ_ERR_ALIGNMENT: pointer or leading dimension misaligned";
        case CQ_ERR_WORKSPACE: return "CQ_ERR_WORKSPACE: workspace smaller than required or misaligned";
        case CQ_ERR_HIP: return "CQ_ERR_HIP: a HIP runtime call failed";
        case CQ_ERR_NO_DEVICE: return "CQ_ERR_NO_DEVICE: no HIP device is current";
        case CQ_ERR_SCRATCH_LIMIT: return "CQ_ERR_SCRATCH_LIMIT: the call needs more than the fixed device scratch of the no-allocation entry point (CQ_MOE_NOALLOC_MAX_BYTES)";
        default: return "unknown cq status";
    }
}

int64_t cq_block_elems(int type) { return elems(type); }
int64_t cq_block_bytes(int type) { return bytes(type); }
int64_t cq_row_bytes(int type, int64_t k) {
    if (elems(type) < 0 || k < 0 || k % elems(type) != 0) return -1;
    return k / elems(type) * bytes(type);
}

int cq_quantize_q8_0(const float* x, int64_t ldx, int64_t rows, int64_t k, void* xq,
                     cq_stream_t stream) {
    if (rows < 0 || k <= 0 || ldx < k) return CQ_ERR_INVALID_ARG;
    if (k % 32 != 0 || k > CQ_MAX_K) return CQ_ERR_SHAPE;
    if (rows == 0) return CQ_OK;
    if (!x || !xq) return CQ_ERR_INVALID_ARG;
    if (!aligned(x, 16) || ldx % 4 != 0 || !aligned(xq, 2)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_quantize_q8_0(x, ldx, rows, k, xq, reinterpret_cast<hipStream_t>(stream)));
}

int cq_gemv(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t batch,
            float* y, int64_t ldy, cq_stream_t stream) {
    if (int rc = check_weights(wt, w, n, k)) return rc;
    if (batch < 1 || batch > CQ_GEMV_MAX_BATCH || ldy < n) return CQ_ERR_INVALID_ARG;
    if (k > CQ_GEMV_MAX_K || gemv_shape_ok(wt, k, batch) != 0) return CQ_ERR_SHAPE;
    if (n == 0) return CQ_OK;
    if (!xq || !y) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 2) || !aligned(y, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_gemv(wt, w, n, k, xq, batch, y, ldy, reinterpret_cast<hipStream_t>(stream)));
}

int cq_gemv_swiglu(int wt, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                   const void* xq, int64_t batch, float* h, int64_t ldh, cq_stream_t stream) {
    if (int rc = check_weights(wt, w_gate, n, k)) return rc;
    if (int rc = check_weights(wt, w_up, n, k)) return rc;
    if (batch < 1 || batch > CQ_GEMV_MAX_BATCH || ldh < n) return CQ_ERR_INVALID_ARG;
    if (gemv_swiglu_shape_ok(wt, k, batch) != 0) return CQ_ERR_SHAPE;
    if (n == 0) return CQ_OK;
    if (!xq || !h) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 16) || !aligned(h, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_gemv_swiglu(wt, w_gate, w_up, n, k, xq, batch, h, ldh,
                                        reinterpret_cast<hipStream_t>(stream)));
}

// shared argument checks of the two decode-MoE GEMV entry points
static int check_moe_gemv(int wt, const void* w, int64_t n_experts, int64_t n, int64_t k,
                          const int32_t* ids, int64_t n_tokens, int64_t top_k, int64_t ldy) {
    if (int rc = check_weights(wt, w, n, k)) return rc;
    if (n_experts < 1 || n_experts > 1024 || n_tokens < 0 || top_k < 1 || top_k > n_experts ||
        ldy < n)
        return CQ_ERR_INVALID_ARG;
    if (moe_gemv_shape_ok(wt, k, n_tokens * top_k) != 0) return CQ_ERR_SHAPE;
    if (!aligned(ids, 4)) return CQ_ERR_ALIGNMENT;
    return CQ_OK;
}

int cq_moe_gemv(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                const void* xq, int x_per_pair, const int32_t* expert_ids, int64_t n_tokens,
                int64_t top_k, float* y, int64_t ldy, int32_t* status, cq_stream_t stream) {
    if (x_per_pair != 0 && x_per_pair != 1) return CQ_ERR_INVALID_ARG;
    if (int rc = check_moe_gemv(wt, w_experts, n_experts, n, k, expert_ids, n_tokens, top_k, ldy))
        return rc;
    if (n == 0 || n_tokens == 0) return CQ_OK;
    if (!xq || !expert_ids || !y || !status) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 16) || !aligned(y, 4) || !aligned(status, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_gemv(wt, w_experts, n_experts, n, k, xq, x_per_pair, expert_ids,
                                     n_tokens, top_k, y, ldy, status,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int cq_moe_gemv_swiglu(int wt, const void* w_gate_experts, const void* w_up_experts,
                       int64_t n_experts, int64_t n, int64_t k, const void* xq,
                       const int32_t* expert_ids, int64_t n_tokens, int64_t top_k, float* h,
                       int64_t ldh, int32_t* status, cq_stream_t stream) {
    if (int rc = check_moe_gemv(wt, w_gate_experts, n_experts, n, k, expert_ids, n_tokens, top_k,
                                ldh))
        return rc;
    if (int rc = check_weights(wt, w_up_experts, n, k)) return rc;
    if (n == 0 || n_tokens == 0) return CQ_OK;
    if (!xq || !expert_ids || !h || !status) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 16) || !aligned(h, 4) || !aligned(status, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_gemv_swiglu(wt, w_gate_experts, w_up_experts, n_experts, n, k, xq,
                                            expert_ids, n_tokens, top_k, h, ldh, status,
                                            reinterpret_cast<hipStream_t>(stream)));
}

size_t cq_argmax_workspace_bytes(int64_t rows, int64_t n) {
    if (rows < 0 || n < 1 || n > 0x7FFFFFFF) return 0;
    return static_cast<size_t>(rows) * static_cast<size_t>(argmax_chunks(n)) * 8u;
}

int cq_argmax(const float* y, int64_t rows, int64_t n, int64_t ldy, int32_t* idx, void* workspace,
              size_t ws_bytes, cq_stream_t stream) {
    if (rows < 0 || n < 1 || ldy < n) return CQ_ERR_INVALID_ARG;
    if (rows > 65535 || n > 0x7FFFFFFF) return CQ_ERR_SHAPE;
    if (rows == 0) return CQ_OK;
    if (!y || !idx || !workspace) return CQ_ERR_INVALID_ARG;
    if (!aligned(y, 4) || !aligned(idx, 4)) return CQ_ERR_ALIGNMENT;
    if (!aligned(workspace, 8) || ws_bytes < cq_argmax_workspace_bytes(rows, n))
        return CQ_ERR_WORKSPACE;
    if (int rc = check_device()) return rc;
    return status_of(launch_argmax(y, rows, n, ldy, idx, workspace,
                                   reinterpret_cast<hipStream_t>(stream)));
}

int cq_topk_softmax(const float* logits, int64_t rows, int64_t n_experts, int64_t ld,
                    int64_t top_k, int32_t* ids, float* w, cq_stream_t stream) {
    if (rows < 0 || n_experts < 1 || n_experts > 1024 || top_k < 1 || top_k > 16 ||
        top_k > n_experts || ld < n_experts)
        return CQ_ERR_INVALID_ARG;
    if (rows > (int64_t(1) << 31)) return CQ_ERR_SHAPE;
    if (rows == 0) return CQ_OK;
    if (!logits || !ids || !w) return CQ_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_topk_softmax(logits, rows, n_experts, ld, top_k, ids, w,
                                         reinterpret_cast<hipStream_t>(stream)));
}

int cq_gemm(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t m, float* y,
            int64_t ldy, cq_stream_t stream) {
    if (int rc = check_weights(wt, w, n, k)) return rc;
    if (wt == CQ_Q1_0 || wt == CQ_TQ2) return CQ_ERR_UNSUPPORTED_TYPE;
    if (m < 0 || ldy < n) return CQ_ERR_INVALID_ARG;
    if (k % 256 != 0 || gemm_shape_ok(wt, n, k) != 0) return CQ_ERR_SHAPE;
    if (n == 0 || m == 0) return CQ_OK;
    if (!xq || !y) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 4) || !aligned(y, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_gemm(wt, w, n, k, xq, m, y, ldy, reinterpret_cast<hipStream_t>(stream)));
}

int cq_moe_group(const int32_t* expert_ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                 int32_t* offsets, int32_t* pairs, int32_t* status, cq_stream_t stream) {
    if (n_tokens < 0 || top_k < 1 || n_experts < 1 || n_experts > 1024 || top_k > n_experts)
        return CQ_ERR_INVALID_ARG;
    if (n_tokens * top_k > (int64_t(1) << 24)) return CQ_ERR_SHAPE;
    if (!offsets || !status || (n_tokens > 0 && (!expert_ids || !pairs))) return CQ_ERR_INVALID_ARG;
    if (!aligned(expert_ids, 4) || !aligned(offsets, 4) || !aligned(pairs, 4) ||
        !aligned(status, 4))
        return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_group(expert_ids, n_tokens, top_k, n_experts, offsets, pairs,
                                      status, reinterpret_cast<hipStream_t>(stream)));
}

// shared checks of the grouped expert products (one-call and split forms)
static int check_moe_gemm(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                          int64_t n_tokens, int64_t top_k, int64_t ldy) {
    if (int rc = check_weights(wt, w_experts, n, k)) return rc;
    if (wt == CQ_Q1_0 || wt == CQ_TQ2) return CQ_ERR_UNSUPPORTED_TYPE;
    if (n_experts < 1 || n_experts > 1024 || n_tokens < 0 || top_k < 1 || top_k > n_experts ||
        ldy < n)
        return CQ_ERR_INVALID_ARG;
    if (k % 256 != 0 || moe_shape_ok(wt, n, k) != 0) return CQ_ERR_SHAPE;
    if (n_tokens * top_k > (int64_t(1) << 24)) return CQ_ERR_SHAPE;
    return CQ_OK;
}

int cq_moe_gemm_grouped(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                        const void* xq, int x_per_pair, const int32_t* offsets,
                        const int32_t* pairs, int64_t n_tokens, int64_t top_k, float* y,
                        int64_t ldy, cq_stream_t stream) {
    if (x_per_pair != 0 && x_per_pair != 1) return CQ_ERR_INVALID_ARG;
    if (int rc = check_moe_gemm(wt, w_experts, n_experts, n, k, n_tokens, top_k, ldy)) return rc;
    if (n == 0 || n_tokens == 0) return CQ_OK;
    if (!xq || !offsets || !pairs || !y) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 2) || !aligned(offsets, 4) || !aligned(pairs, 4) || !aligned(y, 4))
        return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_gemm(wt, w_experts, n_experts, n, k, xq, x_per_pair, offsets,
                                     pairs, n_tokens, top_k, y, ldy,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int cq_moe_gemm_grouped2(int wt, const void* w_a_experts, const void* w_b_experts,
                         int64_t n_experts, int64_t n, int64_t k, const void* xq, int x_per_pair,
                         const int32_t* offsets, const int32_t* pairs, int64_t n_tokens,
                         int64_t top_k, float* y_a, float* y_b, int64_t ldy, cq_stream_t stream) {
    if (x_per_pair != 0 && x_per_pair != 1) return CQ_ERR_INVALID_ARG;
    if (int rc = check_moe_gemm(wt, w_a_experts, n_experts, n, k, n_tokens, top_k, ldy)) return rc;
    if (int rc = check_weights(wt, w_b_experts, n, k)) return rc;
    if (n == 0 || n_tokens == 0) return CQ_OK;
    if (!xq || !offsets || !pairs || !y_a || !y_b) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 2) || !aligned(offsets, 4) || !aligned(pairs, 4) || !aligned(y_a, 4) ||
        !aligned(y_b, 4))
        return CQ_ERR_ALIGNMENT;
    // the two outputs' extents (rows of ldy floats, the last one n long) may not overlap
    using u128 = unsigned __int128;
    const u128 a0 = reinterpret_cast<uintptr_t>(y_a), b0 = reinterpret_cast<uintptr_t>(y_b);
    const u128 span = (static_cast<u128>(n_tokens * top_k - 1) * static_cast<uint64_t>(ldy) +
                       static_cast<uint64_t>(n)) * 4;
    if (a0 < b0 + span && b0 < a0 + span) return CQ_ERR_INVALID_ARG;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_gemm2(wt, w_a_experts, w_b_experts, n_experts, n, k, xq, x_per_pair,
                                      offsets, pairs, n_tokens, top_k, y_a, y_b, ldy,
                                      reinterpret_cast<hipStream_t>(stream)));
}

static bool moe_flags_ok(int flags) {
    return (flags & ~(CQ_MOE_X_PER_PAIR | CQ_MOE_OUT_COMBINE)) == 0;
}

size_t cq_moe_workspace_bytes(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t n,
                              int flags) {
    if (n_tokens < 0 || top_k < 1 || n_experts < 1 || n_experts > 1024 || top_k > n_experts ||
        n < 0 || !moe_flags_ok(flags) || n_tokens * top_k > (int64_t(1) << 24) ||
        n > (int64_t(1) << 24))
        return 0;
    return static_cast<size_t>(moe_layout(n_tokens, top_k, n_experts, n, flags).total);
}

int cq_moe_gemm(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                const void* xq, int flags, const int32_t* expert_ids, const float* route_w,
                int64_t n_tokens, int64_t top_k, float* y, int64_t ldy, void* workspace,
                size_t ws_bytes, cq_stream_t stream) {
    if (!moe_flags_ok(flags)) return CQ_ERR_INVALID_ARG;
    if (int rc = check_moe_gemm(wt, w_experts, n_experts, n, k, n_tokens, top_k, ldy)) return rc;
    if (n > (int64_t(1) << 24)) return CQ_ERR_SHAPE;
    if (n == 0 || n_tokens == 0) return CQ_OK;
    const bool combine = (flags & CQ_MOE_OUT_COMBINE) != 0;
    if (!xq || !expert_ids || !y || !workspace || (combine && !route_w)) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 2) || !aligned(expert_ids, 4) || !aligned(y, 4) ||
        (combine && !aligned(route_w, 4)))
        return CQ_ERR_ALIGNMENT;
    if (!aligned(workspace, 256) ||
        ws_bytes < cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags))
        return CQ_ERR_WORKSPACE;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_routed(wt, w_experts, n_experts, n, k, xq, flags, expert_ids,
                                       route_w, n_tokens, top_k, y, ldy,
                                       static_cast<uint8_t*>(workspace), nullptr,
                                       reinterpret_cast<hipStream_t>(stream)));
}

int cq_moe_gemm_noalloc(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                        const void* xq, int flags, const int32_t* expert_ids,
                        const float* route_w, int64_t n_tokens, int64_t top_k, float* y,
                        int64_t ldy, int32_t* status, cq_stream_t stream) {
    static_assert(CQ_MOE_NOALLOC_MAX_BYTES == kMoeScratchBytes, "one scratch size");
    if (!moe_flags_ok(flags)) return CQ_ERR_INVALID_ARG;
    if (int rc = check_moe_gemm(wt, w_experts, n_experts, n, k, n_tokens, top_k, ldy)) return rc;
    if (n > (int64_t(1) << 24)) return CQ_ERR_SHAPE;
    if (static_cast<int64_t>(cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags)) >
        kMoeScratchBytes)
        return CQ_ERR_SCRATCH_LIMIT;
    if (n == 0 || n_tokens == 0) return CQ_OK;
    const bool combine = (flags & CQ_MOE_OUT_COMBINE) != 0;
    if (!xq || !expert_ids || !y || !status || (combine && !route_w)) return CQ_ERR_INVALID_ARG;
    if (!aligned(xq, 2) || !aligned(expert_ids, 4) || !aligned(y, 4) || !aligned(status, 4) ||
        (combine && !aligned(route_w, 4)))
        return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    uint8_t* ws = nullptr;
    if (int rc = moe_scratch_address(&ws)) return status_of(rc);
    return status_of(launch_moe_routed(wt, w_experts, n_experts, n, k, xq, flags, expert_ids,
                                       route_w, n_tokens, top_k, y, ldy, ws, status,
                                       reinterpret_cast<hipStream_t>(stream)));
}

int cq_swiglu_quantize_q8_0(const float* g, const float* u, int64_t rows, int64_t k,
                            float* h_opt, void* hq, cq_stream_t stream) {
    if (rows < 0 || k <= 0) return CQ_ERR_INVALID_ARG;
    if (k % 32 != 0 || k > CQ_MAX_K) return CQ_ERR_SHAPE;
    if (rows == 0) return CQ_OK;
    if (!g || !u || !hq) return CQ_ERR_INVALID_ARG;
    if (!aligned(g, 16) || !aligned(u, 16) || !aligned(h_opt, 16) || !aligned(hq, 2))
        return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_swiglu_quantize_q8_0(g, u, k, rows, k, h_opt, hq,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

int cq_moe_combine(const float* d, const float* route_w, int64_t n_tokens, int64_t top_k,
                   int64_t n, float* y, int64_t ldy, cq_stream_t stream) {
    if (n_tokens < 0 || top_k < 1 || n < 0 || ldy < n) return CQ_ERR_INVALID_ARG;
    if (n_tokens == 0 || n == 0) return CQ_OK;
    if (!d || !route_w || !y) return CQ_ERR_INVALID_ARG;
    if (!aligned(d, 4) || !aligned(route_w, 4) || !aligned(y, 4)) return CQ_ERR_ALIGNMENT;
    if (int rc = check_device()) return rc;
    return status_of(launch_moe_combine(d, route_w, n_tokens, top_k, n, y, ldy, nullptr, 0,
                                        reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
