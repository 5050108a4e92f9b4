"""Python binding of libcq, the MI355X block-quantized GGUF matmul.

Thin ctypes marshalling over the C ABI declared in include/cq.h: each
function here has the name of the C entry point it calls, turns torch device
tensors into pointers and sizes, passes torch's current HIP stream, and
raises CQError on a non-zero status.  All computation happens in the HIP
kernels of libcq.so; there is no fallback path.  Output tensors that the
caller does not supply are allocated here with torch (the library itself
never allocates).
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcq.so")

Q4_0, Q4_1, Q8_0, Q4_K, Q5_K, Q6_K, Q1_0, TQ2 = 2, 3, 8, 12, 13, 14, 41, 42
BLOCK_ELEMS = {Q4_0: 32, Q4_1: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256, Q1_0: 128, TQ2: 128}
BLOCK_BYTES = {Q4_0: 18, Q4_1: 20, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210, Q1_0: 18, TQ2: 34}
GEMV_MAX_BATCH = 8

STATUS = {0: "CQ_OK", -1: "CQ_ERR_INVALID_ARG", -2: "CQ_ERR_UNSUPPORTED_TYPE",
          -3: "CQ_ERR_SHAPE", -4: "CQ_ERR_ALIGNMENT", -5: "CQ_ERR_WORKSPACE",
          -6: "CQ_ERR_HIP", -7: "CQ_ERR_NO_DEVICE", -8: "CQ_ERR_SCRATCH_LIMIT"}
MOE_NOALLOC_MAX_BYTES = 16 << 20

EXPORTS = [
    "cq_abi_version", "cq_status_string", "cq_block_elems", "cq_block_bytes", "cq_row_bytes",
    "cq_quantize_q8_0", "cq_gemv", "cq_gemv_swiglu", "cq_gemm", "cq_moe_workspace_bytes",
    "cq_moe_gemm", "cq_moe_gemm_noalloc", "cq_moe_group", "cq_moe_gemm_grouped",
    "cq_moe_gemm_grouped2", "cq_swiglu_quantize_q8_0",
    "cq_moe_combine", "cq_moe_gemv", "cq_moe_gemv_swiglu", "cq_argmax_workspace_bytes",
    "cq_argmax", "cq_topk_softmax",
]

# cq_moe_gemm flags
MOE_X_PER_TOKEN, MOE_X_PER_PAIR = 0, 1
MOE_OUT_PER_PAIR, MOE_OUT_COMBINE = 0, 2


class CQError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_lib = None


def load():
    """Load libcq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(or python -m quantized_gguf_block_amd.build)")
    # torch ships its own HIP runtime, linked under the unversioned name
    # libamdhip64.so.  Loading torch first makes libcq's libamdhip64.so.7
    # dependency bind to that same, already loaded runtime (by soname), so
    # pointers, streams and the current device are shared.  Loading libcq
    # first would put a second HIP runtime into the process.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in signatures().items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def signatures():
    """ctypes result and argument types of every exported function."""
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    return {
        "cq_abi_version": (I, []),
        "cq_status_string": (ctypes.c_char_p, [I]),
        "cq_block_elems": (I64, [I]),
        "cq_block_bytes": (I64, [I]),
        "cq_row_bytes": (I64, [I, I64]),
        "cq_quantize_q8_0": (I, [P, I64, I64, I64, P, P]),
        "cq_gemv": (I, [I, P, I64, I64, P, I64, P, I64, P]),
        "cq_gemv_swiglu": (I, [I, P, P, I64, I64, P, I64, P, I64, P]),
        "cq_gemm": (I, [I, P, I64, I64, P, I64, P, I64, P]),
        "cq_moe_group": (I, [P, I64, I64, I64, P, P, P, P]),
        "cq_moe_gemm_grouped": (I, [I, P, I64, I64, I64, P, I, P, P, I64, I64, P, I64, P]),
        "cq_moe_gemm_grouped2": (I, [I, P, P, I64, I64, I64, P, I, P, P, I64, I64, P, P, I64, P]),
        "cq_moe_workspace_bytes": (ctypes.c_size_t, [I64, I64, I64, I64, I]),
        "cq_moe_gemm": (I, [I, P, I64, I64, I64, P, I, P, P, I64, I64, P, I64, P,
                            ctypes.c_size_t, P]),
        "cq_moe_gemm_noalloc": (I, [I, P, I64, I64, I64, P, I, P, P, I64, I64, P, I64, P, P]),
        "cq_swiglu_quantize_q8_0": (I, [P, P, I64, I64, P, P, P]),
        "cq_moe_combine": (I, [P, P, I64, I64, I64, P, I64, P]),
        "cq_moe_gemv": (I, [I, P, I64, I64, I64, P, I, P, I64, I64, P, I64, P, P]),
        "cq_argmax_workspace_bytes": (ctypes.c_size_t, [I64, I64]),
        "cq_argmax": (I, [P, I64, I64, I64, P, P, ctypes.c_size_t, P]),
        "cq_topk_softmax": (I, [P, I64, I64, I64, I64, P, P, P]),
        "cq_moe_gemv_swiglu": (I, [I, P, P, I64, I64, I64, P, P, I64, I64, P, I64, P, P]),
    }


def _check(fn, rc):
    if rc != 0:
        msg = load().cq_status_string(rc).decode()
        raise CQError(fn, rc, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_tensor(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def row_bytes(wt, k):
    return k // BLOCK_ELEMS[wt] * BLOCK_BYTES[wt]


def cq_quantize_q8_0(x, xq=None, stream=None):
    """x: fp32 [rows][k] (rows may be strided, elements contiguous) ->
    uint8 [rows][k/32*34] Q8_0 blocks."""
    import torch
    _dev_tensor(x, "x", torch.float32)
    if x.dim() == 1:
        x = x.view(1, -1)
    rows, k = x.shape
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    if xq is None:
        xq = torch.empty((rows, k // 32 * 34), dtype=torch.uint8, device=x.device)
    _dev_tensor(xq, "xq", torch.uint8)
    _check("cq_quantize_q8_0", load().cq_quantize_q8_0(
        _ptr(x), x.stride(0) if rows > 1 else k, rows, k, _ptr(xq), _stream(stream)))
    return xq


def cq_gemv(wt, w, n, k, xq, batch, y=None, ldy=None, stream=None):
    """y[b][i] = sum_j w_hat[i][j] x_hat[b][j] for b < batch (1..8)."""
    import torch
    _dev_tensor(w, "w", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    if y is None:
        y = torch.empty((batch, n), dtype=torch.float32, device=w.device)
    _dev_tensor(y, "y", torch.float32)
    ldy = ldy if ldy is not None else (y.stride(0) if y.dim() == 2 else n)
    _check("cq_gemv", load().cq_gemv(wt, _ptr(w), n, k, _ptr(xq), batch, _ptr(y), ldy,
                                      _stream(stream)))
    return y


def cq_gemv_swiglu(wt, w_gate, w_up, n, k, xq, batch, h=None, ldh=None, stream=None):
    """h[b][i] = silu(g) * u with g, u the gate and up GEMVs of row b (fused)."""
    import torch
    _dev_tensor(w_gate, "w_gate", torch.uint8)
    _dev_tensor(w_up, "w_up", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    if h is None:
        h = torch.empty((batch, n), dtype=torch.float32, device=w_gate.device)
    _dev_tensor(h, "h", torch.float32)
    ldh = ldh if ldh is not None else (h.stride(0) if h.dim() == 2 else n)
    _check("cq_gemv_swiglu", load().cq_gemv_swiglu(wt, _ptr(w_gate), _ptr(w_up), n, k, _ptr(xq),
                                                    batch, _ptr(h), ldh, _stream(stream)))
    return h


def cq_gemm(wt, w, n, k, xq, m, y=None, ldy=None, stream=None):
    """y[r][i] = sum_j w_hat[i][j] x_hat[r][j] for r < m (int8 MFMA)."""
    import torch
    _dev_tensor(w, "w", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _dev_tensor(y, "y", torch.float32)
    ldy = ldy if ldy is not None else (y.stride(0) if y.dim() == 2 else n)
    _check("cq_gemm", load().cq_gemm(wt, _ptr(w), n, k, _ptr(xq), m, _ptr(y), ldy,
                                      _stream(stream)))
    return y


def cq_moe_group(expert_ids, n_experts, offsets=None, pairs=None, status=None, stream=None):
    """expert_ids: int32 [n_tokens][top_k] -> (offsets int32 [E+1], pairs int32 [T*k],
    status int32 [1]: the number of ids outside [0, E) once the stream has run)."""
    import torch
    _dev_tensor(expert_ids, "expert_ids", torch.int32)
    n_tokens, top_k = expert_ids.shape
    dev = expert_ids.device
    if offsets is None:
        offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    if pairs is None:
        pairs = torch.empty(max(n_tokens * top_k, 1), dtype=torch.int32, device=dev)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=dev)
    _check("cq_moe_group", load().cq_moe_group(_ptr(expert_ids), n_tokens, top_k, n_experts,
                                                _ptr(offsets), _ptr(pairs), _ptr(status),
                                                _stream(stream)))
    return offsets, pairs, status


def cq_moe_gemm_grouped(wt, w_experts, n_experts, n, k, xq, x_per_pair, offsets, pairs,
                        n_tokens, top_k, y=None, ldy=None, stream=None):
    """Grouped expert projection on a cq_moe_group grouping -> y fp32
    [n_tokens*top_k][n], row = pair id."""
    import torch
    _dev_tensor(w_experts, "w_experts", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    if y is None:
        y = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=w_experts.device)
    ldy = ldy if ldy is not None else (y.stride(0) if y.dim() == 2 else n)
    _check("cq_moe_gemm_grouped", load().cq_moe_gemm_grouped(
        wt, _ptr(w_experts), n_experts, n, k, _ptr(xq), int(bool(x_per_pair)), _ptr(offsets),
        _ptr(pairs), n_tokens, top_k, _ptr(y), ldy, _stream(stream)))
    return y


def cq_moe_gemm_grouped2(wt, w_a_experts, w_b_experts, n_experts, n, k, xq, x_per_pair, offsets,
                         pairs, n_tokens, top_k, y_a=None, y_b=None, ldy=None, stream=None):
    """Two grouped expert projections of the same activation rows (gate and
    up) -> (y_a, y_b), each fp32 [n_tokens*top_k][n], row = pair id."""
    import torch
    _dev_tensor(w_a_experts, "w_a_experts", torch.uint8)
    _dev_tensor(w_b_experts, "w_b_experts", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    dev = w_a_experts.device
    if y_a is None:
        y_a = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=dev)
    if y_b is None:
        y_b = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=dev)
    ldy = ldy if ldy is not None else (y_a.stride(0) if y_a.dim() == 2 else n)
    _check("cq_moe_gemm_grouped2", load().cq_moe_gemm_grouped2(
        wt, _ptr(w_a_experts), _ptr(w_b_experts), n_experts, n, k, _ptr(xq), int(bool(x_per_pair)),
        _ptr(offsets), _ptr(pairs), n_tokens, top_k, _ptr(y_a), _ptr(y_b), ldy, _stream(stream)))
    return y_a, y_b


def cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags):
    return load().cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags)


def cq_moe_gemm(wt, w_experts, n_experts, n, k, xq, flags, expert_ids, route_w=None, y=None,
                ldy=None, workspace=None, stream=None):
    """One routed-expert projection (grouping, grouped product and, with
    MOE_OUT_COMBINE, the slot-order combine) -> (y, status): y fp32
    [n_tokens*top_k][n] per pair or [n_tokens][n] combined; status the int32
    workspace word that counts out-of-range expert ids."""
    import torch
    _dev_tensor(w_experts, "w_experts", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(expert_ids, "expert_ids", torch.int32)
    n_tokens, top_k = expert_ids.shape
    rows = n_tokens if flags & MOE_OUT_COMBINE else n_tokens * top_k
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=w_experts.device)
    _dev_tensor(y, "y", torch.float32)
    if route_w is not None:
        _dev_tensor(route_w, "route_w", torch.float32)
    ldy = ldy if ldy is not None else (y.stride(0) if y.dim() == 2 else n)
    need = load().cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=w_experts.device)
    _dev_tensor(workspace, "workspace", torch.uint8)
    _check("cq_moe_gemm", load().cq_moe_gemm(
        wt, _ptr(w_experts), n_experts, n, k, _ptr(xq), flags, _ptr(expert_ids), _ptr(route_w),
        n_tokens, top_k, _ptr(y), ldy, _ptr(workspace), workspace.numel(), _stream(stream)))
    return y, workspace[:4].view(torch.int32)


def cq_moe_gemm_noalloc(wt, w_experts, n_experts, n, k, xq, flags, expert_ids, route_w=None,
                        y=None, ldy=None, status=None, stream=None):
    """cq_moe_gemm without a workspace: the library's fixed device scratch
    serves instead (at most MOE_NOALLOC_MAX_BYTES) -> (y, status)."""
    import torch
    _dev_tensor(w_experts, "w_experts", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(expert_ids, "expert_ids", torch.int32)
    n_tokens, top_k = expert_ids.shape
    rows = n_tokens if flags & MOE_OUT_COMBINE else n_tokens * top_k
    if y is None:
        y = torch.empty((rows, n), dtype=torch.float32, device=w_experts.device)
    _dev_tensor(y, "y", torch.float32)
    if route_w is not None:
        _dev_tensor(route_w, "route_w", torch.float32)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=w_experts.device)
    _dev_tensor(status, "status", torch.int32)
    ldy = ldy if ldy is not None else (y.stride(0) if y.dim() == 2 else n)
    _check("cq_moe_gemm_noalloc", load().cq_moe_gemm_noalloc(
        wt, _ptr(w_experts), n_experts, n, k, _ptr(xq), flags, _ptr(expert_ids), _ptr(route_w),
        n_tokens, top_k, _ptr(y), ldy, _ptr(status), _stream(stream)))
    return y, status


def cq_swiglu_quantize_q8_0(g, u, h=None, want_h=False, hq=None, stream=None):
    """h = silu(g)*u (fp64 inside, fp32 out), quantized to Q8_0 -> (h or None, hq).
    g, u: contiguous fp32 [rows][k]."""
    import torch
    _dev_tensor(g, "g", torch.float32)
    _dev_tensor(u, "u", torch.float32)
    rows, k = g.shape
    if u.shape != g.shape or not g.is_contiguous() or not u.is_contiguous():
        raise ValueError("g and u must be contiguous and of the same shape")
    if h is None and want_h:
        h = torch.empty((rows, k), dtype=torch.float32, device=g.device)
    if hq is None:
        hq = torch.empty((rows, k // 32 * 34), dtype=torch.uint8, device=g.device)
    _check("cq_swiglu_quantize_q8_0", load().cq_swiglu_quantize_q8_0(
        _ptr(g), _ptr(u), rows, k, _ptr(h), _ptr(hq), _stream(stream)))
    return h, hq


def _status_counter(status, dev):
    import torch
    if status is None:
        return torch.zeros(1, dtype=torch.int32, device=dev)
    _dev_tensor(status, "status", torch.int32)
    return status


def cq_moe_gemv(wt, w_experts, n_experts, n, k, xq, x_per_pair, expert_ids, y=None, ldy=None,
                status=None, stream=None):
    """Decode routed experts: y[t*top_k+s] = W[ids[t][s]] x_hat[t or t*top_k+s]
    (one GEMV per pair) -> (y, status): status is the int32 error counter (a
    fresh zeroed one unless given) to which every out-of-range id adds 1."""
    import torch
    _dev_tensor(w_experts, "w_experts", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(expert_ids, "expert_ids", torch.int32)
    n_tokens, top_k = expert_ids.shape
    if y is None:
        y = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=w_experts.device)
    _dev_tensor(y, "y", torch.float32)
    status = _status_counter(status, w_experts.device)
    ldy = ldy if ldy is not None else (y.stride(0) if y.dim() == 2 else n)
    _check("cq_moe_gemv", load().cq_moe_gemv(wt, _ptr(w_experts), n_experts, n, k, _ptr(xq),
                                              int(bool(x_per_pair)), _ptr(expert_ids), n_tokens,
                                              top_k, _ptr(y), ldy, _ptr(status), _stream(stream)))
    return y, status


def cq_moe_gemv_swiglu(wt, w_gate_experts, w_up_experts, n_experts, n, k, xq, expert_ids,
                       h=None, ldh=None, status=None, stream=None):
    """Decode routed gate/up + SwiGLU: h[t*top_k+s] = silu(Wg_e x_t) * (Wu_e x_t),
    e = ids[t][s] -> (h, status) as cq_moe_gemv."""
    import torch
    _dev_tensor(w_gate_experts, "w_gate_experts", torch.uint8)
    _dev_tensor(w_up_experts, "w_up_experts", torch.uint8)
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(expert_ids, "expert_ids", torch.int32)
    n_tokens, top_k = expert_ids.shape
    if h is None:
        h = torch.empty((n_tokens * top_k, n), dtype=torch.float32, device=w_gate_experts.device)
    _dev_tensor(h, "h", torch.float32)
    status = _status_counter(status, w_gate_experts.device)
    ldh = ldh if ldh is not None else (h.stride(0) if h.dim() == 2 else n)
    _check("cq_moe_gemv_swiglu", load().cq_moe_gemv_swiglu(
        wt, _ptr(w_gate_experts), _ptr(w_up_experts), n_experts, n, k, _ptr(xq), _ptr(expert_ids),
        n_tokens, top_k, _ptr(h), ldh, _ptr(status), _stream(stream)))
    return h, status


def cq_argmax(y, idx=None, workspace=None, stream=None):
    """idx[r] = first index of the largest value of row r of fp32 y [rows][n]."""
    import torch
    _dev_tensor(y, "y", torch.float32)
    rows, n = y.shape
    if idx is None:
        idx = torch.empty(rows, dtype=torch.int32, device=y.device)
    _dev_tensor(idx, "idx", torch.int32)
    need = load().cq_argmax_workspace_bytes(rows, n)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=y.device)
    _dev_tensor(workspace, "workspace", torch.uint8)
    ldy = y.stride(0) if rows > 1 else n
    _check("cq_argmax", load().cq_argmax(_ptr(y), rows, n, ldy, _ptr(idx), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return idx


def cq_topk_softmax(logits, top_k, ids=None, w=None, stream=None):
    """Router: (ids int32 [rows][top_k], w fp32 [rows][top_k]) from fp32 logits [rows][E]."""
    import torch
    _dev_tensor(logits, "logits", torch.float32)
    rows, n_experts = logits.shape
    if ids is None:
        ids = torch.empty((rows, top_k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((rows, top_k), dtype=torch.float32, device=logits.device)
    _dev_tensor(ids, "ids", torch.int32)
    _dev_tensor(w, "w", torch.float32)
    ld = logits.stride(0) if rows > 1 else n_experts
    _check("cq_topk_softmax", load().cq_topk_softmax(_ptr(logits), rows, n_experts, ld, top_k,
                                                      _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def cq_moe_combine(d, route_w, y=None, stream=None):
    """y[t] = sum_s route_w[t][s] * d[t*top_k + s] (slot order, fp32)."""
    import torch
    _dev_tensor(d, "d", torch.float32)
    _dev_tensor(route_w, "route_w", torch.float32)
    n_tokens, top_k = route_w.shape
    n = d.shape[1]
    if y is None:
        y = torch.empty((n_tokens, n), dtype=torch.float32, device=d.device)
    _check("cq_moe_combine", load().cq_moe_combine(_ptr(d), _ptr(route_w), n_tokens, top_k, n,
                                                    _ptr(y), y.stride(0), _stream(stream)))
    return y
