"""ctypes shim over liboracle.so, the plain CPU reference.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and bench.py's
CPU-baseline leg may import this package; the product package never does.
This module only marshals numpy arrays to and from the C functions declared
in oracle.h; all arithmetic is in oracle.cpp.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0, Q4_1, Q8_0, Q4_K, Q5_K, Q6_K, Q1_0, TQ2 = 2, 3, 8, 12, 13, 14, 41, 42
TYPES = {"q4_0": Q4_0, "q4_1": Q4_1, "q8_0": Q8_0, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K,
         "q1_0": Q1_0, "tq2": TQ2}

_lib = None


def lib():
    """The oracle library (ORACLE_LIB names another build of it, such as the
    sanitized one the test suite makes)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = ctypes.CDLL(path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "oracle_abi_version": (I, []),
            "oracle_block_elems": (I64, [I]),
            "oracle_block_bytes": (I64, [I]),
            "oracle_half_to_double": (ctypes.c_double, [ctypes.c_uint16]),
            "oracle_float_to_half": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_half_to_double_n": (None, [P, I64, P]),
            "oracle_float_to_half_n": (None, [P, I64, P]),
            "oracle_q4k_scale_min": (None, [P, I, P, P]),
            "oracle_dequantize": (I, [I, P, I64, P]),
            "oracle_quantize_q8_0": (I, [P, I64, I64, I64, P]),
            "oracle_matmul": (I, [I, P, I64, I64, P, I64, P, P, I]),
            "oracle_matmul_sampled": (I, [I, P, I64, I64, P, I64, P, P, I64, P, P, I]),
            "oracle_matmul_factored": (I, [I, P, I64, I64, P, I64, P, I]),
            "oracle_swiglu": (None, [P, P, I64, P]),
            "oracle_moe_group": (I, [P, I64, I64, I64, P, P]),
            "oracle_moe_matmul": (I, [I, P, I64, I64, I64, P, I, P, I64, I64, P, P, I]),
            "oracle_moe_combine": (I, [P, P, P, I64, I64, I64, P, P]),
            "oracle_argmax_rows": (None, [P, I64, I64, I64, P]),
            "oracle_topk_softmax": (I, [P, I64, I64, I64, I64, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with status {rc}")


def _u8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8
    return a


def default_threads():
    return max(1, min(os.cpu_count() or 1, 16))


def block_elems(t):
    return lib().oracle_block_elems(t)


def block_bytes(t):
    return lib().oracle_block_bytes(t)


def half_to_double(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_half_to_double_n(_p(h), h.size, _p(out))
    return out


def float_to_half(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().oracle_float_to_half_n(_p(f), f.size, _p(out))
    return out


def q4k_scale_min(scales12, j):
    s = _u8(np.asarray(scales12, dtype=np.uint8))
    sc, mn = ctypes.c_int(), ctypes.c_int()
    lib().oracle_q4k_scale_min(_p(s), j, ctypes.byref(sc), ctypes.byref(mn))
    return sc.value, mn.value


def dequantize(t, blocks, n_elems):
    blocks = _u8(blocks)
    out = np.empty(n_elems, np.float64)
    _check(lib().oracle_dequantize(t, _p(blocks), n_elems, _p(out)), "dequantize")
    return out


def quantize_q8_0(x):
    """x: fp32 [rows][k] -> uint8 [rows][k/32*34]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    rows, k = x.shape
    out = np.empty((rows, k // 32 * 34), np.uint8)
    _check(lib().oracle_quantize_q8_0(_p(x), rows, k, k, _p(out)), "quantize_q8_0")
    return out


def matmul(t, w, n, k, xq, m, n_threads=None, want_s=True):
    """Returns (y, s): fp64 [m][n]."""
    w, xq = _u8(w), _u8(xq)
    y = np.empty((m, n), np.float64)
    s = np.empty((m, n), np.float64) if want_s else None
    _check(lib().oracle_matmul(t, _p(w), n, k, _p(xq), m, _p(y), _p(s),
                               n_threads or default_threads()), "matmul")
    return y, s


def matmul_sampled(t, w, n, k, xq, m, act_rows, w_rows, n_threads=None):
    w, xq = _u8(w), _u8(xq)
    a = np.ascontiguousarray(act_rows, dtype=np.int64)
    r = np.ascontiguousarray(w_rows, dtype=np.int64)
    y = np.empty(a.size, np.float64)
    s = np.empty(a.size, np.float64)
    _check(lib().oracle_matmul_sampled(t, _p(w), n, k, _p(xq), m, _p(a), _p(r), a.size,
                                       _p(y), _p(s), n_threads or default_threads()),
           "matmul_sampled")
    return y, s


def matmul_factored(t, w, n, k, xq, m, n_threads=None):
    w, xq = _u8(w), _u8(xq)
    y = np.empty((m, n), np.float64)
    _check(lib().oracle_matmul_factored(t, _p(w), n, k, _p(xq), m, _p(y),
                                        n_threads or default_threads()), "matmul_factored")
    return y


def swiglu(g, u):
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.float32)
    lib().oracle_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def moe_group(ids, n_experts):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n_tokens, top_k = ids.shape
    offsets = np.empty(n_experts + 1, np.int32)
    pairs = np.empty(n_tokens * top_k, np.int32)
    _check(lib().oracle_moe_group(_p(ids), n_tokens, top_k, n_experts, _p(offsets), _p(pairs)),
           "moe_group")
    return offsets, pairs


def moe_matmul(t, w, n_experts, n, k, xq, x_per_pair, ids, n_threads=None):
    """Returns (y, s) fp64 [n_tokens*top_k][n]."""
    w, xq = _u8(w), _u8(xq)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n_tokens, top_k = ids.shape
    y = np.empty((n_tokens * top_k, n), np.float64)
    s = np.empty((n_tokens * top_k, n), np.float64)
    _check(lib().oracle_moe_matmul(t, _p(w), n_experts, n, k, _p(xq), int(bool(x_per_pair)),
                                   _p(ids), n_tokens, top_k, _p(y), _p(s),
                                   n_threads or default_threads()), "moe_matmul")
    return y, s


def moe_combine(d, s_in, route_w):
    d = np.ascontiguousarray(d, dtype=np.float64)
    s_in = None if s_in is None else np.ascontiguousarray(s_in, dtype=np.float64)
    route_w = np.ascontiguousarray(route_w, dtype=np.float32)
    n_tokens, top_k = route_w.shape
    n = d.shape[1]
    y = np.empty((n_tokens, n), np.float64)
    s = np.empty((n_tokens, n), np.float64)
    _check(lib().oracle_moe_combine(_p(d), _p(s_in), _p(route_w), n_tokens, top_k, n,
                                    _p(y), _p(s)), "moe_combine")
    return y, (s if s_in is not None else None)


def argmax_rows(y):
    """First index of the largest value of each row of fp32 y [rows][n]."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    rows, n = y.shape
    idx = np.empty(rows, np.int32)
    lib().oracle_argmax_rows(_p(y), rows, n, n, _p(idx))
    return idx


def topk_softmax(logits, top_k):
    """Router: (ids int32 [rows][top_k], w fp32 [rows][top_k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    rows, n_experts = logits.shape
    ids = np.empty((rows, top_k), np.int32)
    w = np.empty((rows, top_k), np.float32)
    _check(lib().oracle_topk_softmax(_p(logits), rows, n_experts, n_experts, top_k, _p(ids), _p(w)),
           "topk_softmax")
    return ids, w

