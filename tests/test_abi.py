"""The C-ABI library on the CPU: it loads, exports every symbol include/cq.h
declares, reports block geometry, and rejects invalid arguments on the host
with the documented status before touching any device (no GPU needed)."""
import ctypes
import os
import re

import pytest

import quantized_gguf_block_amd as cq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cq.h")

OK, INVALID, UNSUPPORTED, SHAPE, ALIGN = 0, -1, -2, -3, -4
FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    """libcq through its binding, or (CQ_TEST_LIB set: the sanitized
    host-validation build) that library through ctypes with the binding's
    signatures."""
    path = os.environ.get("CQ_TEST_LIB")
    if not path:
        return cq.load()
    L = ctypes.CDLL(path)
    for name, (res, args) in cq.signatures().items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(cq.EXPORTS)


def test_version_and_status_strings(lib):
    assert lib.cq_abi_version() == 2
    for code, name in cq.STATUS.items():
        assert lib.cq_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.cq_status_string(12345)


def test_block_geometry(lib):
    assert [lib.cq_block_elems(t) for t in (2, 3, 8, 12, 13, 14)] == [32, 32, 32, 256, 256, 256]
    assert [lib.cq_block_bytes(t) for t in (2, 3, 8, 12, 13, 14)] == [18, 20, 34, 144, 176, 210]
    assert lib.cq_row_bytes(13, 4096) == 2816
    assert (lib.cq_block_elems(41), lib.cq_block_bytes(41), lib.cq_row_bytes(41, 5120)) == (128, 18, 720)
    assert (lib.cq_block_elems(42), lib.cq_block_bytes(42), lib.cq_row_bytes(42, 8192)) == (128, 34, 2176)
    assert lib.cq_row_bytes(42, 8160) == -1
    assert lib.cq_row_bytes(14, 4096) == 3360
    assert lib.cq_row_bytes(12, 4096) == 2304
    assert lib.cq_row_bytes(8, 4096) == 4352
    assert lib.cq_row_bytes(12, 4000) == -1
    assert lib.cq_block_bytes(7) == -1


P = ctypes.c_void_p


def test_quantize_validation(lib):
    f = lib.cq_quantize_q8_0
    assert f(P(FAKE), 64, 2, 48, P(FAKE), None) == SHAPE            # k % 32
    assert f(P(FAKE), 16, 2, 64, P(FAKE), None) == INVALID          # ldx < k
    assert f(None, 64, 2, 64, P(FAKE), None) == INVALID
    assert f(P(FAKE + 4), 64, 2, 64, P(FAKE), None) == ALIGN        # x not 16-aligned
    assert f(P(FAKE), 66, 2, 64, P(FAKE), None) == ALIGN            # ldx % 4
    assert f(P(FAKE), 64, 2, 64, P(FAKE + 1), None) == ALIGN
    assert f(None, 64, 0, 64, None, None) == OK                     # empty: no launch
    assert f(P(FAKE), 1 << 20, 1, 1 << 17, P(FAKE), None) == SHAPE  # k > CQ_MAX_K


def test_gemv_validation(lib):
    f = lib.cq_gemv
    assert f(7, P(FAKE), 8, 256, P(FAKE), 1, P(FAKE), 8, None) == UNSUPPORTED
    assert f(12, P(FAKE), 8, 288, P(FAKE), 1, P(FAKE), 8, None) == SHAPE   # Q4_K needs 256
    assert f(14, P(FAKE), 8, 288, P(FAKE), 1, P(FAKE), 8, None) == SHAPE   # Q6_K needs 256
    assert f(13, P(FAKE), 8, 288, P(FAKE), 1, P(FAKE), 8, None) == SHAPE   # Q5_K needs 256
    assert f(2, P(FAKE), 8, 48, P(FAKE), 1, P(FAKE), 8, None) == SHAPE
    assert f(2, P(FAKE), 8, 256, P(FAKE), 0, P(FAKE), 8, None) == INVALID  # batch 0
    assert f(2, P(FAKE), 8, 256, P(FAKE), 9, P(FAKE), 8, None) == INVALID  # batch 9
    assert f(2, P(FAKE), 8, 256, P(FAKE), 1, P(FAKE), 7, None) == INVALID  # ldy < n
    assert f(2, P(FAKE + 8), 8, 256, P(FAKE), 1, P(FAKE), 8, None) == ALIGN
    assert f(2, P(FAKE), 8, 256, P(FAKE + 1), 1, P(FAKE), 8, None) == ALIGN
    assert f(2, P(FAKE), 8, 256, P(FAKE), 1, P(FAKE + 2), 8, None) == ALIGN
    assert f(2, None, 8, 256, P(FAKE), 1, P(FAKE), 8, None) == INVALID
    assert f(2, None, 0, 256, None, 1, None, 0, None) == OK              # n == 0
    assert f(8, P(FAKE), -1, 256, P(FAKE), 1, P(FAKE), 8, None) == INVALID
    assert f(8, P(FAKE), 8, 32768 + 256, P(FAKE), 1, P(FAKE), 8, None) == SHAPE  # > CQ_GEMV_MAX_K


def test_gemv_swiglu_validation(lib):
    f = lib.cq_gemv_swiglu
    A = (P(FAKE), P(FAKE))
    assert f(7, *A, 8, 256, P(FAKE), 1, P(FAKE), 8, None) == UNSUPPORTED
    assert f(2, *A, 8, 20480, P(FAKE), 1, P(FAKE), 8, None) == SHAPE    # five waves per row
    assert f(2, *A, 8, 352, P(FAKE), 1, P(FAKE), 8, None) == SHAPE      # not 16-byte rows
    assert f(14, *A, 8, 1024, P(FAKE), 1, P(FAKE), 8, None) == SHAPE    # Q6_K needs k % 2048
    assert f(2, *A, 8, 256, P(FAKE), 0, P(FAKE), 8, None) == INVALID    # batch 0
    assert f(2, *A, 8, 256, P(FAKE), 1, P(FAKE), 7, None) == INVALID    # ldh < n
    assert f(2, P(FAKE), P(FAKE + 8), 8, 256, P(FAKE), 1, P(FAKE), 8, None) == ALIGN
    assert f(2, *A, 8, 256, P(FAKE + 2), 1, P(FAKE), 8, None) == ALIGN  # xq 16-aligned
    assert f(2, *A, 0, 256, None, 1, None, 0, None) == OK               # n == 0


def test_moe_gemv_validation(lib):
    f = lib.cq_moe_gemv
    A = (P(FAKE), 32, 64, 2048)
    S = P(FAKE + 64)   # status counter
    assert f(7, *A, P(FAKE), 0, P(FAKE), 1, 4, P(FAKE), 64, S, None) == UNSUPPORTED
    assert f(12, *A, P(FAKE), 2, P(FAKE), 1, 4, P(FAKE), 64, S, None) == INVALID   # x_per_pair
    assert f(12, *A, P(FAKE), 0, P(FAKE), 1, 40, P(FAKE), 64, S, None) == INVALID  # top_k > E
    assert f(12, P(FAKE), 32, 64, 8192, P(FAKE), 0, P(FAKE), 1, 4, P(FAKE), 64, S, None) == SHAPE
    assert f(12, *A, P(FAKE), 0, P(FAKE), 20000, 4, P(FAKE), 64, S, None) == SHAPE  # > 65535 pairs
    assert f(12, *A, P(FAKE + 2), 0, P(FAKE), 1, 4, P(FAKE), 64, S, None) == ALIGN  # xq
    assert f(12, *A, P(FAKE), 0, P(FAKE + 2), 1, 4, P(FAKE), 64, S, None) == ALIGN  # ids
    assert f(12, *A, P(FAKE), 0, P(FAKE), 1, 4, P(FAKE), 64, None, None) == INVALID  # no status
    assert f(12, *A, P(FAKE), 0, P(FAKE), 1, 4, P(FAKE), 64, P(FAKE + 2), None) == ALIGN
    assert f(12, *A, P(FAKE), 0, P(FAKE), 0, 4, P(FAKE), 64, S, None) == OK         # no tokens
    g = lib.cq_moe_gemv_swiglu
    assert g(12, P(FAKE), P(FAKE + 8), 32, 64, 2048, P(FAKE), P(FAKE), 1, 4, P(FAKE), 64,
             S, None) == ALIGN                                                      # w_up
    assert g(12, P(FAKE), P(FAKE), 32, 64, 2048, P(FAKE), P(FAKE), 1, 4, P(FAKE), 63,
             S, None) == INVALID                                                    # ldh < n
    assert g(12, P(FAKE), P(FAKE), 32, 64, 2048, P(FAKE), P(FAKE), 1, 4, P(FAKE), 64,
             None, None) == INVALID                                                 # no status


def test_argmax_and_router_validation(lib):
    assert lib.cq_argmax_workspace_bytes(4, 128256) == 4 * 32 * 8
    assert lib.cq_argmax_workspace_bytes(1, 4096) == 8
    assert lib.cq_argmax_workspace_bytes(1, 0) == 0
    f = lib.cq_argmax
    assert f(P(FAKE), 2, 0, 8, P(FAKE), P(FAKE), 64, None) == INVALID       # n == 0
    assert f(P(FAKE), 2, 8, 7, P(FAKE), P(FAKE), 64, None) == INVALID       # ldy < n
    assert f(P(FAKE), 70000, 8, 8, P(FAKE), P(FAKE), 1 << 20, None) == SHAPE
    assert f(P(FAKE + 2), 2, 8, 8, P(FAKE), P(FAKE), 64, None) == ALIGN
    assert f(P(FAKE), 2, 8, 8, P(FAKE), P(FAKE), 15, None) == -5            # workspace too small
    assert f(P(FAKE), 2, 8, 8, P(FAKE), P(FAKE + 4), 64, None) == -5        # workspace alignment
    assert f(None, 0, 8, 8, None, None, 0, None) == OK                      # no rows
    g = lib.cq_topk_softmax
    assert g(P(FAKE), 4, 32, 32, 0, P(FAKE), P(FAKE), None) == INVALID      # top_k 0
    assert g(P(FAKE), 4, 32, 32, 17, P(FAKE), P(FAKE), None) == INVALID     # top_k > 16
    assert g(P(FAKE), 4, 2000, 2000, 4, P(FAKE), P(FAKE), None) == INVALID  # > 1024 experts
    assert g(P(FAKE), 4, 32, 31, 4, P(FAKE), P(FAKE), None) == INVALID      # ld < E
    assert g(P(FAKE), 4, 32, 32, 4, P(FAKE + 1), P(FAKE), None) == ALIGN
    assert g(None, 0, 32, 32, 4, None, None, None) == OK


def test_gemm_validation(lib):
    f = lib.cq_gemm
    assert f(2, P(FAKE), 8, 32, P(FAKE), 4, P(FAKE), 8, None) == SHAPE     # k % 256
    assert f(2, P(FAKE), 8, 256, P(FAKE), -1, P(FAKE), 8, None) == INVALID
    assert f(2, P(FAKE), 8, 256, None, 0, None, 8, None) == OK             # m == 0
    assert f(5, P(FAKE), 8, 256, P(FAKE), 4, P(FAKE), 8, None) == UNSUPPORTED
    assert f(7, P(FAKE), 8, 256, P(FAKE), 4, P(FAKE), 8, None) == UNSUPPORTED
    assert f(41, P(FAKE), 8, 256, P(FAKE), 4, P(FAKE), 8, None) == UNSUPPORTED  # Q1_0: GEMV only
    assert f(42, P(FAKE), 8, 256, P(FAKE), 4, P(FAKE), 8, None) == UNSUPPORTED  # TQ2: GEMV only
    # Q6_K rows are read with 31-bit offsets: a matrix of 2 GiB or more is refused
    assert f(14, P(FAKE), 1 << 20, 2560, P(FAKE), 4, P(FAKE), 1 << 20, None) == SHAPE


def test_moe_validation(lib):
    g = lib.cq_moe_group
    S = P(FAKE + 64)
    assert g(P(FAKE), 4, 0, 32, P(FAKE), P(FAKE), S, None) == INVALID          # top_k 0
    assert g(P(FAKE), 4, 4, 2000, P(FAKE), P(FAKE), S, None) == INVALID        # > 1024 experts
    assert g(P(FAKE), 4, 8, 4, P(FAKE), P(FAKE), S, None) == INVALID           # top_k > E
    assert g(P(FAKE), 4, 4, 32, P(FAKE), P(FAKE), None, None) == INVALID       # no status
    assert g(P(FAKE + 2), 4, 4, 32, P(FAKE), P(FAKE), S, None) == ALIGN
    assert g(P(FAKE), 4, 4, 32, P(FAKE), P(FAKE), P(FAKE + 1), None) == ALIGN
    m = lib.cq_moe_gemm_grouped
    assert m(12, P(FAKE), 32, 64, 256, P(FAKE), 2, P(FAKE), P(FAKE), 4, 4, P(FAKE), 64,
             None) == INVALID                                                # x_per_pair
    assert m(12, P(FAKE), 32, 64, 288, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, P(FAKE), 64,
             None) == SHAPE
    assert m(12, P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 0, 4, P(FAKE), 64,
             None) == OK                                                     # no tokens
    assert m(7, P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, P(FAKE), 64,
             None) == UNSUPPORTED
    assert m(14, P(FAKE), 2, 1 << 20, 2560, P(FAKE), 0, P(FAKE), P(FAKE), 4, 2, P(FAKE),
             1 << 20, None) == SHAPE                                         # Q6_K expert >= 2 GiB
    m2 = lib.cq_moe_gemm_grouped2
    YA, YB = P(FAKE), P(FAKE + 4 * 64 * 15)      # 16 pair rows of ldy 64: YB = YA's last row
    assert m2(12, P(FAKE), P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, YA, YB, 64,
              None) == INVALID                                           # y_b starts in y_a's last row
    assert m2(12, P(FAKE), P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, YB, YA, 64,
              None) == INVALID                                           # (either order)
    assert m2(12, P(FAKE), None, 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, YA,
              P(FAKE + (1 << 20)), 64, None) == INVALID                    # no second matrix
    assert m2(12, P(FAKE), P(FAKE + 8), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, YA,
              P(FAKE + (1 << 20)), 64, None) == ALIGN                      # second matrix 8-aligned
    assert m2(12, P(FAKE), P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, YA, None,
              64, None) == INVALID                                       # no second output
    assert m2(12, P(FAKE), P(FAKE), 32, 64, 256, P(FAKE), 3, P(FAKE), P(FAKE), 4, 4, YA,
              P(FAKE + (1 << 20)), 64, None) == INVALID                    # x_per_pair
    assert m2(7, P(FAKE), P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 4, 4, YA,
              P(FAKE + (1 << 20)), 64, None) == UNSUPPORTED
    assert m2(12, P(FAKE), P(FAKE), 32, 64, 256, P(FAKE), 0, P(FAKE), P(FAKE), 0, 4, YA, YA, 64,
              None) == OK                                                # no tokens: nothing written
    s = lib.cq_swiglu_quantize_q8_0
    assert s(P(FAKE), P(FAKE), 2, 48, None, P(FAKE), None) == SHAPE
    assert s(P(FAKE), P(FAKE + 4), 2, 64, None, P(FAKE), None) == ALIGN
    assert s(P(FAKE), P(FAKE), 2, 64, P(FAKE + 8), P(FAKE), None) == ALIGN
    assert s(P(FAKE), P(FAKE), 2, 64, None, P(FAKE + 1), None) == ALIGN
    assert s(None, None, 0, 64, None, None, None) == OK
    c = lib.cq_moe_combine
    assert c(P(FAKE), P(FAKE), 4, 4, 64, P(FAKE), 32, None) == INVALID      # ldy < n
    assert c(P(FAKE), P(FAKE), 0, 4, 64, P(FAKE), 64, None) == OK


def test_moe_workspace_bytes(lib):
    """Status word, offsets, pair list and (combined output) the per-pair
    product rows, each part 256-byte aligned."""
    wb = lib.cq_moe_workspace_bytes
    assert wb(256, 4, 32, 2048, 0) == 256 + 256 + 4096
    assert wb(256, 4, 32, 2048, 1) == 256 + 256 + 4096
    assert wb(256, 4, 32, 2048, 2) == 256 + 256 + 4096 + 4 * 1024 * 2048
    assert wb(256, 4, 32, 2048, 3) == 256 + 256 + 4096 + 4 * 1024 * 2048
    assert wb(1, 1, 1024, 5, 2) == 256 + 4352 + 256 + 256
    assert wb(0, 4, 32, 2048, 0) == 256 + 256 + 256
    assert wb(256, 4, 32, 2048, 4) == 0                                     # unknown flag
    assert wb(256, 0, 32, 2048, 0) == 0
    assert wb(256, 40, 32, 2048, 0) == 0                                    # top_k > E
    assert wb(256, 4, 2000, 2048, 0) == 0


def test_moe_one_call_validation(lib):
    f = lib.cq_moe_gemm
    WS = 256 + 256 + 4096 + 4 * 1024 * 2048
    W = P(1 << 20)  # 256-byte aligned fake workspace

    def call(wt=12, n=2048, k=1536, flags=3, ids=P(FAKE), rw=P(FAKE), T=256, top_k=4, y=P(FAKE),
             ldy=2048, ws=W, wsb=WS, xq=P(FAKE)):
        return f(wt, P(FAKE), 32, n, k, xq, flags, ids, rw, T, top_k, y, ldy, ws, wsb, None)

    assert call(flags=4) == INVALID
    assert call(flags=-1) == INVALID
    assert call(wt=41) == UNSUPPORTED
    assert call(wt=42) == UNSUPPORTED
    assert call(wt=7) == UNSUPPORTED
    assert call(k=1000) == SHAPE
    assert call(top_k=40) == INVALID
    assert call(ldy=100) == INVALID
    assert call(rw=None) == INVALID                      # combine needs the route weights
    assert call(ids=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(wsb=WS - 1) == -5
    assert call(ws=P((1 << 20) + 16)) == -5              # 256-byte alignment
    assert call(ids=P(FAKE + 2)) == ALIGN
    assert call(rw=P(FAKE + 1)) == ALIGN
    assert call(T=0) == OK                               # no tokens: nothing launched
    assert call(n=0) == OK


def test_moe_noalloc_validation(lib):
    """The no-allocation routed projection refuses, before any launch, a call
    whose workspace would exceed its fixed scratch, and checks the rest as
    cq_moe_gemm does."""
    f = lib.cq_moe_gemm_noalloc
    S = P(FAKE + 64)

    def call(n=2048, T=256, top_k=4, flags=3, status=S, rw=P(FAKE), k=1536):
        return f(12, P(FAKE), 32, n, k, P(FAKE), flags, P(FAKE), rw, T, top_k, P(FAKE), n,
                 status, None)

    # 256 tokens x 4 pairs x 2048 combined outputs (8.4 MB) fit; 1024 tokens (33.6 MB) do not
    assert lib.cq_moe_workspace_bytes(1024, 4, 32, 2048, 3) > cq.MOE_NOALLOC_MAX_BYTES
    assert call(T=1024) == -8
    assert call(T=1024, flags=1) != -8          # per-pair output needs no product rows
    assert call(flags=8) == INVALID
    assert call(status=None) == INVALID
    assert call(status=P(FAKE + 2)) == ALIGN
    assert call(rw=None) == INVALID
    assert call(k=1000) == SHAPE
    assert call(T=0) == OK
    assert lib.cq_status_string(-8).decode().startswith("CQ_ERR_SCRATCH_LIMIT")
