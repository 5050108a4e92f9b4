"""The no-allocation routed projection (cq_moe_gemm_noalloc) through the C
ABI: two calls in a row on the lfm2moe shape (256 tokens, then 40), each
bitwise equal to cq_moe_gemm on a caller workspace (the same kernels) and
within the oracle tolerance, with the status word stored by each call."""
import numpy as np
import pytest
import torch

import gguf_synth as gs
from gpu_common import assert_close_to_oracle, note, to_dev, to_host

pytestmark = pytest.mark.gpu

C = gs.CONFIGS["q4_k_moe_ffn"]
T, H, F, E, K = C["n_tokens"], C["hidden"], C["ffn"], C["n_experts"], C["top_k"]
FMT = C["fmt"]


@pytest.mark.parametrize("combine", [False, True])
def test_noalloc_matches_workspace_call(cq, orc, combine):
    cfg = C["cfg"]
    wd_h = gs.expert_weights(FMT, E, H, F, cfg, 2)
    wd = to_dev(wd_h)
    flags = cq.MOE_X_PER_PAIR | (cq.MOE_OUT_COMBINE if combine else cq.MOE_OUT_PER_PAIR)
    status = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    for tokens in (T, 40):                    # the second call is smaller
        ids_h, rw_h = gs.routing(tokens, E, K, cfg=900 + tokens)
        hq_h = orc.quantize_q8_0(gs.activations(tokens * K, F, cfg=901 + tokens))
        ids, rw, hq = to_dev(ids_h), to_dev(rw_h), to_dev(hq_h)
        note("moe noalloc", tokens, combine)
        y0, st0 = cq.cq_moe_gemm_noalloc(FMT, wd, E, H, F, hq, flags, ids, route_w=rw,
                                         status=status)
        y0 = to_host(y0)
        assert int(to_host(st0)[0]) == 0
        note("moe with workspace", tokens, combine)
        y1, st1 = cq.cq_moe_gemm(FMT, wd, E, H, F, hq, flags, ids, route_w=rw)
        y1 = to_host(y1)
        assert int(to_host(st1)[0]) == 0
        assert np.array_equal(y0, y1)
        d_ref, s_ref = orc.moe_matmul(FMT, wd_h, E, H, F, hq_h, True, ids_h)
        if combine:
            y_ref, sy = orc.moe_combine(d_ref, s_ref, rw_h)
            mag, _ = orc.moe_combine(np.abs(d_ref), None, np.abs(rw_h))
            assert np.all(np.abs(y0 - y_ref) <= 2e-5 * sy + 4 * 2.0 ** -24 * mag + 1e-30)
        else:
            assert_close_to_oracle(y0, d_ref, s_ref, what=f"noalloc {tokens}")
    # an out-of-range id is counted in the caller's status word
    ids_h[0, 0] = E
    y2, st2 = cq.cq_moe_gemm_noalloc(FMT, wd, E, H, F, hq, flags, to_dev(ids_h), route_w=rw,
                                     status=status)
    assert int(to_host(st2)[0]) == 1
