"""GPU parity of the routed-FFN helper steps: expert grouping (bit-exact
offsets and pair lists) and the slot-order combine."""
import numpy as np
import pytest

import gguf_synth as gs
from gpu_common import note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_tokens,n_experts,top_k", [(256, 32, 4), (1, 32, 4), (2000, 32, 4),
                                                      (300, 1, 1), (700, 1024, 8), (0, 32, 4),
                                                      (4096, 64, 2)])
def test_moe_group_bit_exact(cq, orc, n_tokens, n_experts, top_k):
    note("moe group", n_tokens, n_experts, top_k)
    if n_tokens:
        ids, _ = gs.routing(n_tokens, n_experts, top_k, cfg=500 + n_experts)
    else:
        ids = np.zeros((0, top_k), np.int32)
    off, pairs, st = cq.cq_moe_group(to_dev(ids), n_experts)
    off, pairs = to_host(off), to_host(pairs)
    assert to_host(st)[0] == 0
    off_ref, pairs_ref = orc.moe_group(ids, n_experts) if n_tokens else (
        np.zeros(n_experts + 1, np.int32), np.zeros(0, np.int32))
    assert np.array_equal(off, off_ref)
    assert np.array_equal(pairs[:n_tokens * top_k], pairs_ref)


def test_moe_group_skewed(cq, orc):
    note("moe group skewed")
    ids = np.zeros((1500, 4), np.int32)
    ids[:, 1] = 7
    ids[::3, 2] = 31
    ids[:, 3] = np.arange(1500) % 32
    off, pairs, st = cq.cq_moe_group(to_dev(ids), 32)
    off_ref, pairs_ref = orc.moe_group(ids, 32)
    assert np.array_equal(to_host(off), off_ref)
    assert np.array_equal(to_host(pairs), pairs_ref)
    assert to_host(st)[0] == 0


def test_moe_group_invalid_ids(cq, orc):
    """Ids outside [0, n_experts) are counted in the status word and placed in
    no group; the valid pairs are grouped exactly as the oracle groups them
    once the invalid pairs are removed."""
    note("moe group invalid ids")
    ids, _ = gs.routing(300, 32, 4, cfg=502)
    ids[5, 2] = -7
    ids[100, 0] = 32
    ids[299, 3] = 2 ** 31 - 1
    off, pairs, st = cq.cq_moe_group(to_dev(ids), 32)
    assert to_host(st)[0] == 3
    valid = (ids >= 0) & (ids < 32)
    flat = ids.reshape(-1)
    ok = np.flatnonzero(valid.reshape(-1))
    order = ok[np.argsort(flat[ok], kind="stable")]
    counts = np.bincount(flat[ok], minlength=32)
    assert np.array_equal(to_host(off), np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    assert np.array_equal(to_host(pairs)[:ok.size], order.astype(np.int32))


def test_moe_combine(cq, orc):
    note("moe combine")
    T, K, n = 256, 4, 2048
    rng = np.random.default_rng(9)
    d = rng.standard_normal((T * K, n)).astype(np.float32)
    _, rw = gs.routing(T, 32, K, cfg=501)
    y = to_host(cq.cq_moe_combine(to_dev(d), to_dev(rw)))
    y_ref, s_ref = orc.moe_combine(d.astype(np.float64), np.abs(d).astype(np.float64), rw)
    # four fp32 products summed in slot order: within 4 ulp-ish of the sum of |terms|
    assert np.all(np.abs(y - y_ref) <= 4 * 2.0 ** -24 * s_ref + 1e-30)


@pytest.mark.parametrize("T,K,n", [(5000, 2, 36), (7, 4, 1001), (3, 8, 4096)])
def test_moe_combine_shapes(cq, orc, T, K, n):
    """Token counts past one grid row of workgroups, column counts that are
    not a multiple of four (scalar path) and a strided output."""
    import torch
    note("moe combine shapes", T, K, n)
    rng = np.random.default_rng(10 + n)
    d = rng.standard_normal((T * K, n)).astype(np.float32)
    rw = rng.random((T, K)).astype(np.float32)
    ldy = n + 5
    y = torch.full((T, ldy), -3.0, device="cuda")
    cq.cq_moe_combine(to_dev(d), to_dev(rw), y=y[:, :n])
    yh = to_host(y)
    y_ref, s_ref = orc.moe_combine(d.astype(np.float64), np.abs(d).astype(np.float64), rw)
    assert np.all(np.abs(yh[:, :n] - y_ref) <= 4 * 2.0 ** -24 * s_ref + 1e-30)
    assert np.all(yh[:, n:] == -3.0)
