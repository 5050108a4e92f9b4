"""Helpers for the GPU parity tests: device transfer and the tolerance check
|y - y_ref| <= 2e-5 * sum|w_hat * x_hat| against the fp64 oracle."""
import sys

import numpy as np

TOL = 2e-5


def note(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close_to_oracle(y, y_ref, s_ref, tol=TOL, what=""):
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    bound = tol * s_ref
    bad = err > bound
    # an output whose magnitude sum is exactly 0 must itself be exactly 0
    if bad.any():
        idx = np.argwhere(bad)[:5]
        ratio = float(np.max(err / np.maximum(s_ref, 1e-300)))
        raise AssertionError(f"{what}: {bad.sum()} outputs outside {tol}*S; max err/S = {ratio:.3e}; "
                             f"first {idx.tolist()}: y={y[tuple(idx[0])]!r} ref={y_ref[tuple(idx[0])]!r}")
    return float(np.max(err / np.maximum(s_ref, 1e-300))) if err.size else 0.0
