"""Helpers shared by the GPU parity tests (device transfer, tolerance checks)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"

# Tolerance on float32 state (params, m, v, momentum) after N steps:
# |gpu - oracle| <= REL * |oracle| + ABS.
REL, ABS = 1e-5, 1e-7
U32 = 2.0 ** -24  # float32 unit roundoff


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_state_close(gpu: np.ndarray, ora: np.ndarray, what: str, rel=REL, abs_=ABS):
    g = np.asarray(gpu, np.float64).reshape(-1)
    o = np.asarray(ora, np.float64).reshape(-1)
    assert g.shape == o.shape, f"{what}: shape {g.shape} vs {o.shape}"
    err = np.abs(g - o)
    tol = rel * np.abs(o) + abs_
    bad = ~(err <= tol)
    if bad.any():
        i = int(np.argmax(np.where(bad, err / tol, 0)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside "
                             f"{rel:g}*|x|+{abs_:g}; worst at {i}: gpu {g[i]!r} oracle {o[i]!r}")


def assert_sums_close(gpu_vals, ora_vals, ids, keys, counts, grads):
    """Duplicate sums: the GPU sums in float32 in its own fixed order, the oracle
    in double; allow the recursive-summation bound gamma_{k-1} * sum|g| in float32
    plus the oracle's own final rounding."""
    gpu_vals = np.asarray(gpu_vals, np.float64)
    ora_vals = np.asarray(ora_vals, np.float64)
    width = grads.shape[1] if grads.ndim == 2 else 1
    g2 = grads.reshape(len(ids), width).astype(np.float64)
    order = np.argsort(ids, kind="stable")
    abs_sum = np.add.reduceat(np.abs(g2[order]), np.r_[0, np.cumsum(counts)[:-1]], axis=0) \
        if len(ids) else np.zeros((0, width))
    k = counts.astype(np.float64)[:, None]
    gamma = (k - 1) * U32 / (1 - k * U32)
    tol = gamma * abs_sum + (np.abs(ora_vals) + gamma * abs_sum) * U32 + 1e-30
    err = np.abs(gpu_vals.reshape(tol.shape) - ora_vals.reshape(tol.shape))
    bad = err > tol
    assert not bad.any(), f"{int(bad.sum())} duplicate sums outside the summation bound"
