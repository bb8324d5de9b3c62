"""GPU parity of DormancyDecay across long dormant gaps.

Page: docs.rs optirs_gpu sparse_optimizer, section LazyAdamMode::DormancyDecay:
a coordinate touched at t after last touched at s is decayed by beta^(t - s),
whatever the gap.  The kernels take beta^gap for gaps below 1024 from a table
of the host's pow() values and compute exp2(gap * log2 beta) in double beyond
it (skipped when m = v = 0, a coordinate never touched).  Here coordinates
with nonzero moments sit dormant for 1023, 1024, 1025, 1500, about 70,000 and
about 2^31 steps (set_step on the handle, the same t on the oracle), and are
then touched again, in every update form: the step from raw lookups in one
call, csr_from_lookups + the step, last_step per coordinate and per row, a
width that takes the one-coordinate-at-a-time path, and partial CSR rows.
State within 1e-5 relative + 1e-7 absolute of the oracle, last_step bit-exact.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu

ROWS = 1500
T_MAX = 2 ** 31 - 2  # the last step a handle can take (last_step is int32)


def _schedule(rng):
    """(t to set before the step or None, rows touched at the step) per step.
    Rows 0, 1, 2 are touched at steps 1, 2, 3 only and again at 1026, so their
    gaps are 1025, 1024 and 1023 around the table's edge."""
    common = np.arange(10, 400)
    part = np.arange(10, 200)
    later = np.arange(600, 700)
    return [
        (None, np.r_[0, common]),
        (None, np.r_[1, common]),
        (None, np.r_[2, common]),
        (1025, np.r_[0, 1, 2, part, later]),                       # gaps 1025, 1024, 1023
        (None, np.r_[common]),                                     # gaps 1 and 1024
        (2500, np.r_[3, 0, 1, 2, rng.choice(np.arange(200, 400), 50, replace=False)]),  # 1474
        (None, np.r_[4, rng.choice(np.arange(10, 700), 300, replace=False)]),
        (70_000, np.r_[np.arange(0, 700, 3), 900]),                # about 67,000
        (T_MAX - 1, np.r_[np.arange(0, 700, 7), 901]),             # about 2^31
    ]


def _lookups(rng, rows, cols):
    """Each touched row looked up 1-3 times, in random order; N(0, 0.01) rows."""
    ids = np.repeat(rows.astype(np.int64), rng.integers(1, 4, size=rows.size))
    ids = ids[rng.permutation(ids.size)]
    return ids, (rng.standard_normal((ids.size, cols)) * 0.01).astype(np.float32)


def _check(ora, gpu, what):
    torch.cuda.synchronize()
    assert gpu.t == ora.t, what
    assert np.array_equal(host(gpu.last_step), ora.ls), f"{what}: last_step"
    assert_state_close(host(gpu.params), ora.p, f"{what}: params")
    assert_state_close(host(gpu.m), ora.m, f"{what}: m")
    assert_state_close(host(gpu.v), ora.v, f"{what}: v")


@pytest.mark.parametrize("cols", [128, 6])
@pytest.mark.parametrize("per_row", [False, True])
@pytest.mark.parametrize("calls", ["one_call", "two_calls"])
def test_long_gaps_full_rows(calls, per_row, cols):
    rng = np.random.default_rng(1024 + cols + 2 * per_row)
    p0 = (rng.standard_normal((ROWS, cols)) * 0.01).astype(np.float32)
    cls = oracle.AdamRows if per_row else oracle.Adam
    ora = cls(p0.copy(), mode="dormancy")
    gpu = L.SparseAdam(dev(p0), mode="dormancy", last_step_per_row=per_row)
    for k, (t_set, rows) in enumerate(_schedule(rng)):
        if t_set is not None:
            gpu.handle.set_step(t_set)
            ora.t = t_set
        ids, grads = _lookups(rng, np.unique(rows), cols)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, ROWS)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, ROWS, cols, ROWS, cols)
        ora.step_csr(ro, ci, cv)
        if calls == "one_call":
            gpu.step_lookups(dev(ids), dev(grads))
        else:
            csr, _, _ = L.csr_from_lookups(dev(ids), dev(grads), ROWS)
            gpu.step(csr)
        _check(ora, gpu, f"{calls} per_row={per_row} cols={cols} step {k} (t={ora.t})")
    assert ora.t == T_MAX


def test_long_gaps_partial_rows():
    """Partial CSR rows (a random subset of each touched row's columns), last_step
    per coordinate: the one-lane-per-entry kernel on the same schedule."""
    rng = np.random.default_rng(77)
    cols = 64
    p0 = (rng.standard_normal((ROWS, cols)) * 0.01).astype(np.float32)
    ora = oracle.Adam(p0.copy(), mode="dormancy")
    gpu = L.SparseAdam(dev(p0), mode="dormancy")
    for k, (t_set, rows) in enumerate(_schedule(rng)):
        if t_set is not None:
            gpu.handle.set_step(t_set)
            ora.t = t_set
        rows = np.unique(rows)
        # columns 0..3 of every touched row always, then a random half of the rest
        mask = np.zeros((rows.size, cols), bool)
        mask[:, :4] = True
        mask[:, 4:] = rng.random((rows.size, cols - 4)) < 0.5
        r_i, c_i = np.nonzero(mask)
        lin = (rows[r_i] * cols + c_i).astype(np.int64)
        vals = rng.standard_normal(lin.size).astype(np.float32)
        ro, ci, cv = oracle.csr_from_coo(lin, vals, ROWS * cols, 1, ROWS, cols)
        ora.step_csr(ro, ci, cv)
        csr = L.csr_from_coo(L.CooGradient(dev(lin), dev(vals), dim=ROWS * cols), ROWS, cols)
        gpu.step(csr)
        _check(ora, gpu, f"partial rows step {k} (t={ora.t})")
