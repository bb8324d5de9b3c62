"""Pins of the oracle's row-granular last_step (one int32 per row).

Page: docs.rs optirs_gpu sparse_optimizer, "Lazy Adam" (SparseAdam keeps
last_step per coordinate) and "LazyAdamMode::DormancyDecay" (gap = t -
last_step).  For tables whose gradients always cover whole rows every
coordinate of a row holds the same last_step, so one value per row is the same
state: the row-granular step must equal the per-coordinate step bit for bit,
and a partial row is refused rather than silently breaking that equality.
"""
import numpy as np
import pytest

import oracle


def _full_row_plan(rng, rows, steps):
    plan = []
    for _ in range(steps):
        k = int(rng.integers(1, rows // 2))
        # skewed choice so that some rows come back after gaps of several steps
        r = np.unique((rows * rng.random(k) ** 3).astype(np.int64))
        plan.append(r)
    return plan


@pytest.mark.parametrize("wd_mode,wd", [("l2", 0.0), ("l2", 0.3), ("decoupled", 1.5)])
@pytest.mark.parametrize("mode", ["dormancy", "lazy"])
def test_row_granular_equals_per_coordinate(mode, wd_mode, wd):
    rng = np.random.default_rng(7)
    rows, cols, steps = 60, 12, 25
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    kw = dict(lr=1e-2, mode=mode, weight_decay=wd, weight_decay_mode=wd_mode)
    coord = oracle.Adam(p0.copy(), **kw)
    row = oracle.AdamRows(p0.copy(), **kw)
    for r in _full_row_plan(rng, rows, steps):
        g = rng.standard_normal((r.size, cols)).astype(np.float32)
        coord.step_coo(r, g, width=cols)
        row.step_coo(r, g, width=cols)
    for x, y in ((coord.p, row.p), (coord.m, row.m), (coord.v, row.v)):
        assert x.tobytes() == y.tobytes()
    # every coordinate of a row carries the row's value
    assert (coord.ls == coord.ls[:, :1]).all()
    assert np.array_equal(coord.ls[:, 0], row.ls)
    assert row.ls.max() == steps and (row.ls == 0).any()


def test_gaps_matter():
    """Negative control: the row's gap is used (not 1): a row touched at steps 1
    and 6 differs from a row touched at steps 5 and 6 with the same gradients."""
    p0 = np.ones((3, 4), np.float32)
    a = oracle.AdamRows(p0.copy(), mode="dormancy")
    b = oracle.AdamRows(p0.copy(), mode="dormancy")
    g = np.full((1, 4), 0.5, np.float32)
    a.step_coo([0], g, width=4)
    for _ in range(4):
        a.step_coo([2], g, width=4)
        b.step_coo([2], g, width=4)
    b.step_coo([0], g, width=4)
    a.step_coo([0], -g, width=4)
    b.step_coo([0], -g, width=4)
    assert a.ls[0] == b.ls[0] == 6
    assert np.abs(a.m[0] - b.m[0]).max() > 1e-3


def test_partial_row_is_refused_and_nothing_is_written():
    p0 = np.ones((4, 3), np.float32)
    a = oracle.AdamRows(p0.copy())
    ro = np.array([0, 3, 5, 5, 5], np.int32)      # row 1 has 2 of 3 entries
    ci = np.array([0, 1, 2, 0, 2], np.int32)
    g = np.ones(5, np.float32)
    with pytest.raises(oracle.OracleError) as e:
        a.step_csr(ro, ci, g)
    assert e.value.code == oracle.ESHAPE and a.t == 0
    assert a.p.tobytes() == p0.tobytes() and not a.ls.any()


def test_last_step_not_below_t_is_refused():
    a = oracle.AdamRows(np.ones((2, 2), np.float32))
    a.ls[1] = 5
    with pytest.raises(oracle.OracleError) as e:
        a.step_coo([1], np.ones((1, 2), np.float32), width=2)
    assert e.value.code == oracle.EINVAL
