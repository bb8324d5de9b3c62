"""Pins of the oracle's sparse SGD.

Page: docs.rs optirs_gpu sparse_optimizer, section "Sparse SGD" (params[i] -=
lr*grad[i] on touched coordinates, optional coupled weight decay and momentum
applied lazily on the touched coordinates, untouched coordinates bit-identical);
DiskSparseAdam README, "Explicit Weight Decay Semantics" ("l2": wd*w added to
the gradient) for what "coupled" means.
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("momentum,wd", [(0.0, 0.0), (0.9, 1e-4), (0.5, 0.0), (0.0, 1e-2)])
def test_all_touched_equals_torch_sgd(momentum, wd):
    rng = np.random.default_rng(1)
    dim, steps = 33, 20
    p0 = rng.standard_normal(dim)
    g = rng.standard_normal((steps, dim))
    s = oracle.Sgd64(p0, lr=0.05, momentum=momentum, weight_decay=wd)
    w = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.SGD([w], lr=0.05, momentum=momentum, dampening=0.0, weight_decay=wd)
    for t in range(steps):
        s.step(np.arange(dim), g[t])
        w.grad = torch.tensor(g[t])
        opt.step()
    np.testing.assert_allclose(s.p, w.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_single_step_closed_form():
    p0 = np.array([1.0, -2.0, 0.5])
    g = np.array([0.25, 1.0, -4.0])
    s = oracle.Sgd64(p0, lr=0.1, momentum=0.9, weight_decay=0.01)
    s.step(np.arange(3), g)
    np.testing.assert_allclose(s.p, p0 - 0.1 * (g + 0.01 * p0), rtol=1e-15)


def test_momentum_is_lazy():
    """Touched at steps 1 and 3 only: the buffer is not decayed at step 2.
    b1 = g1 + wd p0; b3 = mu b1 + (g3 + wd p1); p3 = p1 - lr b3."""
    lr, mu, wd = 0.1, 0.9, 0.01
    s = oracle.Sgd64([1.0, 5.0], lr=lr, momentum=mu, weight_decay=wd)
    s.step([0], [0.5])
    p1 = 1.0 - lr * (0.5 + wd * 1.0)
    b1 = 0.5 + wd * 1.0
    s.step([1], [1.0])
    assert s.p[0] == p1 and s.b[0] == b1
    s.step([0], [-0.25])
    b3 = mu * b1 + (-0.25 + wd * p1)
    assert s.b[0] == pytest.approx(b3, rel=1e-15)
    assert s.p[0] == pytest.approx(p1 - lr * b3, rel=1e-15)


def test_untouched_bit_identical_and_table_equals_flat():
    rng = np.random.default_rng(8)
    rows, cols = 25, 16
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    A = oracle.Sgd(p0.copy(), lr=0.05, momentum=0.9, weight_decay=1e-4)
    B = oracle.Sgd(p0.copy(), lr=0.05, momentum=0.9, weight_decay=1e-4)
    for _ in range(8):
        lin = np.unique(rng.integers(0, rows * cols, size=40))
        vals = rng.standard_normal(lin.size).astype(np.float32)
        before = (A.p.copy(), A.b.copy())
        ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
        A.step_csr(ro, ci, cv)
        B.step_coo(lin, vals)
        mask = np.ones(rows * cols, bool)
        mask[lin] = False
        assert A.p.reshape(-1)[mask].tobytes() == before[0].reshape(-1)[mask].tobytes()
        assert A.b.reshape(-1)[mask].tobytes() == before[1].reshape(-1)[mask].tobytes()
    assert A.p.tobytes() == B.p.tobytes() and A.b.tobytes() == B.b.tobytes()


@pytest.mark.parametrize("kw", [dict(lr=-0.1), dict(momentum=1.0), dict(momentum=-0.5),
                                dict(weight_decay=-1e-4)])
def test_bad_hyper_parameters(kw):
    args = dict(lr=0.1, momentum=0.9, weight_decay=0.0)
    args.update(kw)
    s = oracle.Sgd(np.ones((4, 1), np.float32), **args)
    with pytest.raises(oracle.OracleError) as e:
        s.step_coo([0], [1.0])
    assert e.value.code == oracle.EINVAL


def _lazy_touch_steps(rng, rows, cols, steps):
    """Per step: the sorted linear coordinates touched.  Coordinate 0 is touched
    at steps 0 and 3 only, so its momentum buffer sits untouched in between."""
    out = []
    for s in range(steps):
        lin = np.unique(rng.integers(1, rows * cols, size=int(rng.integers(1, 3 * cols))))
        if s in (0, 3):
            lin = np.r_[0, lin]
        out.append(lin.astype(np.int64))
    return out


def _step_float_oracle(A, form, lin, vals, rows, cols):
    if form == "coo":
        A.step_coo(lin, vals)
    else:
        ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
        A.step_csr(ro, ci, cv)


@pytest.mark.parametrize("form", ["coo", "csr"])
@pytest.mark.parametrize("momentum,wd", [(0.9, 1e-4), (0.0, 1e-2), (0.5, 0.0)])
def test_f32_state_is_f64_math_rounded_once(form, momentum, wd):
    """The float32-storage entry points (orc_sgd_coo_f32, orc_sgd_csr_f32) equal,
    bit for bit, the double-storage step started from the same float32 state and
    rounded once per stored value, at every step of a lazily touched run.  A
    momentum buffer that is not stored, or stored for the wrong coordinate, fails
    this from the second touch of a coordinate on."""
    rng = np.random.default_rng(31)
    rows, cols, steps = 19, 12, 12
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    A = oracle.Sgd(p0.copy(), lr=0.05, momentum=momentum, weight_decay=wd)
    for lin in _lazy_touch_steps(rng, rows, cols, steps):
        vals = rng.standard_normal(lin.size).astype(np.float32)
        ref = oracle.Sgd64(A.p.reshape(-1).astype(np.float64), lr=0.05, momentum=momentum,
                           weight_decay=wd)
        if momentum != 0.0:
            ref.b[:] = A.b.reshape(-1).astype(np.float64)
        ref.step(lin, vals.astype(np.float64))
        _step_float_oracle(A, form, lin, vals, rows, cols)
        assert A.p.reshape(-1).tobytes() == ref.p.astype(np.float32).tobytes()
        if momentum != 0.0:
            assert A.b.reshape(-1).tobytes() == ref.b.astype(np.float32).tobytes()
    if momentum != 0.0:
        assert A.b.reshape(-1)[0] != 0.0


@pytest.mark.parametrize("form", ["coo", "csr"])
@pytest.mark.parametrize("momentum,wd", [(0.9, 1e-4), (0.0, 1e-4)])
def test_f32_entry_points_equal_torch_sgd_on_touched_coordinates(form, momentum, wd):
    """Each step of the float32 entry points equals torch.optim.SGD (float64,
    dampening 0, coupled weight_decay) run on the touched coordinates only, with
    the momentum buffer they held before the step, within one float32 rounding:
    lazy momentum is heavy-ball momentum restricted to the touched set (page
    "optirs_gpu::sparse_optimizer", section Sparse SGD).  Independent of the
    oracle's own double path."""
    rng = np.random.default_rng(32)
    rows, cols, steps, lr = 23, 8, 10, 0.05
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    A = oracle.Sgd(p0.copy(), lr=lr, momentum=momentum, weight_decay=wd)
    for lin in _lazy_touch_steps(rng, rows, cols, steps):
        vals = rng.standard_normal(lin.size).astype(np.float32)
        w = torch.tensor(A.p.reshape(-1)[lin].astype(np.float64), requires_grad=True)
        opt = torch.optim.SGD([w], lr=lr, momentum=momentum, dampening=0.0, weight_decay=wd)
        if momentum != 0.0:
            opt.state[w]["momentum_buffer"] = torch.tensor(A.b.reshape(-1)[lin].astype(np.float64))
        w.grad = torch.tensor(vals.astype(np.float64))
        opt.step()
        untouched = np.ones(rows * cols, bool)
        untouched[lin] = False
        before_p = A.p.reshape(-1)[untouched].copy()
        _step_float_oracle(A, form, lin, vals, rows, cols)
        want_p = w.detach().numpy()
        got_p = A.p.reshape(-1)[lin].astype(np.float64)
        assert np.all(np.abs(got_p - want_p) <= 2.0 ** -24 * 1.000001 * np.abs(want_p) + 1e-300)
        assert A.p.reshape(-1)[untouched].tobytes() == before_p.tobytes()
        if momentum != 0.0:
            want_b = opt.state[w]["momentum_buffer"].numpy()
            got_b = A.b.reshape(-1)[lin].astype(np.float64)
            assert np.all(np.abs(got_b - want_b) <= 2.0 ** -24 * 1.000001 * np.abs(want_b) + 1e-300)


def test_full_row_coo_equals_flat_coo():
    """A full-row COO (width == cols, keys are rows) steps the same coordinates
    as the flattened COO of those rows, bit for bit."""
    rng = np.random.default_rng(33)
    rows, cols = 17, 6
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    A = oracle.Sgd(p0.copy(), lr=0.05, momentum=0.9, weight_decay=1e-4)
    B = oracle.Sgd(p0.copy(), lr=0.05, momentum=0.9, weight_decay=1e-4)
    for _ in range(6):
        keys = np.unique(rng.integers(0, rows, size=5))
        vals = rng.standard_normal((keys.size, cols)).astype(np.float32)
        A.step_coo(keys, vals, width=cols)
        B.step_coo((keys[:, None] * cols + np.arange(cols)).reshape(-1), vals.reshape(-1))
    assert A.p.tobytes() == B.p.tobytes() and A.b.tobytes() == B.b.tobytes()
