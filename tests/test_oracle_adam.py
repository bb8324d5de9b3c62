"""Pins of the oracle's sparse / lazy Adam against what the pages and the maths fix.

Page: docs.rs optirs_gpu sparse_optimizer (module page), sections
"Lazy Adam", "LazyAdamMode::Lazy", "LazyAdamMode::DormancyDecay" and the
remark that bias correction uses the global step count.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F = Fraction


def _touch_plan(rng, dim, steps, p_touch):
    """Random touch masks; every step touches at least one coordinate."""
    plan = []
    for _ in range(steps):
        mask = rng.random(dim) < p_touch
        if not mask.any():
            mask[rng.integers(dim)] = True
        plan.append(np.nonzero(mask)[0])
    return plan


def _rational_grad(rng):
    return F(int(rng.integers(-40, 41)), int(rng.integers(1, 9)))


# ---------------------------------------------------------------------------
# Worked example (tests/golden): hand-derived from the page's equations
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["dormancy", "lazy"])
def test_worked_example(mode):
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_one_coordinate.json")))
    h = {k: F(v) for k, v in ex["hyper"].items()}
    a = oracle.Adam64([float(h["p0"])], lr=float(h["lr"]), beta1=float(h["beta1"]),
                      beta2=float(h["beta2"]), eps=float(h["eps"]), mode=mode)
    a.step([0], [2.0])
    e1 = ex["after_t1"]
    assert a.m[0] == float(F(e1["m"])) and a.v[0] == float(F(e1["v"])) and a.ls[0] == 1
    p1 = exact.D(1) - exact.D(h["lr"]) * exact.D(F(e1["m_hat"])) / (
        exact.D(F(e1["v_hat"])).sqrt() + exact.D(h["eps"]))
    assert abs(a.p[0] - float(p1)) <= 1e-15
    a.step(np.zeros(0, np.int64), np.zeros(0))          # t = 2: coordinate dormant
    assert a.ls[0] == 1 and a.m[0] == 1.0
    a.step([0], [4.0])
    e3 = ex["after_t3"][mode]
    assert a.m[0] == float(F(e3["m"])) and a.v[0] == float(F(e3["v"])) and a.ls[0] == 3
    p3 = p1 - exact.D(h["lr"]) * exact.D(F(e3["m_hat"])) / (
        exact.D(F(e3["v_hat"])).sqrt() + exact.D(h["eps"]))
    assert abs(a.p[0] - float(p3)) <= 1e-15


# ---------------------------------------------------------------------------
# DormancyDecay moments == dense Adam fed explicit zeros (exact brute force)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_dormancy_moments_equal_dense_adam_with_zeros(seed):
    rng = np.random.default_rng(seed)
    dim, steps = int(rng.integers(1, 9)), int(rng.integers(3, 13))
    b1, b2 = F(9, 10), F(999, 1000)
    plan = _touch_plan(rng, dim, steps, 0.4)
    grads = [{int(i): _rational_grad(rng) for i in idx} for idx in plan]
    a = oracle.Adam64(np.zeros(dim), lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, mode="dormancy")
    for t in range(steps):
        idx = np.array(sorted(grads[t]), np.int64)
        a.step(idx, [float(grads[t][int(i)]) for i in idx])
        for i in idx:
            dense_g = [grads[s].get(int(i), F(0)) for s in range(t + 1)]
            ms, vs = exact.dense_adam_moments(dense_g, b1, b2)
            assert a.m[i] == pytest.approx(float(ms[-1]), rel=1e-12, abs=1e-300)
            assert a.v[i] == pytest.approx(float(vs[-1]), rel=1e-12, abs=1e-300)


def test_lazy_moments_ignore_the_gap():
    """Lazy: one decay per touch, exact closed form whatever the gap."""
    rng = np.random.default_rng(7)
    b1, b2 = F(9, 10), F(999, 1000)
    touch_steps = [1, 2, 7, 8, 30]
    gs = [_rational_grad(rng) for _ in touch_steps]
    a = oracle.Adam64([0.0], mode="lazy")
    k = 0
    for t in range(1, 31):
        if t in touch_steps:
            a.step([0], [float(gs[k])])
            m, v = exact.lazy_moments(list(zip(touch_steps, gs))[:k + 1], b1, b2)[-1]
            assert a.m[0] == pytest.approx(float(m), rel=1e-13)
            assert a.v[0] == pytest.approx(float(v), rel=1e-13)
            k += 1
        else:
            a.step(np.zeros(0, np.int64), np.zeros(0))
    # and it differs from DormancyDecay once a gap > 1 has occurred
    d = oracle.Adam64([0.0], mode="dormancy")
    k = 0
    for t in range(1, 31):
        if t in touch_steps:
            d.step([0], [float(gs[k])])
            k += 1
        else:
            d.step(np.zeros(0, np.int64), np.zeros(0))
    assert d.m[0] != a.m[0]


def test_lazy_and_dormancy_agree_when_every_gap_is_one():
    rng = np.random.default_rng(3)
    g = rng.standard_normal((10, 6))
    a = oracle.Adam64(np.ones(6), mode="lazy")
    d = oracle.Adam64(np.ones(6), mode="dormancy")
    assert pow(0.9, 1.0) == 0.9 and pow(0.999, 1.0) == 0.999   # host libm
    for t in range(10):
        a.step(np.arange(6), g[t])
        d.step(np.arange(6), g[t])
    assert np.array_equal(a.p, d.p) and np.array_equal(a.m, d.m) and np.array_equal(a.v, d.v)


# ---------------------------------------------------------------------------
# gap == 1 reduces to standard Adam: torch.optim.Adam in float64
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["dormancy", "lazy"])
def test_all_touched_equals_torch_adam(mode):
    rng = np.random.default_rng(11)
    dim, steps = 37, 25
    p0 = rng.standard_normal(dim)
    g = rng.standard_normal((steps, dim)) * 0.1
    a = oracle.Adam64(p0, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, mode=mode)
    w = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([w], lr=1e-2, betas=(0.9, 0.999), eps=1e-8)
    for t in range(steps):
        a.step(np.arange(dim), g[t])
        w.grad = torch.tensor(g[t])
        opt.step()
        assert a.ls.min() == t + 1
    ref = w.detach().numpy()
    np.testing.assert_allclose(a.p, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a.m, opt.state[w]["exp_avg"].numpy(), rtol=1e-13)
    np.testing.assert_allclose(a.v, opt.state[w]["exp_avg_sq"].numpy(), rtol=1e-13)


def test_lazy_equals_torch_sparse_adam():
    """torch.optim.SparseAdam updates only the touched values with one decay per
    touch and global-step bias correction; its eps sits at eps/sqrt(bc2) in our
    notation, so eps is made negligible here."""
    rng = np.random.default_rng(5)
    dim, steps = 50, 30
    p0 = rng.standard_normal(dim)
    a = oracle.Adam64(p0, lr=1e-2, eps=1e-30, mode="lazy")
    w = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.SparseAdam([w], lr=1e-2, betas=(0.9, 0.999), eps=1e-30)
    for t in range(steps):
        n = int(rng.integers(1, 12))
        raw = rng.integers(0, dim, size=n)                 # duplicates allowed
        vals = rng.standard_normal(n)
        w.grad = torch.sparse_coo_tensor(torch.tensor(raw)[None, :], torch.tensor(vals), (dim,))
        opt.step()
        u = np.unique(raw)
        summed = np.array([vals[raw == i].sum() for i in u])
        a.step(u, summed)
    np.testing.assert_allclose(a.p, w.detach().numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Closed forms: first step, first touch at t0 > 1 (global t), eps placement
# ---------------------------------------------------------------------------

def test_first_step_closed_form():
    g = np.array([3.0, -0.5, 1e-3, -7.0])
    a = oracle.Adam64(np.zeros(4), lr=0.01, eps=1e-8)
    a.step(np.arange(4), g)
    np.testing.assert_allclose(a.p, -0.01 * g / (np.abs(g) + 1e-8), rtol=1e-14)


@pytest.mark.parametrize("t0", [2, 5, 40, 300])
def test_first_touch_uses_global_step(t0):
    """A coordinate first touched at global step t0 moves by
    -lr * [(1-b1)/(1-b1^t0)] g / (|g| sqrt((1-b2)/(1-b2^t0)) + eps);
    per-coordinate counting would instead give about -lr*sign(g)."""
    lr, b1, b2, eps, g = 1e-3, 0.9, 0.999, 1e-8, 0.37
    a = oracle.Adam64([1.0, 0.0], lr=lr, beta1=b1, beta2=b2, eps=eps, mode="dormancy")
    for _ in range(t0 - 1):
        a.step([1], [1.0])
    a.step([0], [g])
    c1 = (1 - b1) / (1 - b1 ** t0)
    c2 = np.sqrt((1 - b2) / (1 - b2 ** t0))
    expect = 1.0 - lr * c1 * g / (abs(g) * c2 + eps)
    assert a.p[0] == pytest.approx(expect, rel=1e-14)
    if t0 >= 5:
        assert abs((1.0 - a.p[0]) - lr) > 1e-5      # not the per-row-counter answer


def test_eps_is_added_after_the_square_root():
    """At t = 1, Delta p = -lr g / (|g| + eps): with g = eps the step is lr/2.
    Inside the root it would be -lr g / sqrt(g^2 + eps) instead."""
    a = oracle.Adam64([0.0], lr=1.0, eps=1e-8)
    a.step([0], [1e-8])
    assert a.p[0] == pytest.approx(-0.5, rel=1e-12)


def test_params_differ_from_dense_adam_with_gaps():
    """Negative control: moments agree with dense Adam fed zeros, params do not."""
    p0 = np.array([1.0])
    a = oracle.Adam64(p0, lr=1e-2, mode="dormancy")
    w = torch.tensor(p0, requires_grad=True)
    opt = torch.optim.Adam([w], lr=1e-2)
    gs = [0.5, 0.0, 0.0, -0.25]
    for t, g in enumerate(gs):
        if g != 0.0:
            a.step([0], [g])
        else:
            a.step(np.zeros(0, np.int64), np.zeros(0))
        w.grad = torch.tensor([g], dtype=torch.float64)
        opt.step()
    assert a.m[0] == pytest.approx(opt.state[w]["exp_avg"].item(), rel=1e-14)
    assert a.v[0] == pytest.approx(opt.state[w]["exp_avg_sq"].item(), rel=1e-14)
    assert abs(a.p[0] - w.item()) > 1e-4


# ---------------------------------------------------------------------------
# Float storage, last_step, untouched coordinates, table == flattened 1-D
# ---------------------------------------------------------------------------

def test_f32_state_is_f64_math_rounded_once():
    rng = np.random.default_rng(2)
    dim = 64
    p0 = rng.standard_normal(dim).astype(np.float32)
    g = rng.standard_normal(dim).astype(np.float32)
    a32 = oracle.Adam(p0.copy().reshape(dim, 1))
    a64 = oracle.Adam64(p0.astype(np.float64))
    a32.step_coo(np.arange(dim), g)
    a64.step(np.arange(dim), g.astype(np.float64))
    assert np.array_equal(a32.p.reshape(-1), a64.p.astype(np.float32))
    assert np.array_equal(a32.m.reshape(-1), a64.m.astype(np.float32))
    assert np.array_equal(a32.v.reshape(-1), a64.v.astype(np.float32))


def test_last_step_and_untouched_bit_identical():
    rng = np.random.default_rng(4)
    rows, cols, steps = 40, 6, 15
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    a = oracle.Adam(p0.copy(), mode="dormancy")
    last = np.zeros((rows, cols), np.int32)
    for t in range(1, steps + 1):
        before = (a.p.copy(), a.m.copy(), a.v.copy(), a.ls.copy())
        lin = np.unique(rng.integers(0, rows * cols, size=int(rng.integers(0, 30))))
        a.step_coo(lin, rng.standard_normal(lin.size).astype(np.float32))
        last.reshape(-1)[lin] = t
        untouched = np.ones(rows * cols, bool)
        untouched[lin] = False
        for new, old in zip((a.p, a.m, a.v, a.ls), before):
            assert new.reshape(-1)[untouched].tobytes() == old.reshape(-1)[untouched].tobytes()
        assert np.array_equal(a.ls, last)
    assert a.t == steps


def test_table_forms_equal_flattened_1d():
    """CSR table step == block-COO step == 1-D step over row*cols+col, bitwise."""
    rng = np.random.default_rng(9)
    rows, cols = 30, 8
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    A = oracle.Adam(p0.copy())
    B = oracle.Adam(p0.copy())
    Cc = oracle.Adam(p0.copy())
    for _ in range(6):
        trows = np.unique(rng.integers(0, rows, size=10))
        vals = rng.standard_normal((trows.size, cols)).astype(np.float32)
        ro, ci, cv = oracle.csr_from_coo(trows, vals, rows, cols, rows, cols)
        A.step_csr(ro, ci, cv)
        B.step_coo(trows, vals, width=cols)
        lin, lv = oracle.csr_to_coo(ro, ci, cv, rows, cols)
        Cc.step_coo(lin, lv)
    for x, y, z in ((A.p, B.p, Cc.p), (A.m, B.m, Cc.m), (A.v, B.v, Cc.v), (A.ls, B.ls, Cc.ls)):
        assert x.tobytes() == y.tobytes() == z.tobytes()


# ---------------------------------------------------------------------------
# Rejected calls write nothing and leave t alone
# ---------------------------------------------------------------------------

def _snapshot(a):
    return [x.copy() for x in (a.p, a.m, a.v, a.ls)], a.t


@pytest.mark.parametrize("case,code", [
    ("unsorted", oracle.ENOTCANON), ("duplicate", oracle.ENOTCANON), ("negative", oracle.ERANGE),
    ("too_large", oracle.ERANGE), ("nonfinite", oracle.ENONFINITE)])
def test_rejected_step_writes_nothing(case, code):
    a = oracle.Adam(np.ones((10, 1), np.float32))
    a.step_coo([1, 2], [0.5, 0.5])
    snap, t = _snapshot(a)
    idx, vals = {"unsorted": ([3, 1], [1.0, 1.0]), "duplicate": ([1, 1], [1.0, 1.0]),
                 "negative": ([-1, 2], [1.0, 1.0]), "too_large": ([2, 10], [1.0, 1.0]),
                 "nonfinite": ([2, 3], [1.0, np.inf])}[case]
    with pytest.raises(oracle.OracleError) as e:
        a.step_coo(idx, vals, check_finite=True)
    assert e.value.code == code
    for x, y in zip((a.p, a.m, a.v, a.ls), snap):
        assert x.tobytes() == y.tobytes()
    assert a.t == t


@pytest.mark.parametrize("kw", [dict(beta1=1.0), dict(beta1=-0.1), dict(beta2=1.0), dict(eps=0.0),
                                dict(lr=-1e-3), dict(eps=float("nan"))])
def test_bad_hyper_parameters(kw):
    a = oracle.Adam(np.ones((4, 1), np.float32), **kw)
    with pytest.raises(oracle.OracleError) as e:
        a.step_coo([0], [1.0])
    assert e.value.code == oracle.EINVAL and a.t == 0
