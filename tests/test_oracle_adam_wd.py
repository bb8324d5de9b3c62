"""Pins of the oracle's Adam weight decay against what the pages and libraries fix.

Pages: DiskSparseAdam README, "Explicit Weight Decay Semantics" and the
weight_decay / weight_decay_mode arguments of its API reference: in the
Euclidean case "l2" is classic Adam L2 (wd * w added to the gradient) and
"decoupled" is AdamW (wd * w added to the descent direction).  docs.rs
optirs_gpu sparse_optimizer, "Sparse SGD": decay on the touched coordinates
only, which is the reading taken for Adam as well.
"""
import numpy as np
import pytest
import torch

import oracle

WD = 0.05
LR = 1e-2


def _dense_run(mode, wd_mode, steps=40, dim=24, seed=3):
    """Every coordinate touched every step (gap == 1): sparse Adam with decay
    must be the library's dense optimizer."""
    rng = np.random.default_rng(seed)
    p0 = rng.standard_normal(dim)
    g = rng.standard_normal((steps, dim))
    a = oracle.Adam64(p0, lr=LR, mode=mode, weight_decay=WD, weight_decay_mode=wd_mode)
    w = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    if wd_mode == "l2":
        opt = torch.optim.Adam([w], lr=LR, betas=(0.9, 0.999), eps=1e-8, weight_decay=WD)
    else:
        opt = torch.optim.AdamW([w], lr=LR, betas=(0.9, 0.999), eps=1e-8, weight_decay=WD)
    for t in range(steps):
        a.step(np.arange(dim), g[t])
        w.grad = torch.tensor(g[t])
        opt.step()
    return a, w.detach().numpy(), opt.state[w]


@pytest.mark.parametrize("mode", ["lazy", "dormancy"])
def test_l2_all_touched_equals_torch_adam_weight_decay(mode):
    a, ref, st = _dense_run(mode, "l2")
    np.testing.assert_allclose(a.p, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a.m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(a.v, st["exp_avg_sq"].numpy(), rtol=1e-13)


@pytest.mark.parametrize("mode", ["lazy", "dormancy"])
def test_decoupled_all_touched_equals_torch_adamw(mode):
    a, ref, st = _dense_run(mode, "decoupled")
    np.testing.assert_allclose(a.p, ref, rtol=1e-13, atol=1e-15)
    # decoupled decay leaves the moments those of the plain gradient
    np.testing.assert_allclose(a.m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(a.v, st["exp_avg_sq"].numpy(), rtol=1e-13)


def test_modes_differ_and_l2_changes_the_moments():
    """Negative control: the two modes are different methods."""
    a_l2, _, _ = _dense_run("dormancy", "l2")
    a_dc, _, _ = _dense_run("dormancy", "decoupled")
    assert np.abs(a_l2.p - a_dc.p).max() > 1e-6
    assert np.abs(a_l2.m - a_dc.m).max() > 1e-6


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
def test_first_step_closed_forms(wd_mode):
    """t = 1: m_hat = g', v_hat = g'^2, so p1 = p0 - lr * g' / (|g'| + eps) with
    g' = g + wd * p0 for "l2"; "decoupled" moves by the plain Adam step and
    then by -lr * wd * p0."""
    p0 = np.array([0.75, -1.5, 2.0, 0.0])
    g = np.array([0.5, 0.25, -3.0, 1e-3])
    eps = 1e-8
    a = oracle.Adam64(p0, lr=LR, eps=eps, weight_decay=WD, weight_decay_mode=wd_mode)
    a.step(np.arange(4), g)
    if wd_mode == "l2":
        gp = g + WD * p0
        want = p0 - LR * gp / (np.abs(gp) + eps)
        np.testing.assert_allclose(a.m, 0.1 * gp, rtol=1e-15)
    else:
        want = p0 - LR * g / (np.abs(g) + eps) - LR * WD * p0
        np.testing.assert_allclose(a.m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(a.p, want, rtol=1e-14, atol=1e-17)


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
@pytest.mark.parametrize("mode", ["lazy", "dormancy"])
def test_zero_weight_decay_is_the_undecayed_step_bit_for_bit(mode, wd_mode):
    rng = np.random.default_rng(11)
    rows, cols, steps = 30, 8, 12
    p0 = rng.standard_normal((rows, cols)).astype(np.float32)
    a = oracle.Adam(p0.copy(), mode=mode)
    b = oracle.Adam(p0.copy(), mode=mode, weight_decay=0.0, weight_decay_mode=wd_mode)
    for _ in range(steps):
        idx = np.sort(rng.choice(rows * cols, size=40, replace=False)).astype(np.int64)
        vals = rng.standard_normal(40).astype(np.float32)
        a.step_coo(idx, vals)
        b.step_coo(idx, vals)
    for x, y in ((a.p, b.p), (a.m, b.m), (a.v, b.v), (a.ls, b.ls)):
        assert x.tobytes() == y.tobytes()


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
def test_decay_applies_at_touches_only(wd_mode):
    """A dormant coordinate does not shrink: its parameter is bit-identical
    between touches, untouched coordinates keep their initial bits, and the
    result differs from dense AdamW / Adam-L2 fed zero gradients while dormant
    (which shrink every step)."""
    p0 = np.array([1.0, -2.0, 0.5])
    a = oracle.Adam64(p0, lr=LR, weight_decay=WD, weight_decay_mode=wd_mode)
    a.step([0], [0.3])                                 # t = 1
    after_first = a.p.copy()
    for _ in range(4):                                 # t = 2..5: coordinate 0 dormant
        a.step([1], [0.2])
    assert a.p[0] == after_first[0] and a.p[2] == p0[2]
    a.step([0], [-0.1])                                # t = 6
    w = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = (torch.optim.Adam([w], lr=LR, weight_decay=WD) if wd_mode == "l2"
           else torch.optim.AdamW([w], lr=LR, weight_decay=WD))
    for t, (i, gi) in enumerate([(0, 0.3), (1, 0.2), (1, 0.2), (1, 0.2), (1, 0.2), (0, -0.1)]):
        gr = np.zeros(3)
        gr[i] = gi
        w.grad = torch.tensor(gr)
        opt.step()
    assert abs(w.detach().numpy()[2] - p0[2]) > 1e-6   # dense decays the never-touched one
    assert abs(a.p[0] - w.detach().numpy()[0]) > 1e-9


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
def test_f32_state_is_f64_math_rounded_once_with_decay(wd_mode):
    rng = np.random.default_rng(2)
    p0 = rng.standard_normal(16).astype(np.float32)
    g = rng.standard_normal(16).astype(np.float32)
    a32 = oracle.Adam(p0.reshape(16, 1).copy(), weight_decay=WD, weight_decay_mode=wd_mode)
    a64 = oracle.Adam64(p0.astype(np.float64), weight_decay=WD, weight_decay_mode=wd_mode)
    a32.step_coo(np.arange(16), g)
    a64.step(np.arange(16), g.astype(np.float64))
    assert a32.p.reshape(-1).tobytes() == a64.p.astype(np.float32).tobytes()
    assert a32.m.reshape(-1).tobytes() == a64.m.astype(np.float32).tobytes()


@pytest.mark.parametrize("wd", [-1e-3, float("nan"), float("inf")])
def test_bad_weight_decay(wd):
    a = oracle.Adam(np.ones((4, 1), np.float32), weight_decay=wd)
    with pytest.raises(oracle.OracleError) as e:
        a.step_coo([0], [1.0])
    assert e.value.code == oracle.EINVAL and a.t == 0


def test_bad_weight_decay_mode():
    with pytest.raises(ValueError):
        oracle.Adam(np.ones((4, 1), np.float32), weight_decay_mode="adamw")
    a = oracle.Adam(np.ones((4, 1), np.float32), weight_decay=0.1)
    a.cfg.wd_mode = 2
    with pytest.raises(oracle.OracleError) as e:
        a.step_coo([0], [1.0])
    assert e.value.code == oracle.EINVAL
