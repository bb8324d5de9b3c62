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
