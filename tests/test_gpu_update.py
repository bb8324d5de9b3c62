"""GPU parity of the sparse / lazy Adam and sparse SGD steps against the oracle.

Page: optirs_gpu sparse_optimizer ("Sparse SGD", "LazyAdamMode::Lazy",
"LazyAdamMode::DormancyDecay", global-step bias correction).  After N steps:
last_step bit-exact, params / m / v / momentum within 1e-5*|x| + 1e-7 of the
oracle, every untouched coordinate bit-identical to its initial value.

Two kinds of test: the update alone, fed the oracle's own canonical gradient
(so only the update arithmetic is compared), and the whole path from raw
lookups through the GPU's canonicalisation, CSR assembly and update.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
import synth
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu


def _adam_pair(w, p0, mode=None):
    h = w.hyper
    mode = mode or w.mode
    ora = oracle.Adam(p0.copy(), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                      mode=mode)
    gpu = L.SparseAdam(dev(p0), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                       mode=mode)
    return ora, gpu


def _sgd_pair(w, p0):
    h = w.hyper
    ora = oracle.Sgd(p0.copy(), lr=h["lr"], momentum=h["momentum"], weight_decay=h["weight_decay"])
    gpu = L.SparseSgd(dev(p0), lr=h["lr"], momentum=h["momentum"], weight_decay=h["weight_decay"])
    return ora, gpu


def _compare_adam(ora, gpu, p0, what):
    torch.cuda.synchronize()
    assert gpu.t == ora.t
    ls = host(gpu.last_step)
    assert np.array_equal(ls, ora.ls), f"{what}: last_step differs"
    assert_state_close(host(gpu.params), ora.p, f"{what}: params")
    assert_state_close(host(gpu.m), ora.m, f"{what}: m")
    assert_state_close(host(gpu.v), ora.v, f"{what}: v")
    untouched = ora.ls.reshape(-1) == 0
    gp = host(gpu.params).reshape(-1)
    assert gp[untouched].tobytes() == p0.reshape(-1)[untouched].tobytes()
    assert not host(gpu.m).reshape(-1)[untouched].any()
    assert not host(gpu.v).reshape(-1)[untouched].any()


def _compare_sgd(ora, gpu, p0, touched, what):
    torch.cuda.synchronize()
    assert_state_close(host(gpu.params), ora.p, f"{what}: params")
    if ora.b is not None:
        assert_state_close(host(gpu.momentum_buf), ora.b, f"{what}: momentum")
    gp = host(gpu.params).reshape(-1)
    assert gp[~touched].tobytes() == p0.reshape(-1)[~touched].tobytes()


# ---------------------------------------------------------------------------
# Update alone, fed the oracle's canonical gradient
# ---------------------------------------------------------------------------

SMALL_LOOKUP = {
    2: synth.WORKLOADS[2].scaled(rows=30000, n_lookups=3000, steps=12),
    3: synth.WORKLOADS[3].scaled(rows=40000, n_lookups=4000, steps=12),
    5: synth.WORKLOADS[5].scaled(rows=50000, n_lookups=6000, steps=8),
}


@pytest.mark.parametrize("cfg", [2, 3, 5])
@pytest.mark.parametrize("form", ["csr_touched", "csr_scan", "block_coo", "flat_coo"])
def test_adam_update_on_oracle_gradient(cfg, form):
    w = SMALL_LOOKUP[cfg]
    p0 = synth.init_params(w)
    ora, gpu = _adam_pair(w, p0)
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        if form == "csr_touched":
            g = L.CsrGradient(dev(ro), dev(ci), dev(cv), w.rows, w.cols, touched_rows=dev(keys))
        elif form == "csr_scan":
            g = L.CsrGradient(dev(ro), None, dev(cv), w.rows, w.cols)
        elif form == "block_coo":
            g = L.CooGradient(dev(keys), dev(sums), dim=w.rows, width=w.cols)
        else:
            lin, lv = oracle.csr_to_coo(ro, ci, cv, w.rows, w.cols)
            g = L.CooGradient(dev(lin), dev(lv), dim=w.rows * w.cols, width=1)
        gpu.step(g)
    _compare_adam(ora, gpu, p0, f"cfg{cfg}/{form}")


@pytest.mark.parametrize("mode", ["dormancy", "lazy"])
def test_adam_1d_coo(mode):
    """Config 1: a 4096-vector, 64 unique indices a step, 20 steps (full size)."""
    w = synth.WORKLOADS[1]
    p0 = synth.init_params(w).reshape(-1)
    ora, gpu = _adam_pair(w, p0, mode)
    for s in range(w.steps):
        idx, vals = synth.coo1d(w, s)
        ora.step_coo(idx, vals)
        gpu.step(L.CooGradient(dev(idx), dev(vals), dim=w.rows, width=1))
    _compare_adam(ora, gpu, p0, f"cfg1/{mode}")


@pytest.mark.parametrize("opt", ["sgd", "adam"])
@pytest.mark.parametrize("touched_list", [False, True])
def test_partial_rows(opt, touched_list):
    """Config 4 shape scaled: partial rows of 16-64 columns out of 256."""
    base = synth.WORKLOADS[4] if opt == "sgd" else synth.WORKLOAD_4_ADAM
    w = base.scaled(rows=20000, n_rows_touched=1500, steps=10)
    p0 = synth.init_params(w)
    if opt == "sgd":
        ora, gpu = _sgd_pair(w, p0)
    else:
        ora, gpu = _adam_pair(w, p0)
    touched = np.zeros(w.rows * w.cols, bool)
    for s in range(w.steps):
        er, ec, ev = synth.partial_rows(w, s)
        lin = er * w.cols + ec
        touched[lin] = True
        ro, ci, cv = oracle.csr_from_coo(lin, ev, w.rows * w.cols, 1, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        tr = dev(np.unique(er)) if touched_list else None
        gpu.step(L.CsrGradient(dev(ro), dev(ci), dev(cv), w.rows, w.cols, touched_rows=tr))
    if opt == "sgd":
        _compare_sgd(ora, gpu, p0, touched, "cfg4/sgd")
    else:
        _compare_adam(ora, gpu, p0, "cfg4/adam")


@pytest.mark.parametrize("momentum,wd", [(0.9, 1e-4), (0.0, 0.0), (0.0, 1e-3)])
def test_sgd_full_rows(momentum, wd):
    w = synth.WORKLOADS[4].scaled(kind="lookups", rows=20000, cols=64, n_lookups=3000, zipf_s=1.1,
                                  steps=8, grad_std=0.01,
                                  hyper={"lr": 0.05, "momentum": momentum, "weight_decay": wd})
    p0 = synth.init_params(w)
    ora, gpu = _sgd_pair(w, p0)
    touched = np.zeros(w.rows * w.cols, bool)
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        touched.reshape(w.rows, w.cols)[keys] = True
        ora.step_coo(keys, sums, width=w.cols)
        gpu.step(L.CooGradient(dev(keys), dev(sums), dim=w.rows, width=w.cols))
    _compare_sgd(ora, gpu, p0, touched, f"sgd mu={momentum} wd={wd}")


# ---------------------------------------------------------------------------
# Whole path from raw lookups
# ---------------------------------------------------------------------------

def gpu_lookup_step(gpu, ids_d, vals_d, rows, cols, key_space=None):
    keys, sums, counts, U = L.coo_from_lookups(ids_d, vals_d, key_space or rows)
    coo = L.CooGradient(keys, sums, dim=rows, width=cols, nnz=ids_d.numel(), d_nnz=U)
    csr = L.csr_from_coo(coo, rows, cols, copy_values=False)
    gpu.step(csr)
    return keys, counts, U


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_whole_path_from_lookups(cfg):
    w = SMALL_LOOKUP[cfg]
    p0 = synth.init_params(w)
    ora, gpu = _adam_pair(w, p0)
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, counts = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        gk, gc, U = gpu_lookup_step(gpu, dev(ids), dev(grads), w.rows, w.cols)
        torch.cuda.synchronize()
        u = int(host(U)[0])
        assert u == keys.size
        assert np.array_equal(host(gk)[:u], keys) and np.array_equal(host(gc)[:u], counts)
    _compare_adam(ora, gpu, p0, f"whole path cfg{cfg}")


# ---------------------------------------------------------------------------
# Validation, resume, determinism
# ---------------------------------------------------------------------------

def _snapshot(gpu):
    torch.cuda.synchronize()
    return [host(x).copy() for x in (gpu.params, gpu.m, gpu.v, gpu.last_step)], gpu.t


@pytest.mark.parametrize("case,code", [
    ("unsorted", oracle.ENOTCANON), ("duplicate", oracle.ENOTCANON), ("negative", oracle.ERANGE),
    ("too_large", oracle.ERANGE), ("nonfinite", oracle.ENONFINITE), ("csr_cols", oracle.ENOTCANON),
    ("csr_col_range", oracle.ERANGE), ("touched_list", oracle.ENOTCANON), ("shape", oracle.ESHAPE)])
def test_rejected_step_writes_nothing(case, code):
    rows, cols = 10, 4
    gpu = L.SparseAdam(dev(np.ones((rows, cols), np.float32)))
    gpu.step(L.CooGradient(dev(np.array([1, 2])), dev(np.full(2 * cols, 0.5, np.float32)), dim=rows,
                           width=cols), validate=True)
    snap, t = _snapshot(gpu)
    one = np.ones(2 * cols, np.float32)
    coo = {"unsorted": [3, 1], "duplicate": [1, 1], "negative": [-1, 2], "too_large": [2, 10]}
    if case in coo:
        g = L.CooGradient(dev(np.array(coo[case])), dev(one), dim=rows, width=cols)
    elif case == "nonfinite":
        bad = one.copy()
        bad[3] = np.nan
        g = L.CooGradient(dev(np.array([2, 3])), dev(bad), dim=rows, width=cols)
    elif case == "shape":
        g = L.CooGradient(dev(np.array([2, 3])), dev(one), dim=rows + 1, width=cols)
    else:
        ro = np.zeros(rows + 1, np.int32)
        ro[3:] = 2
        ci = np.array([2, 1] if case == "csr_cols" else [1, 4], np.int32)
        tr = dev(np.array([2, 5])) if case == "touched_list" else None
        if case == "touched_list":
            ci = np.array([0, 1], np.int32)
        g = L.CsrGradient(dev(ro), dev(ci), dev(np.ones(2, np.float32)), rows, cols,
                          touched_rows=tr)
    with pytest.raises(L.SparseOptError) as e:
        gpu.step(g, validate=True)
    assert e.value.code == code
    after, t2 = _snapshot(gpu)
    assert t2 == t
    for x, y in zip(after, snap):
        assert x.tobytes() == y.tobytes()


def test_empty_gradient_advances_t():
    gpu = L.SparseAdam(dev(np.ones((8, 4), np.float32)))
    gpu.step(L.CooGradient(torch.zeros(1, dtype=torch.int64, device="cuda"),
                           torch.zeros(4, device="cuda"), dim=8, width=4, nnz=0))
    assert gpu.t == 1


def test_resume_with_set_step_is_bit_identical():
    w = SMALL_LOOKUP[3].scaled(steps=10)
    p0 = synth.init_params(w)
    batches = [synth.lookups(w, s) for s in range(w.steps)]
    a = L.SparseAdam(dev(p0), mode="dormancy")
    for ids, g in batches:
        gpu_lookup_step(a, dev(ids), dev(g), w.rows, w.cols)
    b = L.SparseAdam(dev(p0), mode="dormancy")
    for ids, g in batches[:5]:
        gpu_lookup_step(b, dev(ids), dev(g), w.rows, w.cols)
    torch.cuda.synchronize()
    saved = [x.clone() for x in (b.params, b.m, b.v, b.last_step)]
    c = L.SparseAdam(saved[0])
    c.m.copy_(saved[1])
    c.v.copy_(saved[2])
    c.last_step.copy_(saved[3])
    c.handle.set_step(b.t)
    for ids, g in batches[5:]:
        gpu_lookup_step(c, dev(ids), dev(g), w.rows, w.cols)
    torch.cuda.synchronize()
    for x, y in zip((a.params, a.m, a.v, a.last_step), (c.params, c.m, c.v, c.last_step)):
        assert host(x).tobytes() == host(y).tobytes()


def test_two_runs_bit_identical():
    w = SMALL_LOOKUP[5].scaled(steps=4)
    p0 = synth.init_params(w)
    outs = []
    for _ in range(2):
        a = L.SparseAdam(dev(p0))
        for s in range(w.steps):
            ids, g = synth.lookups(w, s)
            gpu_lookup_step(a, dev(ids), dev(g), w.rows, w.cols)
        torch.cuda.synchronize()
        outs.append([host(x).tobytes() for x in (a.params, a.m, a.v, a.last_step)])
    assert outs[0] == outs[1]
