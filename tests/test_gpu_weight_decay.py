"""GPU parity of Adam with weight decay (coupled L2 and decoupled AdamW) against
the oracle.

Page: DiskSparseAdam README, "Explicit Weight Decay Semantics" (Euclidean case):
"l2" adds wd * w to the gradient, "decoupled" adds it to the descent direction.
The decay applies to touched coordinates only (docs.rs optirs_gpu
sparse_optimizer applies SGD's coupled decay that way).  Same bar as the
undecayed update: last_step bit-exact, state within 1e-5*|x| + 1e-7, untouched
coordinates bit-identical.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
import synth
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu

# Large enough that the decay moves the result well beyond the tolerance.
WD = {"l2": 0.5, "decoupled": 2.0}


def _pair(w, p0, mode, wd_mode, wd=None):
    h = w.hyper
    wd = WD[wd_mode] if wd is None else wd
    kw = dict(lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"], mode=mode,
              weight_decay=wd, weight_decay_mode=wd_mode)
    return oracle.Adam(p0.copy(), **kw), L.SparseAdam(dev(p0), **kw)


def _compare(ora, gpu, p0, what):
    torch.cuda.synchronize()
    assert gpu.t == ora.t
    assert np.array_equal(host(gpu.last_step), ora.ls), f"{what}: last_step differs"
    assert_state_close(host(gpu.params), ora.p, f"{what}: params")
    assert_state_close(host(gpu.m), ora.m, f"{what}: m")
    assert_state_close(host(gpu.v), ora.v, f"{what}: v")
    untouched = ora.ls.reshape(-1) == 0
    gp = host(gpu.params).reshape(-1)
    assert gp[untouched].tobytes() == p0.reshape(-1)[untouched].tobytes()


W3 = synth.WORKLOADS[3].scaled(rows=40000, n_lookups=4000, steps=10)


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
@pytest.mark.parametrize("mode", ["dormancy", "lazy"])
@pytest.mark.parametrize("form", ["csr_touched", "csr_scan", "block_coo", "flat_coo"])
def test_adam_weight_decay_on_oracle_gradient(form, mode, wd_mode):
    w = W3
    p0 = synth.init_params(w)
    ora, gpu = _pair(w, p0, mode, wd_mode)
    plain = oracle.Adam(p0.copy(), mode=mode)
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        plain.step_csr(ro, ci, cv)
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
    _compare(ora, gpu, p0, f"{form}/{mode}/{wd_mode}")
    # negative control: the decay changed the result beyond the tolerance
    touched = ora.ls != 0
    assert np.abs(ora.p[touched] - plain.p[touched]).max() > 1e-4


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
def test_partial_rows_with_weight_decay(wd_mode):
    w = synth.WORKLOAD_4_ADAM.scaled(rows=20000, n_rows_touched=1500, steps=8)
    p0 = synth.init_params(w)
    ora, gpu = _pair(w, p0, "dormancy", wd_mode)
    for s in range(w.steps):
        er, ec, ev = synth.partial_rows(w, s)
        lin = er * w.cols + ec
        ro, ci, cv = oracle.csr_from_coo(lin, ev, w.rows * w.cols, 1, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        gpu.step(L.CsrGradient(dev(ro), dev(ci), dev(cv), w.rows, w.cols,
                               touched_rows=dev(np.unique(er))))
    _compare(ora, gpu, p0, f"partial rows/{wd_mode}")


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
def test_1d_coo_with_weight_decay(wd_mode):
    w = synth.WORKLOADS[1]
    p0 = synth.init_params(w).reshape(-1)
    ora, gpu = _pair(w, p0, "dormancy", wd_mode)
    for s in range(w.steps):
        idx, vals = synth.coo1d(w, s)
        ora.step_coo(idx, vals)
        gpu.step(L.CooGradient(dev(idx), dev(vals), dim=w.rows, width=1))
    _compare(ora, gpu, p0, f"1-D/{wd_mode}")


def test_whole_path_with_decoupled_weight_decay():
    """Raw lookups through the GPU's canonicalisation and CSR assembly."""
    w = W3
    p0 = synth.init_params(w)
    ora, gpu = _pair(w, p0, "dormancy", "decoupled")
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        gk, gs, _, U = L.coo_from_lookups(dev(ids), dev(grads), w.rows)
        coo = L.CooGradient(gk, gs, dim=w.rows, width=w.cols, nnz=ids.size, d_nnz=U)
        gpu.step(L.csr_from_coo(coo, w.rows, w.cols, copy_values=False))
    _compare(ora, gpu, p0, "whole path/decoupled")


@pytest.mark.parametrize("wd_mode", ["l2", "decoupled"])
def test_zero_weight_decay_is_the_undecayed_step_bit_for_bit(wd_mode):
    w = W3
    p0 = synth.init_params(w)
    _, a = _pair(w, p0, "dormancy", wd_mode, wd=0.0)
    b = L.SparseAdam(dev(p0), lr=w.hyper["lr"], mode="dormancy")
    for s in range(4):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        g = L.CooGradient(dev(keys), dev(sums), dim=w.rows, width=w.cols)
        a.step(g)
        b.step(g)
    torch.cuda.synchronize()
    for x, y in ((a.params, b.params), (a.m, b.m), (a.v, b.v), (a.last_step, b.last_step)):
        assert host(x).tobytes() == host(y).tobytes()
