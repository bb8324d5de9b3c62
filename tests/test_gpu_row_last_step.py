"""GPU parity of Adam with one last_step per row (full-row tables).

Page: docs.rs optirs_gpu sparse_optimizer, "Lazy Adam" / "LazyAdamMode::
DormancyDecay": last_step per coordinate, gap = t - last_step.  In a table whose
gradients always cover whole rows every coordinate of a row holds the same
last_step, so one int32 per row is the same state.  Checked against the
oracle's row-granular step (itself pinned bit for bit to the per-coordinate
step) and against the GPU's own per-coordinate run, bit for bit.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
import synth
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu


def _pair(w, p0, mode, **kw):
    h = w.hyper
    base = dict(lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"], mode=mode, **kw)
    return (oracle.AdamRows(p0.copy(), **base),
            L.SparseAdam(dev(p0), last_step_per_row=True, **base),
            L.SparseAdam(dev(p0), **base))


def _compare(ora, gpu, coord, p0, what):
    torch.cuda.synchronize()
    assert gpu.t == ora.t
    assert np.array_equal(host(gpu.last_step), ora.ls), f"{what}: last_step differs"
    assert_state_close(host(gpu.params), ora.p, f"{what}: params")
    assert_state_close(host(gpu.m), ora.m, f"{what}: m")
    assert_state_close(host(gpu.v), ora.v, f"{what}: v")
    untouched = ora.ls == 0
    assert host(gpu.params)[untouched].tobytes() == p0[untouched].tobytes()
    # the same arithmetic as the per-coordinate layout, bit for bit
    for x, y in ((gpu.params, coord.params), (gpu.m, coord.m), (gpu.v, coord.v)):
        assert host(x).tobytes() == host(y).tobytes(), f"{what}: differs from per-coordinate"
    assert np.array_equal(host(coord.last_step)[:, 0], host(gpu.last_step))


def _run(w, mode, form, steps=None, **kw):
    p0 = synth.init_params(w)
    ora, gpu, coord = _pair(w, p0, mode, **kw)
    for s in range(steps or w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        if form == "csr_touched":
            g = L.CsrGradient(dev(ro), dev(ci), dev(cv), w.rows, w.cols, touched_rows=dev(keys))
        elif form == "csr_scan":
            g = L.CsrGradient(dev(ro), None, dev(cv), w.rows, w.cols)
        else:
            g = L.CooGradient(dev(keys), dev(sums), dim=w.rows, width=w.cols)
        gpu.step(g)
        coord.step(g)
    _compare(ora, gpu, coord, p0, f"{form}/{mode}/cols{w.cols}")


W3 = synth.WORKLOADS[3].scaled(rows=40000, n_lookups=4000, steps=12)


@pytest.mark.parametrize("mode", ["dormancy", "lazy"])
@pytest.mark.parametrize("form", ["csr_touched", "csr_scan", "block_coo"])
def test_row_last_step_on_oracle_gradient(form, mode):
    _run(W3, mode, form)


@pytest.mark.parametrize("cols", [6, 384, 64])
@pytest.mark.parametrize("form", ["csr_touched", "csr_scan"])
def test_row_last_step_other_widths(cols, form):
    """6 columns: the one-coordinate-at-a-time loops, several coordinates per
    lane; 384: several 16-byte vectors per lane; 64: 16 lanes per row."""
    w = W3.scaled(rows=5000, cols=cols, n_lookups=1500, steps=10)
    _run(w, "dormancy", form)


def test_row_last_step_with_weight_decay():
    _run(W3, "dormancy", "csr_touched", steps=8, weight_decay=1.0,
         weight_decay_mode="decoupled")


def test_whole_path_from_lookups():
    w = W3
    p0 = synth.init_params(w)
    ora, gpu, coord = _pair(w, p0, "dormancy")
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        gk, gs, _, U = L.coo_from_lookups(dev(ids), dev(grads), w.rows)
        coo = L.CooGradient(gk, gs, dim=w.rows, width=w.cols, nnz=ids.size, d_nnz=U)
        csr = L.csr_from_coo(coo, w.rows, w.cols, copy_values=False)
        gpu.step(csr)
        coord.step(csr)
    _compare(ora, gpu, coord, p0, "whole path")


def test_flat_coo_and_partial_rows_are_refused():
    rows, cols = 50, 8
    p0 = np.ones((rows, cols), np.float32)
    gpu = L.SparseAdam(dev(p0), last_step_per_row=True)
    flat = L.CooGradient(dev(np.array([3, 9], np.int64)), dev(np.ones(2, np.float32)),
                         dim=rows * cols, width=1)
    with pytest.raises(L.SparseOptError) as e:
        gpu.step(flat)
    assert e.value.code == oracle.ESHAPE
    ro = np.zeros(rows + 1, np.int32)
    ro[2:] = cols          # row 1 full
    ro[4:] = cols + 3      # row 3 partial (3 of 8 columns)
    ci = np.concatenate([np.arange(cols), np.arange(3)]).astype(np.int32)
    csr = L.CsrGradient(dev(ro), dev(ci), dev(np.ones(cols + 3, np.float32)), rows, cols)
    with pytest.raises(L.SparseOptError) as e:
        gpu.step(csr, validate=True)
    assert e.value.code == oracle.ESHAPE
    torch.cuda.synchronize()
    assert gpu.t == 0 and host(gpu.params).tobytes() == p0.tobytes()
    assert not host(gpu.last_step).any()
