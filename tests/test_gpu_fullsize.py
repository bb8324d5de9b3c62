"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (raw lookups -> csr_from_lookups -> step; the 1M x 64 run takes
the two calls coo_from_lookups -> csr_from_coo instead).

* 1M x 64 Lazy, 100 steps: every coordinate of the table against the oracle.
* 2M x 256 partial rows, SGD then DormancyDecay Adam, 100 steps each: every
  coordinate against the oracle.
* 10M x 128 (200 steps) and 50M x 128 (50 steps) DormancyDecay: every step's
  distinct keys and multiplicities and three steps' row_offsets bit-exact
  against the oracle; the state of sampled rows (the hottest rows, random
  touched rows, rows touched once) against the oracle run on those rows only,
  and every never-touched row of the table bit-identical to its initial
  values, with m = v = last_step = 0.
The 1-D 4096-vector workload runs at full size in test_gpu_update.
Pages: optirs_gpu sparse_optimizer (the update, canonical COO/CSR, untouched
coordinates bit-identical); DiskSparseAdam README (duplicates summed).
"""
import gc
import sys
import time

import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
import synth
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu


def log(msg):
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _free_gpu():
    yield
    gc.collect()
    torch.cuda.empty_cache()


class LookupPath:
    """The benchmark's per-step calls with preallocated outputs: the one call
    sparse_step_from_lookups (mode "one_call", the benchmark's default),
    csr_from_lookups then the step ("two_calls"), or coo_from_lookups,
    csr_from_coo, then the step ("separate")."""

    def __init__(self, opt, rows, cols, n, mode="one_call"):
        self.opt, self.rows, self.cols, self.n, self.mode = opt, rows, cols, n, mode
        self.keys = torch.empty(n, dtype=torch.int64, device="cuda")
        self.sums = torch.empty((n, cols), dtype=torch.float32, device="cuda")
        self.counts = torch.empty(n, dtype=torch.int32, device="cuda")
        self.U = torch.empty(1, dtype=torch.int64, device="cuda")
        self.ws = torch.empty(L.sparse_opt_workspace_size(n, cols, rows), dtype=torch.uint8,
                              device="cuda")
        self.row_offsets = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
        self.col_indices = torch.empty(n * cols, dtype=torch.int32, device="cuda")

    def step(self, ids, grads):
        out = dict(out_keys=self.keys, out_vals=self.sums, out_counts=self.counts,
                   d_nunique=self.U, row_offsets=self.row_offsets,
                   col_indices=self.col_indices, workspace=self.ws)
        if self.mode == "one_call":
            self.opt.step_lookups(dev(ids), dev(grads), **out)
            return
        if self.mode == "two_calls":
            csr, _, _ = L.csr_from_lookups(dev(ids), dev(grads), self.rows, **out)
        else:
            L.coo_from_lookups(dev(ids), dev(grads), self.rows, out_keys=self.keys,
                               out_vals=self.sums, out_counts=self.counts, d_nunique=self.U,
                               workspace=self.ws)
            coo = L.CooGradient(self.keys, self.sums, dim=self.rows, width=self.cols,
                                nnz=self.n, d_nnz=self.U)
            csr = L.csr_from_coo(coo, self.rows, self.cols, row_offsets=self.row_offsets,
                                 col_indices=self.col_indices, copy_values=False)
        self.opt.step(csr)


def test_table_1M_x_64_lazy_full_compare():
    w = synth.WORKLOADS[2]
    h = w.hyper
    p0 = synth.init_params(w)
    ora = oracle.Adam(p0.copy(), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                      mode="lazy")
    gpu = L.SparseAdam(dev(p0), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                       mode="lazy")
    path = LookupPath(gpu, w.rows, w.cols, w.n_lookups, mode="separate")
    for s, (ids, grads) in enumerate(synth.lookups_many(w, range(w.steps))):
        keys, sums, counts = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        path.step(ids, grads)
        torch.cuda.synchronize()
        u = int(host(path.U)[0])
        assert u == keys.size
        assert np.array_equal(host(path.keys)[:u], keys)
        assert np.array_equal(host(path.counts)[:u], counts)
        if s in (0, w.steps - 1):
            assert np.array_equal(host(path.row_offsets), ro)
            assert np.array_equal(host(path.col_indices)[:u * w.cols], ci)
    torch.cuda.synchronize()
    assert np.array_equal(host(gpu.last_step), ora.ls)
    assert_state_close(host(gpu.params), ora.p, "1Mx64 params")
    assert_state_close(host(gpu.m), ora.m, "1Mx64 m")
    assert_state_close(host(gpu.v), ora.v, "1Mx64 v")
    untouched = ora.ls.reshape(-1) == 0
    assert host(gpu.params).reshape(-1)[untouched].tobytes() == p0.reshape(-1)[untouched].tobytes()


@pytest.mark.parametrize("opt", ["sgd", "adam"])
def test_table_2M_x_256_partial_rows_full_compare(opt):
    w = synth.WORKLOADS[4] if opt == "sgd" else synth.WORKLOAD_4_ADAM
    h = w.hyper
    p0 = synth.init_params(w)
    if opt == "sgd":
        ora = oracle.Sgd(p0.copy(), lr=h["lr"], momentum=h["momentum"],
                         weight_decay=h["weight_decay"])
        gpu = L.SparseSgd(dev(p0), lr=h["lr"], momentum=h["momentum"],
                          weight_decay=h["weight_decay"])
    else:
        ora = oracle.Adam(p0.copy(), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"],
                          eps=h["eps"], mode="dormancy")
        gpu = L.SparseAdam(dev(p0), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                           mode="dormancy")
    row_offsets = torch.empty(w.rows + 1, dtype=torch.int32, device="cuda")
    touched = np.zeros(w.rows * w.cols, bool)
    t0 = time.time()
    entries = synth.partial_rows_many(w, range(w.steps))
    log(f"2Mx256 {opt}: inputs in {time.time() - t0:.1f} s")
    for s, (er, ec, ev) in enumerate(entries):
        lin = er * w.cols + ec
        touched[lin] = True
        ro, ci, cv = oracle.csr_from_coo(lin, ev, w.rows * w.cols, 1, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        coo = L.CooGradient(dev(lin), dev(ev), dim=w.rows * w.cols, width=1)
        csr = L.csr_from_coo(coo, w.rows, w.cols, row_offsets=row_offsets)
        gpu.step(csr)
        if s in (0, w.steps - 1):
            torch.cuda.synchronize()
            assert np.array_equal(host(csr.row_offsets), ro)
            assert np.array_equal(host(csr.col_indices)[:lin.size], ci)
    torch.cuda.synchronize()
    assert_state_close(host(gpu.params), ora.p, f"2Mx256 {opt} params")
    gp = host(gpu.params).reshape(-1)
    assert gp[~touched].tobytes() == p0.reshape(-1)[~touched].tobytes()
    if opt == "sgd":
        assert_state_close(host(gpu.momentum_buf), ora.b, "2Mx256 sgd momentum")
    else:
        assert np.array_equal(host(gpu.last_step), ora.ls)
        assert_state_close(host(gpu.m), ora.m, "2Mx256 adam m")
        assert_state_close(host(gpu.v), ora.v, "2Mx256 adam v")


def _sampled_lookup_run(cfg, mode="one_call"):
    w = synth.WORKLOADS[cfg]
    h = w.hyper
    R, C = w.rows, w.cols
    t0 = time.time()
    p0 = synth.init_params(w)
    log(f"cfg{cfg}: initial table in {time.time() - t0:.1f} s")
    gpu = L.SparseAdam(torch.from_numpy(p0).to("cuda"), lr=h["lr"], beta1=h["beta1"],
                       beta2=h["beta2"], eps=h["eps"], mode=w.mode)
    path = LookupPath(gpu, R, C, w.n_lookups, mode)
    t0 = time.time()
    batches = synth.lookups_many(w, range(w.steps))
    log(f"cfg{cfg}: {w.steps} steps of lookups in {time.time() - t0:.1f} s")
    check_ro = {0, w.steps // 2, w.steps - 1}
    touch_count = np.zeros(R, np.int32)
    for s, (ids, grads) in enumerate(batches):
        path.step(ids, grads)
        ok, _, oc = oracle.coo_from_lookups(ids, np.zeros(ids.size, np.float32), R)
        touch_count[ok] += 1
        torch.cuda.synchronize()
        u = int(host(path.U)[0])
        assert u == ok.size, f"step {s}: U {u} vs {ok.size}"
        assert np.array_equal(host(path.keys)[:u], ok), f"step {s}: keys"
        assert np.array_equal(host(path.counts)[:u], oc), f"step {s}: counts"
        if s in check_ro:
            ro, _, _ = oracle.csr_from_coo(ok, np.zeros((ok.size, C), np.float32), R, C, R, C)
            assert np.array_equal(host(path.row_offsets), ro), f"step {s}: row_offsets"
            assert np.array_equal(host(path.col_indices)[:u * C],
                                  np.tile(np.arange(C, dtype=np.int32), u)), f"step {s}: cols"
    log(f"cfg{cfg}: GPU path done, keys/counts/row_offsets/col_indices bit-exact")

    rng = np.random.default_rng(cfg)
    touched_rows = np.nonzero(touch_count)[0]
    once = np.nonzero(touch_count == 1)[0]
    sample = np.unique(np.concatenate([
        np.arange(64),                                              # the hottest rows
        rng.choice(touched_rows, size=min(512, touched_rows.size), replace=False),
        rng.choice(once, size=min(128, once.size), replace=False)]))
    ora = oracle.Adam(p0[sample].copy(), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"],
                      eps=h["eps"], mode=w.mode)
    for ids, grads in batches:
        mask = np.isin(ids, sample)
        keys, sums, _ = oracle.coo_from_lookups(ids[mask], grads[mask], R)
        ora.step_coo(np.searchsorted(sample, keys), sums, width=C)
    idx = torch.from_numpy(sample).to("cuda")
    assert np.array_equal(host(gpu.last_step.index_select(0, idx)), ora.ls)
    assert_state_close(host(gpu.params.index_select(0, idx)), ora.p, f"cfg{cfg} params")
    assert_state_close(host(gpu.m.index_select(0, idx)), ora.m, f"cfg{cfg} m")
    assert_state_close(host(gpu.v.index_select(0, idx)), ora.v, f"cfg{cfg} v")

    n_never = _check_never_touched(gpu, p0, touch_count == 0)
    log(f"cfg{cfg}: {sample.size} sampled rows within tolerance; all {n_never} never-touched "
        f"rows bit-identical to the initial table, m = v = last_step = 0")


def _check_never_touched(gpu, p0, never, chunk=1 << 20):
    """Every row outside the union of the touched rows, over the whole table, in
    chunks on the device: params bit-identical to the initial table, m, v and
    last_step all-zero bits.  Returns the number of such rows."""
    for r0 in range(0, p0.shape[0], chunk):
        r1 = min(r0 + chunk, p0.shape[0])
        quiet = torch.from_numpy(never[r0:r1]).to("cuda")
        init = torch.from_numpy(p0[r0:r1]).to("cuda")
        diff = (gpu.params[r0:r1].view(torch.int32) != init.view(torch.int32)).any(dim=1)
        for x in (gpu.m, gpu.v, gpu.last_step):
            diff |= (x[r0:r1].view(torch.int32) != 0).any(dim=1)
        bad = torch.nonzero(diff & quiet).flatten()
        assert bad.numel() == 0, f"never-touched rows changed, first {r0 + int(bad[0])}"
    return int(never.sum())


@pytest.mark.parametrize("mode", ["one_call", "two_calls"])
def test_table_10M_x_128_dormancy_sampled(mode):
    _sampled_lookup_run(3, mode)


def test_table_50M_x_128_dormancy_sampled():
    _sampled_lookup_run(5)
