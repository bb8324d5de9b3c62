"""GPU parity of csr_from_lookups: raw lookups -> full-row CSR in one call.

Pages: DiskSparseAdam README, "Safe Duplicate Aggregation & Sorted I/O"
(duplicates summed, ids sorted); optirs_gpu sparse_optimizer, "Sparse gradient
representations" (CsrGradient::from_coo: row_offsets[r] = cols * #ids below r,
columns 0..cols-1 per full row).  Checked against the oracle's
coo_from_lookups + csr_from_coo (integers bit for bit, sums within the float32
summation bound) and bit for bit against the library's own two calls.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
from tests.gpu_util import assert_sums_close, dev, host

pytestmark = pytest.mark.gpu


def _ids(rows, n, pattern, rng):
    if pattern == "uniform":
        return rng.integers(0, rows, size=n, dtype=np.int64)
    if pattern == "hot":          # one id takes 60%: a segment over many 256-lookup tiles
        ids = rng.integers(0, rows, size=n, dtype=np.int64)
        ids[rng.random(n) < 0.6] = rows // 3
        return ids
    if pattern == "all":          # every row touched
        ids = rng.integers(0, rows, size=n, dtype=np.int64)
        ids[:rows] = np.arange(rows)
        return rng.permutation(ids)
    if pattern == "last_rows":    # ids only in the last 50 rows: long gap before the first
        return rng.integers(rows - 50, rows, size=n, dtype=np.int64)
    if pattern == "first_rows":   # ids only in the first 50 rows: long gap after the last
        return rng.integers(0, 50, size=n, dtype=np.int64)
    raise ValueError(pattern)


def _check(rows, cols, ids, vals, ro_shift=0, want_cols=True):
    n = ids.size
    ro_buf = torch.full((rows + 1 + ro_shift,), -7, dtype=torch.int32, device="cuda")
    csr, counts, U = L.csr_from_lookups(dev(ids), dev(vals), rows,
                                        row_offsets=ro_buf[ro_shift:],
                                        want_col_indices=want_cols)
    torch.cuda.synchronize()
    u = int(host(U)[0])
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, rows)
    ro, ci, cv = oracle.csr_from_coo(ok, ov, rows, cols, rows, cols)
    assert u == ok.size
    assert np.array_equal(host(csr.row_offsets), ro)
    assert (host(ro_buf)[:ro_shift] == -7).all()
    assert np.array_equal(host(csr.touched_rows)[:u], ok)
    assert np.array_equal(host(counts)[:u], oc)
    if want_cols:
        assert np.array_equal(host(csr.col_indices)[:u * cols], ci)
    else:
        assert csr.col_indices is None
    got = host(csr.values).reshape(-1, cols)[:u]
    assert_sums_close(got, ov.reshape(-1, cols), ids, ok, oc, vals)
    # the library's two calls give the same bits
    keys2, sums2, counts2, U2 = L.coo_from_lookups(dev(ids), dev(vals), rows)
    coo = L.CooGradient(keys2, sums2, dim=rows, width=cols, nnz=n, d_nnz=U2)
    csr2 = L.csr_from_coo(coo, rows, cols, copy_values=False)
    torch.cuda.synchronize()
    assert host(csr2.row_offsets).tobytes() == host(csr.row_offsets).tobytes()
    assert host(sums2)[:u].tobytes() == host(csr.values)[:u].tobytes()
    assert host(counts2)[:u].tobytes() == host(counts)[:u].tobytes()


@pytest.mark.parametrize("rows,cols,n,pattern,ro_shift", [
    (50000, 128, 20000, "uniform", 0),
    (50000, 128, 20000, "hot", 0),
    (8191, 8, 4000, "uniform", 0),            # row_offsets exactly one 8192-row block
    (8192, 8, 4000, "uniform", 0),            # a second block of one entry
    (16384, 4, 200000, "all", 0),             # every row touched
    (24577, 4, 9000, "hot", 3),               # row_offsets not 16-byte aligned
    (2_000_000, 4, 500, "last_rows", 0),      # the first id's gap spans 244 blocks
    (2_000_000, 4, 500, "first_rows", 0),     # the last id's gap spans 244 blocks
    (1000, 6, 3000, "hot", 0),                # columns not in groups of 4: the two calls
    (1000, 3, 3000, "uniform", 1),
    (10, 4, 1, "uniform", 0),
])
def test_matches_oracle_and_two_calls(rows, cols, n, pattern, ro_shift):
    rng = np.random.default_rng(rows + n)
    ids = _ids(rows, n, pattern, rng)
    vals = rng.standard_normal((n, cols)).astype(np.float32)
    _check(rows, cols, ids, vals, ro_shift)


def test_many_row_blocks_repeatedly():
    """Regression test: 50M rows make 6104 row_offsets blocks a call; every call
    over 25 steps of Zipf lookups must give exactly the offsets of csr_from_coo
    (a missing barrier between zeroing a block's LDS flags and setting them once
    dropped a key from a block now and then)."""
    import synth
    w = synth.WORKLOADS[5].scaled(cols=4)
    R, C, n = w.rows, w.cols, w.n_lookups
    ws = torch.empty(L.sparse_opt_workspace_size(n, C, R), dtype=torch.uint8, device="cuda")
    ro1 = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    ro2 = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    for s in range(25):
        ids, grads = synth.lookups(w, s)
        csr, _, U = L.csr_from_lookups(dev(ids), dev(grads), R, row_offsets=ro1,
                                       want_col_indices=False, workspace=ws)
        coo = L.CooGradient(csr.touched_rows, csr.values, dim=R, width=C, nnz=n, d_nnz=U)
        L.csr_from_coo(coo, R, C, row_offsets=ro2, want_col_indices=False, copy_values=False)
        torch.cuda.synchronize()
        assert torch.equal(ro1, ro2), f"step {s}"


def test_without_col_indices():
    rng = np.random.default_rng(5)
    ids = _ids(30000, 5000, "hot", rng)
    _check(30000, 64, ids, rng.standard_normal((5000, 64)).astype(np.float32), want_cols=False)


def test_empty_lookups():
    rows, cols = 9000, 8
    ro = torch.full((rows + 1,), -7, dtype=torch.int32, device="cuda")
    csr, counts, U = L.csr_from_lookups(torch.zeros(0, dtype=torch.int64, device="cuda"),
                                        torch.zeros((0, cols), device="cuda"), rows,
                                        row_offsets=ro)
    torch.cuda.synchronize()
    assert int(host(U)[0]) == 0
    assert not host(ro).any()


def test_workspace_reused_across_calls():
    """The per-block counts are rewritten in full by every call."""
    rows, cols = 100_000, 16
    rng = np.random.default_rng(9)
    ws = torch.empty(L.sparse_opt_workspace_size(6000, cols, rows), dtype=torch.uint8,
                     device="cuda")
    for n, pattern in [(6000, "first_rows"), (4000, "last_rows"), (3000, "uniform")]:
        ids = _ids(rows, n, pattern, rng)
        vals = rng.standard_normal((n, cols)).astype(np.float32)
        csr, counts, U = L.csr_from_lookups(dev(ids), dev(vals), rows, workspace=ws)
        torch.cuda.synchronize()
        ok, ov, oc = oracle.coo_from_lookups(ids, vals, rows)
        ro, _, _ = oracle.csr_from_coo(ok, ov, rows, cols, rows, cols)
        assert np.array_equal(host(csr.row_offsets), ro), pattern


def test_trusted_out_of_range_gives_empty_csr():
    rows, cols = 20000, 8
    ids = np.array([5, rows, 7, 19999], np.int64)
    ro = torch.full((rows + 1,), -7, dtype=torch.int32, device="cuda")
    csr, counts, U = L.csr_from_lookups(dev(ids), dev(np.ones((4, cols), np.float32)), rows,
                                        row_offsets=ro)
    torch.cuda.synchronize()
    assert int(host(U)[0]) == 0
    assert not host(ro).any()


def test_validate_errors():
    rows, cols = 500, 4
    vals = np.ones((3, cols), np.float32)
    with pytest.raises(L.SparseOptError) as e:
        L.csr_from_lookups(dev(np.array([0, 500, 2], np.int64)), dev(vals), rows, validate=True)
    assert e.value.code == oracle.ERANGE
    bad = vals.copy()
    bad[2, 1] = np.nan
    with pytest.raises(L.SparseOptError) as e:
        L.csr_from_lookups(dev(np.array([0, 1, 2], np.int64)), dev(bad), rows, validate=True)
    assert e.value.code == oracle.ENONFINITE


def test_step_on_the_fused_gradient():
    """Adam DormancyDecay over a few steps from csr_from_lookups equals the
    oracle's step on its own CSR."""
    import synth
    w = synth.WORKLOADS[3].scaled(rows=60000, n_lookups=5000, steps=6)
    p0 = synth.init_params(w)
    h = w.hyper
    kw = dict(lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"], mode="dormancy")
    ora = oracle.Adam(p0.copy(), **kw)
    gpu = L.SparseAdam(dev(p0), **kw)
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        csr, _, _ = L.csr_from_lookups(dev(ids), dev(grads), w.rows, want_col_indices=False)
        gpu.step(csr)
    torch.cuda.synchronize()
    from tests.gpu_util import assert_state_close
    assert_state_close(host(gpu.params), ora.p, "params")
    assert_state_close(host(gpu.m), ora.m, "m")
    assert_state_close(host(gpu.v), ora.v, "v")
    assert np.array_equal(host(gpu.last_step), ora.ls)
