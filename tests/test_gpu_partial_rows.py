"""GPU parity of the partial-row path: a flat (width-1) COO to CSR, then the
SGD or Adam step on a CSR without a touched-row list.

Page: docs.rs optirs_gpu sparse_optimizer, sections Sparse gradient
representations (CsrGradient::from_coo: row = idx / cols, col = idx % cols,
row_offsets over every row) and Sparse SGD / LazyAdamMode::DormancyDecay (the
update of the touched coordinates only).  row_offsets and col_indices must be
bit-exact against the oracle; state within 1e-5 relative + 1e-7 absolute,
last_step and untouched coordinates bit-exact.

The CSR build writes the first offset of every 4096-row block from the entry
that crosses into it, then fills each block from its two bounds; the update
scans row_offsets 64 rows per wave, one lane per entry.  The shapes below put
block and wave edges where they can go wrong.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu


def _entries(rng, rows, cols, pattern):
    if pattern == "uniform":
        lin = rng.choice(rows * cols, size=min(rows * cols, 3 * rows), replace=False)
    elif pattern == "one_row":
        r = rows // 2
        lin = r * cols + rng.choice(cols, size=max(1, cols // 2), replace=False)
    elif pattern == "last_row":
        lin = (rows - 1) * cols + np.arange(cols)
    elif pattern == "first_row":
        lin = rng.choice(cols, size=max(1, cols // 3), replace=False)
    elif pattern == "gaps":  # touched rows far apart: several row blocks between them
        rs = np.array([0, 4095, 4096, 9000, 20479, 20480, rows - 1])
        rs = np.unique(rs[rs < rows])
        lin = (rs[:, None] * cols + np.arange(min(cols, 5))[None, :]).reshape(-1)
    elif pattern == "dense":  # whole runs of full rows: waves with many rounds of entries
        lin = np.arange(min(rows, 700) * cols)
    else:
        raise ValueError(pattern)
    return np.unique(lin).astype(np.int64)


@pytest.mark.parametrize("rows,cols", [(4096, 8), (4095, 8), (4097, 8), (12289, 3), (50000, 64),
                                       (1, 16), (257, 256)])
@pytest.mark.parametrize("pattern", ["uniform", "one_row", "last_row", "first_row", "gaps",
                                     "dense"])
def test_csr_from_flat_coo_edges(rows, cols, pattern):
    rng = np.random.default_rng(rows * 7 + cols)
    lin = _entries(rng, rows, cols, pattern)
    vals = rng.standard_normal(lin.size).astype(np.float32)
    ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
    # row_offsets full of stale values from an earlier, different gradient
    ro_buf = torch.full((rows + 1,), 123456, dtype=torch.int32, device="cuda")
    # a device-side count below the arrays' length (nnz is then an upper bound)
    pad = 37
    idx_d = dev(np.r_[lin, np.full(pad, rows * cols - 1, np.int64)])
    val_d = dev(np.r_[vals, np.zeros(pad, np.float32)])
    n_d = dev(np.array([lin.size], np.int64))
    coo = L.CooGradient(idx_d, val_d, dim=rows * cols, width=1, nnz=lin.size + pad, d_nnz=n_d)
    csr = L.csr_from_coo(coo, rows, cols, row_offsets=ro_buf)
    torch.cuda.synchronize()
    assert np.array_equal(host(csr.row_offsets), ro)
    assert np.array_equal(host(csr.col_indices)[:lin.size], ci)
    assert np.array_equal(host(csr.values)[:lin.size], cv)


def test_csr_from_empty_flat_coo_clears_stale_offsets():
    rows, cols = 20000, 4
    ro_buf = torch.full((rows + 1,), 99, dtype=torch.int32, device="cuda")
    coo = L.CooGradient(torch.zeros(1, dtype=torch.int64, device="cuda"),
                        torch.zeros(1, device="cuda"), dim=rows * cols, width=1, nnz=0)
    csr = L.csr_from_coo(coo, rows, cols, row_offsets=ro_buf)
    torch.cuda.synchronize()
    assert not host(csr.row_offsets).any()


def _pair(kind, p0, mode="dormancy"):
    if kind == "sgd":
        kw = dict(lr=0.05, momentum=0.9, weight_decay=1e-4)
        return oracle.Sgd(p0.copy(), **kw), L.SparseSgd(dev(p0), **kw)
    return (oracle.Adam(p0.copy(), mode=mode), L.SparseAdam(dev(p0), mode=mode))


@pytest.mark.parametrize("kind,mode", [("sgd", None), ("adam", "dormancy"), ("adam", "lazy")])
@pytest.mark.parametrize("rows,cols", [(3001, 256), (513, 8), (700, 3)])
def test_flat_update_matches_oracle(kind, mode, rows, cols):
    """Several steps of mixed patterns (dense runs, gaps, single rows, empty
    gradients) through csr_from_coo and the step; the whole table compared."""
    rng = np.random.default_rng(rows + cols)
    p0 = (rng.standard_normal((rows, cols)) * 0.01).astype(np.float32)
    ora, gpu = _pair(kind, p0, mode or "dormancy")
    touched = np.zeros(rows * cols, bool)
    patterns = ["uniform", "dense", "gaps", "empty", "one_row", "uniform", "last_row", "uniform"]
    for s, pattern in enumerate(patterns):
        lin = np.zeros(0, np.int64) if pattern == "empty" else _entries(rng, rows, cols, pattern)
        vals = rng.standard_normal(lin.size).astype(np.float32)
        touched[lin] = True
        ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
        ora.step_csr(ro, ci, cv)
        if lin.size:
            coo = L.CooGradient(dev(lin), dev(vals), dim=rows * cols, width=1)
        else:
            coo = L.CooGradient(torch.zeros(1, dtype=torch.int64, device="cuda"),
                                torch.zeros(1, device="cuda"), dim=rows * cols, width=1, nnz=0)
        gpu.step(L.csr_from_coo(coo, rows, cols))
    torch.cuda.synchronize()
    gp = host(gpu.params)
    assert_state_close(gp, ora.p, f"{kind} params")
    assert gp.reshape(-1)[~touched].tobytes() == p0.reshape(-1)[~touched].tobytes()
    if kind == "sgd":
        assert_state_close(host(gpu.momentum_buf), ora.b, "sgd momentum")
    else:
        assert np.array_equal(host(gpu.last_step), ora.ls)
        assert_state_close(host(gpu.m), ora.m, "adam m")
        assert_state_close(host(gpu.v), ora.v, "adam v")


def test_flat_update_full_rows_without_columns():
    """A CSR of full rows with no col_indices (columns implicit), no touched-row
    list: the flat kernel takes each entry's column from its place in the row."""
    rng = np.random.default_rng(5)
    rows, cols = 2000, 12
    p0 = (rng.standard_normal((rows, cols)) * 0.01).astype(np.float32)
    ora, gpu = _pair("adam", p0)
    for _ in range(4):
        keys = np.unique(rng.integers(0, rows, size=600)).astype(np.int64)
        sums = rng.standard_normal((keys.size, cols)).astype(np.float32)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, rows, cols, rows, cols)
        ora.step_csr(ro, ci, cv)
        gpu.step(L.CsrGradient(dev(ro), None, dev(cv), rows, cols))
    torch.cuda.synchronize()
    assert np.array_equal(host(gpu.last_step), ora.ls)
    assert_state_close(host(gpu.params), ora.p, "params")
    assert_state_close(host(gpu.m), ora.m, "m")
    assert_state_close(host(gpu.v), ora.v, "v")


@pytest.mark.parametrize("pattern", ["gaps", "last_row", "first_row", "one_row"])
def test_csr_from_flat_coo_indices_beyond_32_bits(pattern):
    """A 40M x 128 view: linear indices up to 5.1e9, so row and column come
    from 64-bit division by the column count."""
    rows, cols = 40_000_001, 128
    rng = np.random.default_rng(11)
    lin = _entries(rng, rows, cols, pattern)
    lin = np.unique(np.r_[lin, (rows - 3) * cols + 5, 2**32 + 7]).astype(np.int64)
    vals = rng.standard_normal(lin.size).astype(np.float32)
    ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
    csr = L.csr_from_coo(L.CooGradient(dev(lin), dev(vals), dim=rows * cols, width=1), rows, cols)
    torch.cuda.synchronize()
    assert np.array_equal(host(csr.row_offsets), ro)
    assert np.array_equal(host(csr.col_indices)[:lin.size], ci)
