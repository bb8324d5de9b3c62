"""Pins of the oracle's canonicalisation and COO <-> CSR conversions.

Pages: docs.rs optirs_gpu sparse_optimizer, section "Sparse gradient
representations" (canonical COO: strictly ascending indices; CSR: strictly
ascending columns in each row; lossless CSR <-> COO via row*c + col);
DiskSparseAdam README, "Safe Duplicate Aggregation & Sorted I/O" and the
step() method (duplicates summed, indices in [0, N), finite gradients).
"""
import math

import numpy as np
import pytest
import scipy.sparse as sp

import oracle

U32 = 2.0 ** -24    # float32 unit roundoff


def _lookups(rng, n, key_space, width, hot=0.0):
    ids = rng.integers(0, key_space, size=n)
    if hot and n:
        ids[rng.random(n) < hot] = key_space - 1
    vals = rng.standard_normal((n, width)).astype(np.float32)
    return ids.astype(np.int64), vals


@pytest.mark.parametrize("n,key_space,width,hot", [
    (0, 10, 1, 0.0), (1, 1, 1, 0.0), (1, 7, 3, 0.0), (200, 5, 1, 0.0), (500, 100000, 4, 0.0),
    (3000, 50, 16, 0.5), (4096, 4096, 2, 0.0), (1000, 1, 8, 0.0)])
def test_keys_counts_match_numpy_unique(n, key_space, width, hot):
    rng = np.random.default_rng(n + key_space)
    ids, vals = _lookups(rng, n, key_space, width, hot)
    keys, sums, counts = oracle.coo_from_lookups(ids, vals, key_space)
    uk, uc = np.unique(ids, return_counts=True)
    assert np.array_equal(keys, uk) and np.array_equal(counts, uc)
    assert sums.shape == (uk.size, width)


@pytest.mark.parametrize("seed", range(4))
def test_duplicate_sums(seed):
    """Brute force by dict in lookup order (double, then one float rounding), and
    within half an ulp plus the recursive-summation bound of the exact sum."""
    rng = np.random.default_rng(seed)
    ids, vals = _lookups(rng, 2000, 60, 5, hot=0.3)
    keys, sums, counts = oracle.coo_from_lookups(ids, vals, 60)
    acc = {}
    for i, k in enumerate(ids):
        row = acc.setdefault(int(k), [0.0] * 5)
        for c in range(5):
            row[c] += float(vals[i, c])
    for u, k in enumerate(keys):
        assert np.array_equal(sums[u], np.array(acc[int(k)], dtype=np.float32))
        members = vals[ids == k].astype(np.float64)
        for c in range(5):
            ex = math.fsum(members[:, c])
            bound = (counts[u] - 1) * 2.0 ** -53 / (1 - counts[u] * 2.0 ** -53) * np.abs(
                members[:, c]).sum()
            assert abs(float(sums[u, c]) - ex) <= bound + (abs(ex) + bound) * U32 + 1e-300


def test_zero_sum_duplicates_stay_present():
    ids = np.array([4, 4, 2], np.int64)
    vals = np.array([[1.5], [-1.5], [0.0]], np.float32)
    keys, sums, counts = oracle.coo_from_lookups(ids, vals, 8)
    assert keys.tolist() == [2, 4] and counts.tolist() == [1, 2] and sums[:, 0].tolist() == [0, 0]


@pytest.mark.parametrize("ids,code", [([0, -1], oracle.ERANGE), ([3, 10], oracle.ERANGE)])
def test_lookup_range_errors(ids, code):
    with pytest.raises(oracle.OracleError) as e:
        oracle.coo_from_lookups(np.array(ids), np.ones((2, 1), np.float32), 10)
    assert e.value.code == code


def test_lookup_nonfinite_error():
    v = np.ones((3, 2), np.float32)
    v[1, 1] = np.nan
    oracle.coo_from_lookups(np.array([0, 1, 2]), v, 4)               # not checked by default
    with pytest.raises(oracle.OracleError) as e:
        oracle.coo_from_lookups(np.array([0, 1, 2]), v, 4, check_finite=True)
    assert e.value.code == oracle.ENONFINITE


# ---------------------------------------------------------------------------
# COO <-> CSR
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,nnz", [(1, 1, 1), (7, 5, 0), (50, 13, 200), (300, 1, 120),
                                           (20, 64, 1280)])
def test_csr_from_scalar_coo_matches_scipy(rows, cols, nnz):
    rng = np.random.default_rng(rows * cols + nnz)
    lin = np.sort(rng.choice(rows * cols, size=nnz, replace=False)).astype(np.int64)
    vals = rng.standard_normal(nnz).astype(np.float32)
    ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
    ref = sp.coo_matrix((vals, (lin // cols, lin % cols)), shape=(rows, cols)).tocsr()
    ref.sort_indices()
    assert np.array_equal(ro, ref.indptr) and np.array_equal(ci, ref.indices)
    assert np.array_equal(cv, ref.data)
    back, bv = oracle.csr_to_coo(ro, ci, cv, rows, cols)
    assert np.array_equal(back, lin) and np.array_equal(bv, vals)


@pytest.mark.parametrize("rows,cols,k", [(10, 4, 3), (1000, 16, 37), (5, 3, 5), (9, 2, 0)])
def test_csr_from_full_row_coo_matches_scipy(rows, cols, k):
    rng = np.random.default_rng(k)
    r = np.sort(rng.choice(rows, size=k, replace=False)).astype(np.int64)
    vals = rng.standard_normal((k, cols)).astype(np.float32)
    ro, ci, cv = oracle.csr_from_coo(r, vals, rows, cols, rows, cols)
    dense = np.zeros((rows, cols), np.float32)
    dense[r] = vals
    mask = np.zeros((rows, cols), bool)
    mask[r] = True
    rr, cc = np.nonzero(mask)
    ref = sp.csr_matrix((dense[rr, cc], (rr, cc)), shape=(rows, cols))
    ref.sort_indices()
    assert np.array_equal(ro, ref.indptr) and np.array_equal(ci, ref.indices)
    assert np.array_equal(cv, ref.data)


def test_csr_round_trip_from_csr_side():
    rng = np.random.default_rng(3)
    m = sp.random(40, 17, density=0.2, format="csr", random_state=3, dtype=np.float32)
    m.sort_indices()
    lin, lv = oracle.csr_to_coo(m.indptr.astype(np.int32), m.indices.astype(np.int32), m.data, 40, 17)
    ro, ci, cv = oracle.csr_from_coo(lin, lv, 40 * 17, 1, 40, 17)
    assert np.array_equal(ro, m.indptr) and np.array_equal(ci, m.indices)
    assert np.array_equal(cv, m.data)


@pytest.mark.parametrize("case,code", [("unsorted", oracle.ENOTCANON), ("dup", oracle.ENOTCANON),
                                       ("range", oracle.ERANGE), ("shape", oracle.ESHAPE)])
def test_csr_from_coo_errors(case, code):
    idx = {"unsorted": [5, 2], "dup": [2, 2], "range": [2, 40], "shape": [1, 2]}[case]
    dim = 39 if case == "shape" else 40
    with pytest.raises(oracle.OracleError) as e:
        oracle.csr_from_coo(np.array(idx), np.ones(2, np.float32), dim, 1, 10, 4)
    assert e.value.code == code


def test_csr_to_coo_rejects_non_canonical_rows():
    with pytest.raises(oracle.OracleError) as e:
        oracle.csr_to_coo(np.array([0, 2, 2], np.int32), np.array([3, 1], np.int32),
                          np.ones(2, np.float32), 2, 4)
    assert e.value.code == oracle.ENOTCANON
