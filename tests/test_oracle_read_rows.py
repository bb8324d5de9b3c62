"""Pins of the oracle's forward gather (read_rows).

Page: DiskSparseAdam README, API reference, read_rows(indices): the current rows
for the indices, indices validated, corrupted rows refused.  The plain
definition is numpy's fancy indexing (take along axis 0).
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("rows,cols,n", [(1000, 128, 3000), (50, 3, 7), (10, 1, 10), (5, 64, 0)])
def test_equals_numpy_take(rows, cols, n):
    rng = np.random.default_rng(rows + n)
    p = rng.standard_normal((rows, cols)).astype(np.float32)
    idx = rng.integers(0, rows, size=n)
    if n:
        idx[0] = rows - 1                      # last row and duplicates included
        idx[-1] = idx[0]
    out = oracle.read_rows(p, idx)
    assert out.shape == (n, cols)
    assert out.tobytes() == np.take(p, idx, axis=0).tobytes()


@pytest.mark.parametrize("bad", [-1, 50])
def test_out_of_range_is_refused(bad):
    p = np.ones((50, 4), np.float32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.read_rows(p, [0, bad, 3])
    assert e.value.code == oracle.ERANGE


def test_corrupted_row_is_refused_only_when_checked():
    p = np.ones((8, 4), np.float32)
    p[5, 2] = np.nan
    with pytest.raises(oracle.OracleError) as e:
        oracle.read_rows(p, [1, 5], check_finite=True)
    assert e.value.code == oracle.ENONFINITE
    out = oracle.read_rows(p, [1, 5])
    assert np.isnan(out[1, 2]) and (out[0] == 1).all()
    assert oracle.read_rows(p, [1, 2], check_finite=True).shape == (2, 4)
