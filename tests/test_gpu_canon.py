"""GPU parity of canonicalisation and COO <-> CSR against the oracle.

Integer outputs (distinct keys, U, multiplicities, row_offsets, col_indices,
linear indices) must match bit for bit; duplicate sums within the float32
summation bound (the order of a float32 sum is not fixed by the pages).
Pages: optirs_gpu sparse_optimizer, "Sparse gradient representations";
DiskSparseAdam README, "Safe Duplicate Aggregation & Sorted I/O".
"""
import zlib

import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
from tests.gpu_util import assert_sums_close, dev, host

pytestmark = pytest.mark.gpu


def _run(ids, vals, key_space, validate=False):
    n = len(ids)
    keys, sums, counts, U = L.coo_from_lookups(dev(ids), dev(vals.reshape(n, -1) if n else vals),
                                               key_space, validate=validate)
    torch.cuda.synchronize()
    u = int(host(U)[0])
    return host(keys)[:u], host(sums)[:u], host(counts)[:u], u


CASES = [
    # (name, n, key_space, width, hot_fraction)
    ("single", 1, 10, 4, 0.0),
    ("key_space_1", 300, 1, 3, 0.0),
    ("two_passes", 5000, 200, 1, 0.0),
    ("ragged_width3", 3333, 70000, 3, 0.0),
    ("width64_zipfish", 8192, 1_000_000, 64, 0.2),
    ("width128_heavy", 20000, 10_000_000, 128, 0.6),
    ("width256", 4100, 2_000_000, 256, 0.1),
    ("width1_heavy", 70000, 5000, 1, 0.7),
    ("four_passes", 2048, 1 << 30, 2, 0.0),
    ("33bit_keys", 1500, 6_400_000_000, 1, 0.3),
    ("all_distinct", 4096, 4096, 8, 0.0),
    ("sort_tile_plus_one", 2049, 300, 2, 0.5),
    # every row-sum layout: 4-, 2- and 1-float lanes over 16-, 32- and 64-lane
    # groups, and rows wider than one group's columns
    ("width17", 3000, 5000, 17, 0.3),
    ("width50", 3000, 5000, 50, 0.3),
    ("width67", 2500, 3000, 67, 0.3),
    ("width130", 2500, 3000, 130, 0.3),
    ("width384", 1500, 100000, 384, 0.5),
]


@pytest.mark.parametrize("name,n,key_space,width,hot", CASES, ids=[c[0] for c in CASES])
def test_coo_from_lookups_matches_oracle(name, n, key_space, width, hot):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    ids = rng.integers(0, key_space, size=n, dtype=np.int64)
    if hot:
        ids[rng.random(n) < hot] = key_space - 1      # one long segment at the last key
    vals = rng.standard_normal((n, width)).astype(np.float32)
    gk, gv, gc, u = _run(ids, vals, key_space)
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, key_space)
    assert u == ok.size
    assert np.array_equal(gk, ok) and np.array_equal(gc, oc)
    assert_sums_close(gv, ov, ids, ok, oc, vals)


@pytest.mark.parametrize("run", [1, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1100])
def test_runs_on_chunk_edges(run):
    """Runs of equal ids of fixed length, so segment ends fall on every offset of
    the 16-lookup waves and 256-lookup tiles of the summing kernel (exactly on
    their edges for 16, 32, 64 and 512), and segments cross several tiles."""
    rng = np.random.default_rng(run)
    n_ids, width = max(24, 30000 // run), 128
    ids = np.repeat(rng.permutation(100000)[:n_ids].astype(np.int64), run)
    ids = ids[rng.permutation(ids.size)]
    vals = rng.standard_normal((ids.size, width)).astype(np.float32)
    gk, gv, gc, u = _run(ids, vals, 100000)
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, 100000)
    assert u == ok.size == n_ids and (oc == run).all()
    assert np.array_equal(gk, ok) and np.array_equal(gc, oc)
    assert_sums_close(gv, ov, ids, ok, oc, vals)


def test_unaligned_values():
    """Value rows that are only 4-byte aligned take the one-float path."""
    rng = np.random.default_rng(5)
    n, width, ks = 5000, 128, 3000
    ids = rng.integers(0, ks, size=n, dtype=np.int64)
    vals = rng.standard_normal((n, width)).astype(np.float32)
    buf = torch.zeros(n * width + 1, dtype=torch.float32, device="cuda")
    buf[1:] = torch.from_numpy(vals.reshape(-1)).to("cuda")
    out = torch.zeros(n * width + 1, dtype=torch.float32, device="cuda")
    keys, sums, counts, U = L.coo_from_lookups(dev(ids), buf[1:].view(n, width), ks,
                                               out_vals=out[1:].view(n, width))
    torch.cuda.synchronize()
    u = int(host(U)[0])
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, ks)
    assert u == ok.size
    assert np.array_equal(host(keys)[:u], ok) and np.array_equal(host(counts)[:u], oc)
    assert_sums_close(host(sums)[:u], ov, ids, ok, oc, vals)


def test_empty_lookups():
    keys, sums, counts, U = L.coo_from_lookups(dev(np.zeros(0, np.int64)),
                                               dev(np.zeros((0, 4), np.float32)), 10)
    torch.cuda.synchronize()
    assert int(host(U)[0]) == 0


def test_deterministic_run_to_run():
    rng = np.random.default_rng(1)
    ids = np.minimum(rng.zipf(1.3, size=30000) - 1, 99999).astype(np.int64)
    vals = rng.standard_normal((30000, 128)).astype(np.float32)
    a = _run(ids, vals, 100000)
    b = _run(ids, vals, 100000)
    for x, y in zip(a[:3], b[:3]):
        assert x.tobytes() == y.tobytes()


def test_zero_sum_duplicates_stay_present():
    ids = np.array([4, 4, 2], np.int64)
    vals = np.array([[1.5], [-1.5], [0.0]], np.float32)
    gk, gv, gc, u = _run(ids, vals, 8)
    assert gk.tolist() == [2, 4] and gc.tolist() == [1, 2] and gv.reshape(-1).tolist() == [0, 0]


def test_validate_range_and_nonfinite():
    vals = np.ones((3, 2), np.float32)
    with pytest.raises(L.SparseOptError) as e:
        _run(np.array([0, 7, 2], np.int64), vals, 5, validate=True)
    assert e.value.code == oracle.ERANGE
    with pytest.raises(L.SparseOptError) as e:
        _run(np.array([0, -1, 2], np.int64), vals, 5, validate=True)
    assert e.value.code == oracle.ERANGE
    bad = vals.copy()
    bad[1, 1] = np.inf
    with pytest.raises(L.SparseOptError) as e:
        _run(np.array([0, 1, 2], np.int64), bad, 5, validate=True)
    assert e.value.code == oracle.ENONFINITE


def test_trusted_out_of_range_gives_empty_result():
    gk, gv, gc, u = _run(np.array([0, 9, 2], np.int64), np.ones((3, 2), np.float32), 5)
    assert u == 0
    # one key only: no radix pass runs
    gk, gv, gc, u = _run(np.array([0, 3, 0], np.int64), np.ones((3, 2), np.float32), 1)
    assert u == 0


@pytest.mark.parametrize("validate", [False, True])
def test_out_of_range_in_a_later_pack_chunk(validate):
    """70,000 lookups: more 2048-lookup chunks than pack blocks, so block 0
    also packs chunk 32, which holds the bad id."""
    n = 70000
    ids = np.arange(n, dtype=np.int64) % 1000
    ids[66000] = 1000
    vals = np.ones((n, 1), np.float32)
    if validate:
        with pytest.raises(L.SparseOptError) as e:
            _run(ids, vals, 1000, validate=True)
        assert e.value.code == oracle.ERANGE
    else:
        assert _run(ids, vals, 1000)[3] == 0


@pytest.mark.parametrize("n,key_space,pattern", [
    (8192, 1_000_000, "one_id"), (8192, 1_000_000, "random"), (8191, 2, "random"),
    (8193, 1_000_000, "random"), (8192, 1 << 40, "random"), (257, 5000, "sorted_desc"),
    (4096, 3, "random")])
def test_lookup_counts_around_four_radix_tiles(n, key_space, pattern):
    """Lookup counts at and around four 2048-lookup radix tiles (one id only,
    1-bit and 40-bit keys, ids in descending order): the oracle's keys and
    counts bit for bit."""
    rng = np.random.default_rng(n + key_space % 97)
    if pattern == "one_id":
        ids = np.full(n, key_space // 3, np.int64)
    elif pattern == "sorted_desc":
        ids = np.sort(rng.integers(0, key_space, size=n, dtype=np.int64))[::-1].copy()
    else:
        ids = rng.integers(0, key_space, size=n, dtype=np.int64)
    vals = rng.standard_normal((n, 8)).astype(np.float32)
    gk, gv, gc, u = _run(ids, vals, key_space)
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, key_space)
    assert u == ok.size
    assert np.array_equal(gk, ok) and np.array_equal(gc, oc)
    assert_sums_close(gv, ov, ids, ok, oc, vals)


@pytest.mark.parametrize("validate", [False, True])
@pytest.mark.parametrize("where", [0, 4095, 8191])
def test_out_of_range_within_8192_lookups(validate, where):
    n = 8192
    ids = np.arange(n, dtype=np.int64) % 700
    ids[where] = -5 if where == 4095 else 700
    vals = np.ones((n, 2), np.float32)
    if validate:
        with pytest.raises(L.SparseOptError) as e:
            _run(ids, vals, 700, validate=True)
        assert e.value.code == oracle.ERANGE
    else:
        assert _run(ids, vals, 700)[3] == 0
    # the next call on fresh inputs is unaffected
    ids[where] = 3
    gk, gv, gc, u = _run(ids, vals, 700)
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, 700)
    assert u == ok.size and np.array_equal(gk, ok) and np.array_equal(gc, oc)


def test_a_million_lookups():
    """A million lookups: 977 sort tiles and 3907 segment tiles, more than the
    device runs at once, and about 15 chunks of 2048 lookups per pack block."""
    rng = np.random.default_rng(11)
    n, key_space = 1_000_000, 5_000_000
    ids = rng.integers(0, key_space, size=n, dtype=np.int64)
    ids[rng.random(n) < 0.1] = 4321
    vals = rng.standard_normal((n, 1)).astype(np.float32)
    gk, gv, gc, u = _run(ids, vals, key_space)
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, key_space)
    assert u == ok.size
    assert np.array_equal(gk, ok) and np.array_equal(gc, oc)
    assert_sums_close(gv, ov, ids, ok, oc, vals)


def test_workspace_too_small():
    ids = dev(np.arange(100, dtype=np.int64))
    vals = dev(np.ones((100, 4), np.float32))
    with pytest.raises(L.SparseOptError) as e:
        L.coo_from_lookups(ids, vals, 100, workspace=torch.empty(16, dtype=torch.uint8,
                                                                   device="cuda"))
    assert e.value.code == oracle.EWORKSPACE


# ---------------------------------------------------------------------------
# COO <-> CSR
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,n,ro_shift", [
    (1000, 64, 3000, 0), (50000, 128, 20000, 0), (7, 4, 30, 0), (9000, 3, 500, 0),
    # row_offsets blocks of 8192 entries: a full last block, a one-entry last
    # block, and a row_offsets array that is not 16-byte aligned (scalar stores)
    (8191, 8, 4000, 0), (8192, 8, 4000, 0), (50000, 128, 20000, 1), (24577, 4, 9000, 3),
    # every row touched: blocks holding 8192 keys each; 200,000 entries make
    # the search over the keys take three rounds
    (16384, 4, 200000, 0)])
def test_csr_from_full_row_coo(rows, cols, n, ro_shift):
    rng = np.random.default_rng(rows)
    ids = rng.integers(0, rows, size=n, dtype=np.int64)
    ids[:5] = rows - 1
    vals = rng.standard_normal((n, cols)).astype(np.float32)
    keys, sums, counts, U = L.coo_from_lookups(dev(ids), dev(vals), rows)
    coo = L.CooGradient(keys, sums, dim=rows, width=cols, nnz=n, d_nnz=U)
    ro_buf = torch.full((rows + 1 + ro_shift,), -7, dtype=torch.int32, device="cuda")
    csr = L.csr_from_coo(coo, rows, cols, row_offsets=ro_buf[ro_shift:])
    torch.cuda.synchronize()
    u = int(host(U)[0])
    ok, ov, oc = oracle.coo_from_lookups(ids, vals, rows)
    ro, ci, cv = oracle.csr_from_coo(ok, ov, rows, cols, rows, cols)
    assert np.array_equal(host(csr.row_offsets), ro)
    assert (host(ro_buf)[:ro_shift] == -7).all()
    assert np.array_equal(host(csr.col_indices)[:u * cols], ci)
    assert np.array_equal(host(csr.touched_rows)[:u], ok)
    assert np.array_equal(host(csr.values)[:u * cols], host(sums)[:u].reshape(-1))


@pytest.mark.parametrize("rows,cols,nnz", [(2000, 256, 40000), (300, 7, 900), (5000, 1, 1200),
                                           (1, 16, 16), (64, 8, 0)])
def test_csr_from_scalar_coo_and_back(rows, cols, nnz):
    rng = np.random.default_rng(nnz + rows)
    lin = np.sort(rng.choice(rows * cols, size=nnz, replace=False)).astype(np.int64)
    vals = rng.standard_normal(nnz).astype(np.float32)
    coo = L.CooGradient(dev(lin) if nnz else torch.zeros(1, dtype=torch.int64, device="cuda"),
                        dev(vals) if nnz else torch.zeros(1, device="cuda"), dim=rows * cols,
                        width=1, nnz=nnz)
    csr = L.csr_from_coo(coo, rows, cols)
    torch.cuda.synchronize()
    ro, ci, cv = oracle.csr_from_coo(lin, vals, rows * cols, 1, rows, cols)
    assert np.array_equal(host(csr.row_offsets), ro)
    assert np.array_equal(host(csr.col_indices)[:nnz], ci)
    assert np.array_equal(host(csr.values)[:nnz], cv)
    back = L.csr_to_coo(csr)
    torch.cuda.synchronize()
    assert np.array_equal(host(back.indices)[:nnz], lin)
    assert np.array_equal(host(back.values)[:nnz], vals)


def test_csr_validate_errors():
    lin = dev(np.array([5, 2], np.int64))
    v = dev(np.ones(2, np.float32))
    with pytest.raises(L.SparseOptError) as e:
        L.csr_from_coo(L.CooGradient(lin, v, dim=40, width=1), 10, 4, validate=True)
    assert e.value.code == oracle.ENOTCANON
    with pytest.raises(L.SparseOptError) as e:
        L.csr_from_coo(L.CooGradient(lin, v, dim=39, width=1), 10, 4)
    assert e.value.code == oracle.ESHAPE
    bad = L.CsrGradient(dev(np.array([0, 2, 2], np.int32)), dev(np.array([3, 1], np.int32)),
                        v, rows=2, cols=4)
    with pytest.raises(L.SparseOptError) as e:
        L.csr_to_coo(bad, validate=True)
    assert e.value.code == oracle.ENOTCANON
