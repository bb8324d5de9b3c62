"""GPU parity of the forward gather (read_rows) against the oracle.

Page: DiskSparseAdam README, API reference, read_rows(indices).  Bit-exact: the
gather moves float32 values unchanged.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,n", [(5000, 128, 4099), (3000, 64, 1000), (800, 3, 333),
                                         (600, 6, 77), (400, 384, 50), (1000, 1, 17),
                                         (50, 130, 16)])
def test_read_rows_matches_oracle(rows, cols, n):
    rng = np.random.default_rng(rows + cols)
    p = rng.standard_normal((rows, cols)).astype(np.float32)
    idx = rng.integers(0, rows, size=n)
    idx[0] = rows - 1
    idx[-1] = idx[0]                         # a duplicate
    out = L.read_rows(dev(p), dev(idx))
    torch.cuda.synchronize()
    assert host(out).tobytes() == oracle.read_rows(p, idx).tobytes()


def test_unaligned_buffers_take_the_one_float_path():
    rng = np.random.default_rng(1)
    rows, cols, n = 700, 128, 300
    p = rng.standard_normal((rows, cols)).astype(np.float32)
    idx = rng.integers(0, rows, size=n)
    pbuf = torch.zeros(rows * cols + 1, device="cuda")
    pbuf[1:] = dev(p.reshape(-1))
    obuf = torch.full((n * cols + 1,), -3.0, device="cuda")
    L.read_rows(pbuf[1:].view(rows, cols), dev(idx), out=obuf[1:].view(n, cols))
    torch.cuda.synchronize()
    o = host(obuf)
    assert o[0] == -3.0
    assert o[1:].tobytes() == oracle.read_rows(p, idx).reshape(-1).tobytes()


def test_reads_the_table_after_a_step_on_the_same_stream():
    w = synth.WORKLOADS[3].scaled(rows=20000, n_lookups=3000, steps=3)
    p0 = synth.init_params(w)
    ora = oracle.Adam(p0.copy(), mode=w.mode)
    gpu = L.SparseAdam(dev(p0), mode=w.mode)
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ora.step_coo(keys, sums, width=w.cols)
        gpu.step(L.CooGradient(dev(keys), dev(sums), dim=w.rows, width=w.cols))
        nxt, _ = synth.lookups(w, s + 100)
        got = gpu.read_rows(dev(nxt))        # no synchronisation in between
        torch.cuda.synchronize()
        assert host(got).tobytes() == host(gpu.params)[nxt].tobytes()
        want = oracle.read_rows(ora.p, nxt)
        assert np.abs(host(got) - want).max() <= 1e-5 * np.abs(want).max() + 1e-7


def test_out_of_range_and_corrupted_rows():
    rows, cols = 100, 16
    p = np.ones((rows, cols), np.float32)
    p[7, 3] = np.inf
    out = torch.full((3, cols), 5.0, device="cuda")
    idx = dev(np.array([2, 7, 100], np.int64))
    with pytest.raises(L.SparseOptError) as e:
        L.read_rows(dev(p), idx, out=out, validate=True)
    assert e.value.code == oracle.ERANGE
    with pytest.raises(L.SparseOptError) as e:
        L.read_rows(dev(p), dev(np.array([2, 7], np.int64)), out=out[:2], validate=True)
    assert e.value.code == oracle.ENONFINITE
    torch.cuda.synchronize()
    assert (host(out) == 5.0).all()          # nothing written on error
    L.read_rows(dev(p), idx, out=out)         # trusted: the bad index reads zeros
    torch.cuda.synchronize()
    o = host(out)
    assert (o[0] == 1).all() and np.isinf(o[1, 3]) and (o[2] == 0).all()
    assert L.read_rows(dev(p), dev(np.zeros(0, np.int64))).shape == (0, cols)


def test_read_rows_full_size_table():
    """The 10M x 128 table and one step's 65,536 Zipf lookups, bit-exact."""
    w = synth.WORKLOADS[3]
    p0 = synth.init_params(w)
    params = torch.from_numpy(p0).to("cuda")
    ids, _ = synth.lookups(w, 0)
    out = L.read_rows(params, dev(ids))
    torch.cuda.synchronize()
    assert host(out).tobytes() == oracle.read_rows(p0, ids).tobytes()
