"""The allocation-free step from raw lookups (sparse_step_from_lookups_noalloc,
workspace in the library's fixed device scratch) against the same step with a
caller-allocated workspace (sparse_step_from_lookups), through the C ABI.

Two calls in a row on each pair of tables, the second with fewer lookups, so
the second call runs on scratch that still holds the first call's contents.
Both calls run the same kernels on the same inputs, so every output (distinct
ids, counts, summed rows, row_offsets, col_indices, U) and the whole table
after each call must agree bit for bit (page "optirs_gpu::sparse_optimizer",
the step from a CooGradient; DiskSparseAdam README, duplicates summed).
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


class Outs:
    def __init__(self, n, rows, cols):
        self.keys = torch.full((n,), -1, dtype=torch.int64, device="cuda")
        self.vals = torch.full((n, cols), -1.0, dtype=torch.float32, device="cuda")
        self.counts = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        self.U = torch.full((1,), -1, dtype=torch.int64, device="cuda")
        self.ro = torch.full((rows + 1,), -1, dtype=torch.int32, device="cuda")
        self.ci = torch.full((n * cols,), -1, dtype=torch.int32, device="cuda")

    def kw(self):
        return dict(out_keys=self.keys, out_vals=self.vals, out_counts=self.counts,
                    d_nunique=self.U, row_offsets=self.ro, col_indices=self.ci)

    def result(self, cols):
        u = int(host(self.U)[0])
        return [u, host(self.keys)[:u].tobytes(), host(self.counts)[:u].tobytes(),
                host(self.vals)[:u].tobytes(), host(self.ro).tobytes(),
                host(self.ci)[:u * cols].tobytes()]


def _state(t):
    parts = [t.params] + ([t.m, t.v, t.last_step] if isinstance(t, L.SparseAdam)
                          else [t.momentum_buf])
    return [host(x).tobytes() for x in parts]


@pytest.mark.parametrize("kind", ["adam", "sgd"])
def test_noalloc_step_matches_step_with_workspace(kind):
    w = synth.WORKLOADS[3].scaled(rows=300_000, n_lookups=30000)
    p0 = synth.init_params(w)
    if kind == "adam":
        a, b = (L.SparseAdam(dev(p0), mode="dormancy") for _ in range(2))
    else:
        a, b = (L.SparseSgd(dev(p0), lr=0.05, momentum=0.9, weight_decay=1e-4) for _ in range(2))
    n_max = w.n_lookups
    oa, ob = Outs(n_max, w.rows, w.cols), Outs(n_max, w.rows, w.cols)
    ws = torch.empty(L.sparse_opt_workspace_size(n_max, w.cols, w.rows), dtype=torch.uint8,
                     device="cuda")
    for s, n in enumerate((n_max, 4000)):   # the second call with fewer lookups
        ids, grads = synth.lookups(w, s, n)
        di, dg = dev(ids), dev(grads)
        L.sparse_step_from_lookups(a.handle, di, dg, workspace=ws, **oa.kw())
        L.sparse_step_from_lookups_noalloc(b.handle, di, dg, **ob.kw())
        torch.cuda.synchronize()
        ra, rb = oa.result(w.cols), ob.result(w.cols)
        assert ra[0] == rb[0] > 0, f"call {s}: U"
        names = ["U", "keys", "counts", "sums", "row_offsets", "col_indices"]
        for name, x, y in zip(names, ra, rb):
            assert x == y, f"call {s}: {name} differs"
        assert _state(a) == _state(b), f"call {s}: table differs"
    assert a.t == b.t == 2


def test_noalloc_step_on_another_table_after_a_larger_one():
    """A second handle of another shape (64 columns, 1M rows) after the calls
    above left the scratch holding a larger layout: still bit for bit."""
    w = synth.WORKLOADS[2].scaled(n_lookups=8192)
    p0 = synth.init_params(w)
    a, b = (L.SparseAdam(dev(p0), mode="lazy") for _ in range(2))
    for s, n in enumerate((8192, 1500)):
        oa, ob = Outs(n, w.rows, w.cols), Outs(n, w.rows, w.cols)
        ids, grads = synth.lookups(w, s, n)
        di, dg = dev(ids), dev(grads)
        L.sparse_step_from_lookups(a.handle, di, dg, **oa.kw())
        L.sparse_step_from_lookups_noalloc(b.handle, di, dg, **ob.kw())
        torch.cuda.synchronize()
        assert oa.result(w.cols) == ob.result(w.cols), f"call {s}"
        assert _state(a) == _state(b), f"call {s}: table differs"
