"""Host-resident state (tables larger than device memory): p, m, v and last_step
in mapped pinned host memory, updated in place by the same kernels, so only the
touched rows cross the host link.

Page: DiskSparseAdam README, "Key Features" (w, m, v and step counters out of
core; only the rows a batch touches are loaded and written back).  Checked
against the oracle and bit for bit against the same steps on device-resident
state, and through the one-call step from raw lookups.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import lazy_optimizer_step_amd._lib as _lib
import oracle
import synth
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("per_row", [False, True])
def test_host_resident_adam_whole_path(per_row):
    w = synth.WORKLOADS[3].scaled(rows=50000, n_lookups=5000, steps=8)
    p0 = synth.init_params(w)
    kw = dict(lr=1e-2, mode="dormancy", last_step_per_row=per_row)
    hst = L.SparseAdam.host_resident(p0, **kw)
    one = L.SparseAdam.host_resident(p0, **kw)      # stepped through the one call
    devr = L.SparseAdam(dev(p0), **kw)
    ora = (oracle.AdamRows if per_row else oracle.Adam)(p0.copy(), lr=1e-2, mode="dormancy")
    for s in range(w.steps):
        ids, grads = synth.lookups(w, s)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        gk, gs, _, U = L.coo_from_lookups(dev(ids), dev(grads), w.rows)
        coo = L.CooGradient(gk, gs, dim=w.rows, width=w.cols, nnz=ids.size, d_nnz=U)
        csr = L.csr_from_coo(coo, w.rows, w.cols, copy_values=False)
        hst.step(csr)
        devr.step(csr)
        one.step_lookups(dev(ids), dev(grads))
    torch.cuda.synchronize()
    hp, hm, hv, hl = (a.numpy() for a in (hst.params, hst.m, hst.v, hst.last_step))
    assert np.array_equal(hl, ora.ls)
    assert_state_close(hp, ora.p, "host params")
    assert_state_close(hm, ora.m, "host m")
    assert_state_close(hv, ora.v, "host v")
    for a, b in ((hp, devr.params), (hm, devr.m), (hv, devr.v), (hl, devr.last_step)):
        assert a.tobytes() == host(b).tobytes()
    for a, b in ((hp, one.params), (hm, one.m), (hv, one.v), (hl, one.last_step)):
        assert a.tobytes() == b.numpy().tobytes()
    untouched = ora.ls.reshape(w.rows, -1)[:, 0] == 0
    assert hp[untouched].tobytes() == p0[untouched].tobytes()
    # forward gather straight from the host-resident table
    nxt, _ = synth.lookups(w, 99)
    got = hst.read_rows(dev(nxt))
    torch.cuda.synchronize()
    assert host(got).tobytes() == hp[nxt].tobytes()


def test_host_alloc_errors_and_foreign_pinned_memory():
    h, d = C.c_void_p(), C.c_void_p()
    assert _lib.lib().sparse_opt_host_alloc(0, C.byref(h), C.byref(d)) == _lib.EINVAL
    assert _lib.lib().sparse_opt_host_device_pointer(None, C.byref(d)) == _lib.EINVAL
    plain = np.zeros(1024, np.float32)               # pageable: no device mapping
    assert _lib.lib().sparse_opt_host_device_pointer(C.c_void_p(plain.ctypes.data),
                                                     C.byref(d)) == _lib.EINVAL
    # pinned memory from torch: used only if the runtime reports a device mapping
    t = torch.arange(64 * 8, dtype=torch.float32).reshape(64, 8).pin_memory()
    rc = _lib.lib().sparse_opt_host_device_pointer(C.c_void_p(t.data_ptr()), C.byref(d))
    if rc == _lib.OK:
        out = torch.empty((3, 8), device="cuda")
        idx = dev(np.array([5, 0, 63], np.int64))
        _lib.check(_lib.lib().read_rows(d, 64, 8, C.c_void_p(idx.data_ptr()), 3,
                                        C.c_void_p(out.data_ptr()), None, 0))
        torch.cuda.synchronize()
        assert host(out).tobytes() == t.numpy()[[5, 0, 63]].tobytes()
    else:
        assert rc == _lib.EINVAL
