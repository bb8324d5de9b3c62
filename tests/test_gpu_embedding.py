"""The embedding training path: read_rows forward, autograd backward, and the
whole sparse step, against the oracle on the same per-lookup gradients.

Pages: DiskSparseAdam README (training loop: read_rows, then step with the
lookup indices and gradient rows; duplicates summed); optirs_gpu
sparse_optimizer (the update on touched rows only).  The per-lookup gradient
rows are the GPU autograd's, copied to the host and fed to the oracle as
inputs; the oracle computes every expected value.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from lazy_optimizer_step_amd.embedding import SparseEmbedding
from tests.gpu_util import assert_state_close, dev, host

pytestmark = pytest.mark.gpu


def _train(opt_name, mode="dormancy", batches_per_step=1, steps=6, **kw):
    w = synth.WORKLOADS[3].scaled(rows=30000, n_lookups=2000, steps=steps)
    p0 = synth.init_params(w)
    emb = SparseEmbedding(w.rows, w.cols, optimizer=opt_name, weight=p0, **kw)
    if opt_name == "adam":
        ora = oracle.Adam(p0.copy(), mode=mode, **{k: v for k, v in kw.items() if k != "mode"})
    else:
        ora = oracle.Sgd(p0.copy(), **kw)
    rng = np.random.default_rng(3)
    for s in range(steps):
        all_ids = []
        for b in range(batches_per_step):
            ids, _ = synth.lookups(w, s * 10 + b)
            target = torch.from_numpy(rng.standard_normal((ids.size, w.cols)).astype(np.float32))
            out = emb(dev(ids))
            torch.cuda.synchronize()
            # the forward is the current table's rows
            assert host(out).tobytes() == oracle.read_rows(host(emb.weight), ids).tobytes()
            loss = ((out - target.cuda()) ** 2).sum()
            loss.backward()
            all_ids.append(ids)
        ids = np.concatenate(all_ids)
        grads = np.concatenate([host(g) for _, g in emb._pending])
        assert np.array_equal(np.concatenate([host(i) for i, _ in emb._pending]), ids)
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        ora.step_csr(ro, ci, cv)
        assert emb.step() == ids.size
        assert not emb._pending
    torch.cuda.synchronize()
    assert_state_close(host(emb.weight), ora.p, f"{opt_name} params")
    return emb, ora


@pytest.mark.parametrize("batches_per_step", [1, 3])
def test_embedding_adam(batches_per_step):
    emb, ora = _train("adam", lr=1e-2, batches_per_step=batches_per_step)
    assert np.array_equal(host(emb.opt.last_step), ora.ls)
    assert_state_close(host(emb.opt.m), ora.m, "m")
    assert_state_close(host(emb.opt.v), ora.v, "v")


def test_embedding_adam_with_decay():
    emb, ora = _train("adam", lr=1e-2, weight_decay=0.5, weight_decay_mode="decoupled")
    assert np.array_equal(host(emb.opt.last_step), ora.ls)


def test_embedding_sgd():
    emb, ora = _train("sgd", lr=0.05, momentum=0.9, weight_decay=1e-4)
    assert_state_close(host(emb.opt.momentum_buf), ora.b, "momentum")


def test_step_without_lookups_does_nothing():
    emb = SparseEmbedding(100, 8)
    w0 = host(emb.weight).copy()
    assert emb.step() == 0
    assert emb.opt.t == 0 and host(emb.weight).tobytes() == w0.tobytes()
