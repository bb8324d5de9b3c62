"""GPU parity of sparse_step_from_lookups: raw lookups -> one optimizer step in one call.

Pages: optirs_gpu sparse_optimizer, "LazyAdamMode::Lazy" /
"LazyAdamMode::DormancyDecay" and "Sparse SGD" (the update of the touched
coordinates), applied to the canonical gradient of the DiskSparseAdam README,
"Safe Duplicate Aggregation & Sorted I/O" (duplicates summed, ids sorted).
Checked bit for bit against the library's two calls (csr_from_lookups, then the
step on its CSR), which the other GPU tests hold to the oracle, and over several
steps against the oracle itself (its canonicalisation, then its step) within the
state tolerance.
"""
import numpy as np
import pytest
import torch

import lazy_optimizer_step_amd as L
import oracle
from tests.gpu_util import assert_state_close, dev, host
from tests.test_gpu_csr_from_lookups import _ids

pytestmark = pytest.mark.gpu


def _make(kind, rows, cols, seed, cfg):
    rng = np.random.default_rng(seed)
    p0 = (rng.standard_normal((rows, cols)) * 0.01).astype(np.float32)
    cls = L.SparseAdam if kind == "adam" else L.SparseSgd
    return cls(dev(p0), **cfg), cls(dev(p0), **cfg), p0


def _state(o):
    if isinstance(o, L.SparseAdam):
        ts = [o.params, o.m, o.v, o.last_step]
    else:
        ts = [o.params] + ([o.momentum_buf] if o.momentum_buf is not None else [])
    return [host(t).tobytes() for t in ts]


def _outputs(csr, counts, U, cols):
    u = int(host(U)[0])
    out = [u, host(csr.touched_rows)[:u].tobytes(),
           host(csr.values).reshape(-1)[:u * cols].tobytes(), host(counts)[:u].tobytes(),
           host(csr.row_offsets).tobytes()]
    if csr.col_indices is not None:
        out.append(host(csr.col_indices)[:u * cols].tobytes())
    return out


def _run_pair(kind, cfg, rows, cols, n, pattern, steps=3, seed=0, ro_shift=0, want_cols=True,
              validate=False):
    a, b, _ = _make(kind, rows, cols, seed, cfg)
    rng = np.random.default_rng(seed + 1)
    ro_buf = torch.empty(rows + 1 + ro_shift, dtype=torch.int32, device="cuda")
    for s in range(steps):
        ids = _ids(rows, n, pattern, rng)
        vals = rng.standard_normal((n, cols)).astype(np.float32)
        di, dv = dev(ids), dev(vals)
        got = a.step_lookups(di, dv, row_offsets=ro_buf[ro_shift:], want_col_indices=want_cols,
                             validate=validate)
        csr, counts, U = L.csr_from_lookups(di, dv, rows, want_col_indices=want_cols)
        b.step(csr)
        torch.cuda.synchronize()
        assert a.t == b.t == s + 1
        assert _outputs(*got, cols) == _outputs(csr, counts, U, cols), f"outputs, step {s + 1}"
        assert _state(a) == _state(b), f"table, step {s + 1}"


ADAM_CFGS = [
    dict(mode="dormancy"),
    dict(mode="lazy", weight_decay=0.01, weight_decay_mode="l2"),
    dict(mode="dormancy", weight_decay=0.02, weight_decay_mode="decoupled"),
    dict(mode="dormancy", last_step_per_row=True),
    dict(mode="lazy", weight_decay=0.01, weight_decay_mode="decoupled", last_step_per_row=True),
]


@pytest.mark.parametrize("pattern", ["uniform", "hot"])
@pytest.mark.parametrize("cfg", ADAM_CFGS, ids=lambda c: "-".join(f"{k}={v}" for k, v in c.items()))
def test_adam_matches_two_calls(cfg, pattern):
    _run_pair("adam", cfg, 50000, 128, 20000, pattern)


@pytest.mark.parametrize("cfg", [dict(lr=0.05), dict(lr=0.05, momentum=0.9, weight_decay=0.01)],
                         ids=["plain", "momentum-wd"])
@pytest.mark.parametrize("pattern", ["uniform", "hot"])
def test_sgd_matches_two_calls(cfg, pattern):
    _run_pair("sgd", cfg, 50000, 128, 20000, pattern)


@pytest.mark.parametrize("rows,cols,n,pattern,ro_shift", [
    (4000, 4, 30000, "uniform", 0),     # 4 lanes per row
    (3000, 12, 9000, "hot", 0),         # 16 lanes, 3 vectors per row
    (3000, 64, 9000, "all", 0),         # 16 lanes, every row touched
    (3000, 256, 5000, "uniform", 0),    # 64 lanes per row
    (20000, 128, 65536, "hot", 0),      # a segment over 150 tiles: the combine in runs
    (1000, 6, 3000, "hot", 0),          # columns not in groups of 4: the two calls inside
    (24577, 8, 9000, "hot", 3),         # row_offsets not 16-byte aligned: the two calls inside
    (2_000_000, 4, 500, "last_rows", 0),
    (5, 8, 7000, "uniform", 0),         # a handful of rows, long segments
    (1, 8, 5000, "uniform", 0),         # one row: 0 key bits, no radix pass, one segment
    (2, 16, 3000, "uniform", 0),        # two rows: one 1-bit pass
])
def test_shapes_match_two_calls(rows, cols, n, pattern, ro_shift):
    _run_pair("adam", dict(mode="dormancy"), rows, cols, n, pattern, ro_shift=ro_shift)


def test_without_col_indices():
    _run_pair("adam", dict(mode="dormancy"), 30000, 32, 12000, "hot", want_cols=False)


def test_validated_call_matches_two_calls():
    _run_pair("adam", dict(mode="dormancy", last_step_per_row=True), 30000, 16, 12000, "hot",
              validate=True)


def test_many_steps_reusing_buffers():
    """Ten steps through the same output and workspace buffers, the number of
    lookups changing, against the two calls on their own buffers."""
    rows, cols = 100000, 64
    a, b, _ = _make("adam", rows, cols, 3, dict(mode="dormancy"))
    nmax = 40000
    ws = torch.empty(L.sparse_opt_workspace_size(nmax, cols, rows), dtype=torch.uint8,
                     device="cuda")
    bufs = dict(out_keys=torch.empty(nmax, dtype=torch.int64, device="cuda"),
                out_vals=torch.empty((nmax, cols), dtype=torch.float32, device="cuda"),
                out_counts=torch.empty(nmax, dtype=torch.int32, device="cuda"),
                d_nunique=torch.empty(1, dtype=torch.int64, device="cuda"),
                row_offsets=torch.empty(rows + 1, dtype=torch.int32, device="cuda"),
                col_indices=torch.empty(nmax * cols, dtype=torch.int32, device="cuda"))
    rng = np.random.default_rng(4)
    for s, n in enumerate([40000, 1, 25000, 0, 39999, 256, 257, 2048, 30000, 40000]):
        ids = _ids(rows, n, "hot" if s % 2 else "uniform", rng)
        vals = rng.standard_normal((n, cols)).astype(np.float32)
        di, dv = dev(ids), dev(vals)
        kw = dict(bufs)
        kw["out_keys"] = bufs["out_keys"][:max(n, 1)]
        kw["out_vals"] = bufs["out_vals"][:max(n, 1)]
        kw["out_counts"] = bufs["out_counts"][:max(n, 1)]
        kw["col_indices"] = bufs["col_indices"][:max(n * cols, 1)]
        got = a.step_lookups(di, dv, workspace=ws, **kw)
        csr, counts, U = L.csr_from_lookups(di, dv, rows)
        b.step(csr)
        torch.cuda.synchronize()
        assert _outputs(*got, cols) == _outputs(csr, counts, U, cols), f"outputs, step {s + 1}"
        assert _state(a) == _state(b), f"table, step {s + 1} ({n} lookups)"


def test_empty_lookups():
    rows, cols = 5000, 16
    a, _, p0 = _make("adam", rows, cols, 5, dict(mode="dormancy"))
    csr, counts, U = a.step_lookups(torch.empty(0, dtype=torch.int64, device="cuda"),
                                    torch.empty((0, cols), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert a.t == 1
    assert int(host(U)[0]) == 0
    assert not host(csr.row_offsets).any()
    assert host(a.params).tobytes() == p0.tobytes()
    assert not host(a.last_step).any()


def test_trusted_out_of_range_id_touches_nothing():
    """Trusted mode: an id outside the table gives U = 0 (the canonicalisation's
    rule), so no row is updated; t still advances, as with the two calls."""
    rows, cols = 20000, 32
    a, b, p0 = _make("adam", rows, cols, 6, dict(mode="dormancy"))
    rng = np.random.default_rng(7)
    ids = _ids(rows, 9000, "hot", rng)
    ids[4321] = rows + 5
    vals = rng.standard_normal((9000, cols)).astype(np.float32)
    got = a.step_lookups(dev(ids), dev(vals))
    csr, counts, U = L.csr_from_lookups(dev(ids), dev(vals), rows)
    b.step(csr)
    torch.cuda.synchronize()
    assert a.t == 1 and int(host(got[2])[0]) == 0
    assert host(a.params).tobytes() == p0.tobytes()
    assert _state(a) == _state(b)
    with pytest.raises(L.SparseOptError):
        a.step_lookups(dev(ids), dev(vals), validate=True)
    assert a.t == 1


@pytest.mark.parametrize("kind,cfg", [
    ("adam", dict(mode="dormancy")),
    ("adam", dict(mode="lazy", weight_decay=0.01, weight_decay_mode="decoupled")),
    ("sgd", dict(lr=0.05, momentum=0.9, weight_decay=0.01)),
])
def test_against_oracle(kind, cfg):
    """Four steps from raw lookups against the oracle's canonicalisation and step."""
    rows, cols, n = 30000, 64, 15000
    a, _, p0 = _make(kind, rows, cols, 8, cfg)
    if kind == "adam":
        o = oracle.Adam(p0.copy(), **cfg)
    else:
        o = oracle.Sgd(p0.copy(), **cfg)
    rng = np.random.default_rng(9)
    for s in range(4):
        ids = _ids(rows, n, "hot" if s % 2 else "uniform", rng)
        vals = rng.standard_normal((n, cols)).astype(np.float32)
        a.step_lookups(dev(ids), dev(vals))
        ok, ov, oc = oracle.coo_from_lookups(ids, vals, rows)
        o.step_coo(ok, ov, width=cols)
    torch.cuda.synchronize()
    assert_state_close(host(a.params), o.p, "params")
    if kind == "adam":
        assert_state_close(host(a.m), o.m, "m")
        assert_state_close(host(a.v), o.v, "v")
        assert np.array_equal(host(a.last_step), o.ls)
    else:
        assert_state_close(host(a.momentum_buf), o.b, "momentum")


@pytest.mark.parametrize("n", [65536, 70001])
def test_every_lookup_on_one_row(n):
    """All lookups hit one row: one segment across every segment tile (256 and
    274 tiles), summed by the combine in 16 runs, then one row updated; against
    the oracle, and bit for bit against the two calls."""
    rows, cols = 5000, 128
    cfg = dict(mode="dormancy")
    a, b, p0 = _make("adam", rows, cols, 21, cfg)
    o = oracle.Adam(p0.copy(), **cfg)
    rng = np.random.default_rng(22)
    for s in range(2):
        ids = np.full(n, 1234 + s, np.int64)
        vals = rng.standard_normal((n, cols)).astype(np.float32)
        di, dv = dev(ids), dev(vals)
        got = a.step_lookups(di, dv)
        csr, counts, U = L.csr_from_lookups(di, dv, rows)
        b.step(csr)
        ok, ov, oc = oracle.coo_from_lookups(ids, vals, rows)
        o.step_coo(ok, ov, width=cols)
        torch.cuda.synchronize()
        assert int(host(got[2])[0]) == 1 and int(host(got[1])[0]) == n
        assert _outputs(*got, cols) == _outputs(csr, counts, U, cols)
        assert _state(a) == _state(b)
    assert_state_close(host(a.params), o.p, "params")
    assert_state_close(host(a.m), o.m, "m")
    assert_state_close(host(a.v), o.v, "v")
    assert np.array_equal(host(a.last_step), o.ls)


def test_binding_checks_shapes_against_the_handle():
    """The binding sizes and checks every array from the handle's rows and cols,
    so vals of another width are refused before the library is called."""
    a, _, _ = _make("adam", 1000, 8, 10, dict(mode="dormancy"))
    ids = torch.zeros(16, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        a.step_lookups(ids, torch.zeros((16, 4), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        a.step_lookups(ids, torch.zeros(16 * 8 + 1, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):   # row_offsets for fewer rows than the table's
        a.step_lookups(ids, torch.zeros((16, 8), dtype=torch.float32, device="cuda"),
                       row_offsets=torch.empty(500, dtype=torch.int32, device="cuda"))
    assert a.t == 0
    a.step_lookups(ids, torch.ones(16 * 8, dtype=torch.float32, device="cuda"))  # flat is fine
    torch.cuda.synchronize()
    assert a.t == 1 and host(a.last_step)[0].tolist() == [1] * 8


def test_scrambled_zipf_lookups_match_two_calls_and_oracle():
    """Zipf lookups with the hot rows spread over the table (the scrambled
    placement), three steps: bit for bit against the two calls, and the touched
    rows within tolerance of the oracle."""
    import synth
    w = synth.WORKLOADS[3].scaled(rows=2_000_000, n_lookups=30000, scramble=999983)
    h = w.hyper
    a, b, p0 = _make("adam", w.rows, w.cols, 11, dict(mode="dormancy"))
    touched = []
    for s in range(3):
        ids, grads = synth.lookups(w, s)
        touched.append(ids)
        got = a.step_lookups(dev(ids), dev(grads))
        csr, counts, U = L.csr_from_lookups(dev(ids), dev(grads), w.rows)
        b.step(csr)
        torch.cuda.synchronize()
        assert _outputs(*got, w.cols) == _outputs(csr, counts, U, w.cols), f"outputs, step {s + 1}"
        assert _state(a) == _state(b), f"table, step {s + 1}"
    rows = np.unique(np.concatenate(touched))
    o = oracle.Adam(p0[rows].copy(), lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"],
                    eps=h["eps"], mode="dormancy")
    for s in range(3):
        ids, grads = synth.lookups(w, s)
        ok, ov, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        o.step_coo(np.searchsorted(rows, ok), ov, width=w.cols)
    idx = torch.from_numpy(rows).cuda()
    assert_state_close(host(a.params.index_select(0, idx)), o.p, "params")
    assert_state_close(host(a.m.index_select(0, idx)), o.m, "m")
    assert np.array_equal(host(a.last_step.index_select(0, idx)), o.ls)


def test_random_configurations_match_two_calls():
    """A seeded sweep over widths (every lanes-per-row shape, rows wider than one
    vector per lane, widths not in groups of 4), table sizes, lookup counts, id
    patterns and optimizer forms: two steps each, bit for bit against the two
    calls."""
    rng = np.random.default_rng(2026)
    widths = [1, 3, 4, 8, 12, 16, 20, 32, 64, 100, 128, 256, 300, 302, 512]
    cfgs = ADAM_CFGS + [dict(lr=0.05), dict(lr=0.05, momentum=0.9, weight_decay=0.01)]
    for case in range(24):
        cols = int(widths[case % len(widths)])
        rows = int(rng.integers(1, 200_000))
        n = int(rng.integers(0, 20_000))
        pattern = ["uniform", "hot", "last_rows", "first_rows"][int(rng.integers(0, 4))]
        if pattern in ("last_rows", "first_rows") and rows < 50:
            pattern = "uniform"
        cfg = cfgs[int(rng.integers(0, len(cfgs)))]
        kind = "sgd" if "momentum" in cfg or "mode" not in cfg else "adam"
        try:
            _run_pair(kind, cfg, rows, cols, n, pattern, steps=2, seed=case)
        except AssertionError as e:
            raise AssertionError(f"case {case}: rows {rows} cols {cols} n {n} {pattern} "
                                 f"{kind} {cfg}: {e}") from None


def test_one_call_resume_and_repeat_are_bit_identical():
    """Ten one-call steps: a run stopped after five, its state copied into a new
    handle whose step counter is set to 5, then resumed, ends bit for bit where
    the uninterrupted run does; and a second uninterrupted run repeats it."""
    import synth
    w = synth.WORKLOADS[3].scaled(rows=200_000, n_lookups=20000)
    p0 = synth.init_params(w)
    batches = [synth.lookups(w, s) for s in range(10)]
    runs = []
    for _ in range(2):
        a = L.SparseAdam(dev(p0), mode="dormancy")
        for ids, g in batches:
            a.step_lookups(dev(ids), dev(g))
        torch.cuda.synchronize()
        runs.append([host(x).tobytes() for x in (a.params, a.m, a.v, a.last_step)])
    assert runs[0] == runs[1]
    b = L.SparseAdam(dev(p0), mode="dormancy")
    for ids, g in batches[:5]:
        b.step_lookups(dev(ids), dev(g))
    torch.cuda.synchronize()
    c = L.SparseAdam(b.params.clone(), mode="dormancy")
    c.m.copy_(b.m)
    c.v.copy_(b.v)
    c.last_step.copy_(b.last_step)
    c.handle.set_step(b.t)
    for ids, g in batches[5:]:
        c.step_lookups(dev(ids), dev(g))
    torch.cuda.synchronize()
    assert c.t == 10
    assert [host(x).tobytes() for x in (c.params, c.m, c.v, c.last_step)] == runs[0]


def test_two_tables_on_two_streams():
    """Two tables stepped through the one call on two streams at once (each with
    its own buffers and workspace, the calls interleaved on the host): each ends
    bit for bit where the same steps on the default stream end."""
    import synth
    w1 = synth.WORKLOADS[3].scaled(rows=300_000, n_lookups=30000)
    w2 = synth.WORKLOADS[2].scaled(rows=100_000, n_lookups=8192)
    runs = {}
    for mode in ("sequential", "concurrent"):
        tabs = [L.SparseAdam(dev(synth.init_params(w)), mode=m)
                for w, m in ((w1, "dormancy"), (w2, "lazy"))]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()] if mode == "concurrent" else [None, None]
        torch.cuda.synchronize()
        for s in range(6):
            for k, (w, t) in enumerate(zip((w1, w2), tabs)):
                ids, g = synth.lookups(w, s)
                di, dg = dev(ids), dev(g)
                if streams[k] is not None:
                    streams[k].wait_stream(torch.cuda.current_stream())   # inputs copied
                    with torch.cuda.stream(streams[k]):
                        t.step_lookups(di, dg, stream=streams[k])
                        di.record_stream(streams[k])
                        dg.record_stream(streams[k])
                else:
                    t.step_lookups(di, dg)
        torch.cuda.synchronize()
        runs[mode] = [[host(x).tobytes() for x in (t.params, t.m, t.v, t.last_step)] for t in tabs]
    assert runs["sequential"] == runs["concurrent"]


def test_stream_argument_not_current_keeps_its_workspace():
    """stream= given without making it current: the binding allocates the call's
    workspace and outputs on that stream, so memory the current stream allocates
    and overwrites right after the call is never the memory the call's kernels
    (held back behind a bounded spin on their stream) still use.  Results equal
    the same calls on the current stream, bit for bit: the one-call step (stream
    as a torch.cuda.Stream) and coo_from_lookups (stream as a raw handle)."""
    import synth
    w = synth.WORKLOADS[3].scaled(rows=300_000, n_lookups=30000)
    batches = [synth.lookups(w, s) for s in range(4)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1 << 20)
    e1.record()
    torch.cuda.synchronize()
    hold = int((1 << 20) * 3.0 / max(e0.elapsed_time(e1), 1e-3))  # about 3 ms
    nbytes = L.sparse_opt_workspace_size(w.n_lookups, w.cols, w.rows)
    runs = {}
    for mode in ("current", "other"):
        t = L.SparseAdam(dev(synth.init_params(w)), mode="dormancy")
        side = torch.cuda.Stream()
        outs = []
        for ids, g in batches:
            di, dg = dev(ids), dev(g)
            if mode == "current":
                csr, counts, U = t.step_lookups(di, dg)
                keys, sums, cnt, u = L.coo_from_lookups(di, dg, w.rows)
            else:
                side.wait_stream(torch.cuda.current_stream())  # inputs copied
                with torch.cuda.stream(side):
                    torch.cuda._sleep(hold)
                csr, counts, U = t.step_lookups(di, dg, stream=side)
                junk = [torch.full((nbytes // 4 + 4096,), float("nan"), device="cuda")
                        for _ in range(3)]
                with torch.cuda.stream(side):
                    torch.cuda._sleep(hold)
                keys, sums, cnt, u = L.coo_from_lookups(di, dg, w.rows, stream=side.cuda_stream)
                junk += [torch.full((nbytes // 4 + 4096,), float("nan"), device="cuda")
                         for _ in range(3)]
                for x in (di, dg):
                    x.record_stream(side)
            outs.append((csr.touched_rows, csr.values, counts, U, keys, sums, cnt, u))
        torch.cuda.synchronize()
        res = []
        for o in outs:
            n = int(host(o[3])[0])
            assert n == int(host(o[7])[0])
            res.append([host(o[0])[:n].tobytes(), host(o[1])[:n].tobytes(),
                        host(o[2])[:n].tobytes(), host(o[4])[:n].tobytes(),
                        host(o[5])[:n].tobytes(), host(o[6])[:n].tobytes()])
        res.append([host(x).tobytes() for x in (t.params, t.m, t.v, t.last_step)])
        runs[mode] = res
    assert runs["current"] == runs["other"]
