"""Benchmark of the sparse / lazy Adam step on one MI355X.

One step is the whole hot path over one batch of raw lookups, in one call:
  sparse_step_from_lookups  (radix sort, dedupe, duplicate sums; then one
                             launch that completes the tile-crossing sums,
                             writes row_offsets over every table row and
                             col_indices, and applies the DormancyDecay update
                             to the touched coordinates)
(--two-calls: csr_from_lookups then sparse_adam_step on its CSR;
--separate-calls: coo_from_lookups, csr_from_coo, sparse_adam_step.)
on the 10M x 128 float32 table (65,536 Zipf(1.05) lookups per step, last_step
int32 per coordinate).  Inputs for every step are generated up front and are
resident in HBM before the timed region starts.

Prints one JSON line:  value = touched coordinates updated per second over the
whole timed region (G/s); roofline = the algorithmic bytes of the launch that
updates the table / its mean duration (HIP events that the library attaches to
that launch's dispatch through its timing hook, so they take the kernel's own
start and end times on its stream, at every step of the timed region) against
8 TB/s, with a plain 1 GiB device copy measured
alongside as the practical bandwidth ceiling; breakdown_us = p10 / median / p90
of each call, of that launch and of the whole step from a second, separately
timed pass over the same inputs; cold = that launch again in a third pass that
writes a 512 MB buffer before every step, so the state rows come from HBM
rather than the 256 MB last-level cache; read_rows = the forward gather of each
step's lookups, timed in a pass of its own; cpu_baseline = the CPU oracle on a
bounded sample of the same workload.

--workload picks another workload of the same family: table1Mx64 (1M x 64
rows, 8,192 Zipf(1.1) lookups a step, Lazy), table50Mx128 (50M x 128 rows,
262,144 Zipf(1.2) lookups, DormancyDecay), or partial2Mx256-sgd /
partial2Mx256-adam (2M x 256 rows, 16,384 rows a step with 16-64 of their
columns each: csr_from_coo of the step's flat COO, then sparse_sgd_step
(lr 0.05, momentum 0.9, coupled weight decay 1e-4) or the DormancyDecay
sparse_adam_step on that CSR).  Each prints its own JSON line of the same
form; the value is touched coordinates (nonzeros for partial rows) per second.

Events are created through the HIP runtime with hipEventDisableSystemFence:
they only take timestamps, and skipping the system-scope release (an L2
writeback and invalidate per record) keeps them from slowing the work they
bracket.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "touched coords updated/sec (G/s) + achieved HBM GB/s % of peak, 10M x 128 table"
HBM_PEAK_GBS = 8000.0
# Algorithmic bytes of the DormancyDecay update: per touched coordinate read p, m, v,
# last_step, g (20 B) and write p, m, v, last_step (16 B); per touched row read its id
# (8 B) and two row offsets (8 B).  With one last_step per row (--last-step-per-row):
# 28 B per coordinate, and the row's last_step read and written (8 B more per row).
BYTES_PER_COORD = 36
BYTES_PER_ROW = 16
BYTES_PER_COORD_ROW_LS = 28
BYTES_PER_ROW_ROW_LS = 24
# The one-call step (sparse_step_from_lookups) updates the table in the same
# launch that writes the CSR: col_indices (4 B per touched coordinate), each
# distinct id read once more by the row_offsets blocks (8 B per touched row),
# row_offsets (4 B per table row, plus one) and the per-8192-row id counts
# they read (4 B per block).  Not counted: the combine's reads of the double
# partial sums of tile-crossing segments (at most two 8*cols B rows per
# 256-lookup tile, about 0.5% of the launch's bytes here).
# --scrambled: a prime multiplier, coprime to the 10M rows.
SCRAMBLE = 999983
CSR_BYTES_PER_COORD = 4
CSR_BYTES_PER_ROW = 8
CSR_BYTES_PER_TABLE_ROW = 4

# HBM bytes per launch of the kernel that updates the table, from two
# rocprofv3 --pmc passes of this command (FETCH_SIZE scaled by 2.0 and
# WRITE_SIZE by 1.0: a plain 1 GiB device copy reads 512 MiB by FETCH_SIZE and
# writes 1 GiB by WRITE_SIZE), keyed by (workload, step form): the one-call
# step's k_step_lookups, the two-call step's k_update_rows, and the partial-row
# step's k_update_csr_scan.  Valid only for the kernel sources they were taken
# with; reported as null once those sources change.
UPDATE_SOURCES = ("lazy_optimizer_step_amd/csrc/update.hip",
                  "lazy_optimizer_step_amd/csrc/common.hpp",
                  "lazy_optimizer_step_amd/csrc/csr_full.hpp",
                  "lazy_optimizer_step_amd/csrc/seg_combine.hpp")
_SHA = "fb924673ee4e4dd63f645161355a1fed2c1b8a51e099d49dd4dd835d4bfeee81"
TRAFFIC = {
    ("table10Mx128_zipf1.05_dormancy", "one_call"): {
        "sources_sha256": _SHA, "fetch_bytes": 2.0 * 33409.7 * 1024,
        "write_bytes": 1.0 * 104262.0 * 1024},
    ("table10Mx128_zipf1.05_dormancy", "two_calls"): {
        "sources_sha256": _SHA, "fetch_bytes": 2.0 * 33768.9 * 1024,
        "write_bytes": 1.0 * 52105.9 * 1024},
    ("table2Mx256_csr16-64_sgd", "two_calls"): {
        "sources_sha256": _SHA, "fetch_bytes": 2.0 * 23935.2 * 1024,
        "write_bytes": 1.0 * 23465.3 * 1024},
    ("table2Mx256_csr16-64_dormancy", "two_calls"): {
        "sources_sha256": _SHA, "fetch_bytes": 2.0 * 40161.6 * 1024,
        "write_bytes": 1.0 * 46930.6 * 1024},
}


def sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in UPDATE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--two-calls", action="store_true",
                    help="step with csr_from_lookups + sparse_adam_step instead of the one "
                         "call sparse_step_from_lookups")
    ap.add_argument("--separate-calls", action="store_true",
                    help="step with coo_from_lookups + csr_from_coo + sparse_adam_step")
    ap.add_argument("--last-step-per-row", action="store_true",
                    help="keep one last_step per table row instead of one per coordinate")
    ap.add_argument("--scrambled", action="store_true",
                    help="the same Zipf frequencies with the hot rows spread over the table "
                         "(rank k -> row (k-1)*999983 mod rows) instead of at the lowest ids")
    ap.add_argument("--host-state", action="store_true",
                    help="keep the table and its state in mapped pinned host memory")
    ap.add_argument("--workload", default="table10Mx128", choices=sorted(WORKLOAD_CHOICES),
                    help="table10Mx128 (default), table1Mx64, table50Mx128, partial2Mx256-sgd "
                         "or partial2Mx256-adam")
    return ap.parse_args()


# --workload: (synth workload number, optimizer of the partial-row workload)
WORKLOAD_CHOICES = {"table1Mx64": (2, None), "table10Mx128": (3, None),
                    "table50Mx128": (5, None), "partial2Mx256-sgd": (4, "sgd"),
                    "partial2Mx256-adam": (4, "adam")}


class HipEvents:
    """Timing-only HIP events (hipEventDisableSystemFence) recorded on a given
    stream, from the HIP runtime this process has already loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, count: int):
        import ctypes as C

        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        self.C = C
        self.hip = C.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = []
        for _ in range(count):
            e = C.c_void_p()
            self._check(self.hip.hipEventCreateWithFlags(C.byref(e), self.DISABLE_SYSTEM_FENCE),
                        "hipEventCreateWithFlags")
            self.ev.append(e)

    @staticmethod
    def _check(rc: int, what: str) -> None:
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, i: int, stream) -> None:
        self._check(self.hip.hipEventRecord(self.ev[i], self.C.c_void_p(stream.cuda_stream)),
                    "hipEventRecord")

    def ms(self, i: int, j: int) -> float:
        out = self.C.c_float()
        self._check(self.hip.hipEventElapsedTime(self.C.byref(out), self.ev[i], self.ev[j]),
                    "hipEventElapsedTime")
        return float(out.value)

    def close(self) -> None:
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def calibrate_sleep(torch, stream, hold_ms: float) -> int:
    """Spin-kernel cycles that hold the stream for about hold_ms milliseconds."""
    probe = 1 << 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(probe)
    e0.record(stream)
    torch.cuda._sleep(probe)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = max(e0.elapsed_time(e1), 1e-3)
    return int(min(probe * hold_ms / ms, 1 << 40))


def device_copy_gbs(torch, stream) -> float:
    """Best of 5 plain 1 GiB device-to-device copies (torch's copy kernel), in
    GB/s of bytes read + written: the practical ceiling next to the peak."""
    n = 1 << 28
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    ev = HipEvents(2)
    best = float("inf")
    for _ in range(5):
        ev.record(0, stream)
        b.copy_(a)
        ev.record(1, stream)
        torch.cuda.synchronize()
        best = min(best, ev.ms(0, 1))
    ev.close()
    return 2.0 * 4 * n / (best * 1e-3) / 1e9


def host_link_gbs(torch, stream) -> dict:
    """Best of 3 copies of 1 GiB between pinned host memory and the device, each
    direction, in GB/s: the host link's practical rate."""
    n = 1 << 28
    h = torch.ones(n, dtype=torch.float32).pin_memory()
    d = torch.empty(n, dtype=torch.float32, device="cuda")
    ev = HipEvents(2)
    out = {}
    for name, dst, src in (("host_to_device", d, h), ("device_to_host", h, d)):
        best = float("inf")
        for _ in range(3):
            ev.record(0, stream)
            dst.copy_(src, non_blocking=True)
            ev.record(1, stream)
            torch.cuda.synchronize()
            best = min(best, ev.ms(0, 1))
        out[name] = 4.0 * n / (best * 1e-3) / 1e9
    ev.close()
    return out


def pcts(x_ms) -> dict:
    """p10 / median / p90 of per-launch milliseconds, in microseconds."""
    import numpy as np

    p10, p50, p90 = np.percentile(np.asarray(x_ms) * 1e3, [10, 50, 90])
    return {"p10": float(p10), "p50": float(p50), "p90": float(p90)}


def copy_probe(steps: int) -> None:
    import torch

    n = 1 << 28  # 1 GiB of float32
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                      "launches": steps}), flush=True)


def cpu_baseline(w, host_p0, batches, budget_s: float, per_row: bool = False):
    """The oracle, as it stands, on the first steps of the same workload until the
    time budget is spent (at least 2 steps); single thread."""
    import numpy as np

    import oracle

    h = w.hyper
    m = np.zeros((w.rows, w.cols), np.float32)       # zero pages are mapped lazily
    v = np.zeros((w.rows, w.cols), np.float32)
    ls = np.zeros((w.rows,) if per_row else (w.rows, w.cols), np.int32)
    cls = oracle.AdamRows if per_row else oracle.Adam
    opt = cls(host_p0, lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
              mode=w.mode, m=m, v=v, last_step=ls)
    coords = 0
    steps = 0
    t_canon = 0.0
    t0 = time.perf_counter()
    for ids, grads in batches:
        tc = time.perf_counter()
        keys, sums, _ = oracle.coo_from_lookups(ids, grads, w.rows)
        ro, ci, cv = oracle.csr_from_coo(keys, sums, w.rows, w.cols, w.rows, w.cols)
        t_canon += time.perf_counter() - tc
        opt.step_csr(ro, ci, cv)
        coords += keys.size * w.cols
        steps += 1
        if steps >= 2 and time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": coords / dt / 1e9, "unit": "G touched coords/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {steps} steps of the same workload (whole step: canonicalise, CSR, "
                      f"update; {coords} touched coords in {dt:.2f} s, one thread)",
            "canonicalise_s": t_canon, "update_s": dt - t_canon,
            "host": {"cpu": cpu_model(), "nproc": os.cpu_count()}}


def kernel_label(op: str, lpr: int, iters: int, one_call: bool, src: str) -> str:
    if one_call:
        return f"k_step_lookups<{op}, {lpr}, {iters}> (tile combine + update + CSR blocks)"
    return f"k_update_rows<{op}, {src}, {lpr}, {iters}>"


def lanes_per_row(cols: int) -> int:
    """Lanes the update kernels give one full row (16-byte vectors, as the library)."""
    nvec = (cols + 3) // 4
    return 4 if nvec <= 4 else 16 if nvec <= 16 else 32 if nvec <= 32 else 64


def timed_passes(torch, stream, K, W, step, L, ev_count_per_step=None):
    """The timed pass (value) and the update launch's per-step durations: K steps
    queued behind a bounded spin, events around the region and the library's
    pair on each update launch."""
    ev = HipEvents(2 + 2 * K)
    cycles = calibrate_sleep(torch, stream, hold_ms=2.0 + 0.5 * K)
    log(f"timed {K} steps (queued behind a {cycles}-cycle spin)")
    torch.cuda._sleep(cycles)
    ev.record(0, stream)
    for k, s in enumerate(range(W, W + K)):
        L.set_step_events(ev.ev[2 + 2 * k], ev.ev[3 + 2 * k])
        step(s)
    L.set_step_events()
    ev.record(1, stream)
    torch.cuda.synchronize()
    import numpy as np

    total_ms = ev.ms(0, 1)
    upd = np.array([ev.ms(2 + 2 * k, 3 + 2 * k) for k in range(K)])
    ev.close()
    return total_ms, upd, cycles


def breakdown_pass(torch, stream, K, W, calls, step, L, cycles, one_call):
    """The same K inputs again, every call bracketed by events and the update
    launch by the hook's pair (not part of the value)."""
    import numpy as np

    E = len(calls) + 3  # events per step: before each call, after the last, the hook's two
    bev = HipEvents(E * K)
    torch.cuda._sleep(cycles)
    for k, s in enumerate(range(W, W + K)):
        L.set_step_events(bev.ev[E * k + E - 2], bev.ev[E * k + E - 1])
        step(s, bev, E * k)
    L.set_step_events()
    torch.cuda.synchronize()
    breakdown = {}
    for c, (name, _) in enumerate(calls):
        breakdown[name] = pcts(np.array([bev.ms(E * k + c, E * k + c + 1) for k in range(K)]))
    breakdown["update_launch"] = pcts(
        np.array([bev.ms(E * k + E - 2, E * k + E - 1) for k in range(K)]))
    if one_call:
        # the canonicalisation kernels of the one call, before its last launch
        breakdown["before_update_launch"] = pcts(
            np.array([bev.ms(E * k, E * k + E - 2) for k in range(K)]))
    breakdown["step"] = pcts(np.array([bev.ms(E * k, E * k + len(calls)) for k in range(K)]))
    bev.close()
    return breakdown


def cold_passes(torch, K, W, step, L):
    """The update launch with the last-level cache evicted before every step, two
    ways: a 512 MB buffer written (its dirty lines are written back while the
    step runs, as after a training step's other work) and the same buffer only
    read (clean lines, so the launch's own traffic alone).  Not part of the value."""
    import numpy as np

    scrub = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    out = {}
    for kind in ("written", "read"):
        log(f"cold pass (512 MB {kind} between steps)")
        cev = HipEvents(2 * K)
        for k, s in enumerate(range(W, W + K)):
            if kind == "written":
                scrub.fill_(float(k))
            else:
                torch.sum(scrub, dim=0, keepdim=True, out=sink)
            L.set_step_events(cev.ev[2 * k], cev.ev[2 * k + 1])
            step(s)
        L.set_step_events()
        torch.cuda.synchronize()
        out[kind] = np.array([cev.ms(2 * k, 2 * k + 1) for k in range(K)])
        cev.close()
    del scrub
    return out["written"], out["read"]


def roofline_block(upd, upd_cold, upd_clean, upd_bytes, coords, copy_gbs, traffic, kernel):
    achieved = float((upd_bytes / (upd * 1e-3)).mean() / 1e9)

    def regime(x):
        a = float((upd_bytes / (x * 1e-3)).mean() / 1e9)
        return {"achieved": a, "frac": a / HBM_PEAK_GBS,
                "traffic_GBs": None if traffic is None else traffic / (x.mean() * 1e-3) / 1e9,
                "mean_us": float(x.mean() * 1e3), "us": pcts(x)}

    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_GBs": None if traffic is None else traffic / (upd.mean() * 1e-3) / 1e9,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled)",
            "algorithmic_bytes_per_launch": float(upd_bytes.mean()),
            "kernel": kernel,
            "mean_us": float(upd.mean() * 1e3), "us": pcts(upd),
            "coords_per_s_G": float((coords / (upd * 1e-3)).mean() / 1e9),
            "device_copy_GBs": copy_gbs,
            "frac_of_device_copy": achieved / copy_gbs,
            "cold": regime(upd_cold), "cold_clean": regime(upd_clean)}


def traffic_for(name: str, form: str):
    # the three-call step's update launch is the two-call step's, on the same CSR
    t = TRAFFIC.get((name, "two_calls" if form == "separate_calls" else form))
    if t is None or sources_sha256() != t["sources_sha256"]:
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def result_head(w, K, W, total_ms, coords_total, metric):
    return {
        "metric": metric,
        "value": coords_total / (total_ms * 1e-3) / 1e9,
        "unit": "G touched coords/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": total_ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
    }


def run_lookups(args, cfg: int) -> dict:
    import numpy as np
    import torch

    import lazy_optimizer_step_amd as L
    import synth

    w = synth.WORKLOADS[cfg]
    if args.scrambled:
        w = w.scaled(name=w.name + "_scrambled", scramble=SCRAMBLE)
    R, Cc, n = w.rows, w.cols, w.n_lookups
    K, W = args.steps, args.warmup
    h = w.hyper

    log(f"initial table {R}x{Cc} float32 (N(0, {w.init_std}))")
    host_p0 = synth.init_params(w)
    per_row = args.last_step_per_row
    akw = dict(lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"], mode=w.mode,
               last_step_per_row=per_row)
    if args.host_state:
        log("table and state in mapped pinned host memory")
        opt = L.SparseAdam.host_resident(host_p0, **akw)
    else:
        opt = L.SparseAdam(torch.from_numpy(host_p0).to("cuda"), **akw)
    params = opt.params
    log(f"inputs of {W + K} steps ({n} lookups each)")
    batches = synth.lookups_many(w, range(W + K))
    ids_d = [torch.from_numpy(i).to("cuda") for i, _ in batches]
    grads_d = [torch.from_numpy(g).to("cuda") for _, g in batches]

    keys = torch.empty(n, dtype=torch.int64, device="cuda")
    sums = torch.empty((n, Cc), dtype=torch.float32, device="cuda")
    counts = torch.empty(n, dtype=torch.int32, device="cuda")
    nuniq = torch.zeros(W + K, dtype=torch.int64, device="cuda")
    ws = torch.empty(L.sparse_opt_workspace_size(n, Cc, R), dtype=torch.uint8, device="cuda")
    row_offsets = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    col_indices = torch.empty(n * Cc, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def canon(s: int) -> None:
        L.coo_from_lookups(ids_d[s], grads_d[s], R, out_keys=keys, out_vals=sums,
                           out_counts=counts, d_nunique=nuniq[s:s + 1], workspace=ws,
                           stream=stream)

    def csr(s: int):
        coo = L.CooGradient(keys, sums, dim=R, width=Cc, nnz=n, d_nnz=nuniq[s:s + 1])
        return L.csr_from_coo(coo, R, Cc, row_offsets=row_offsets, col_indices=col_indices,
                              copy_values=False, stream=stream)

    def lookups_csr(s: int):
        return L.csr_from_lookups(ids_d[s], grads_d[s], R, out_keys=keys, out_vals=sums,
                                  out_counts=counts, d_nunique=nuniq[s:s + 1],
                                  row_offsets=row_offsets, col_indices=col_indices,
                                  workspace=ws, stream=stream)[0]

    def fused(s: int) -> None:
        opt.step_lookups(ids_d[s], grads_d[s], out_keys=keys, out_vals=sums, out_counts=counts,
                         d_nunique=nuniq[s:s + 1], row_offsets=row_offsets,
                         col_indices=col_indices, workspace=ws, stream=stream)

    def adam(g) -> None:
        opt.step(g, stream=stream)

    # The calls of one step, named for the breakdown; each takes the step
    # index, or (the step call) the gradient the previous call returned.
    if args.separate_calls:
        calls = [("coo_from_lookups", canon), ("csr_from_coo", csr), ("sparse_adam_step", adam)]
    elif args.two_calls:
        calls = [("csr_from_lookups", lookups_csr), ("sparse_adam_step", adam)]
    else:
        calls = [("sparse_step_from_lookups", fused)]
    one_call = len(calls) == 1

    def step(s: int, ev=None, base: int = 0) -> None:
        """One step; with ev, event base + c is recorded before call c and
        base + len(calls) after the last."""
        g = None
        for c, (name, f) in enumerate(calls):
            if ev is not None:
                ev.record(base + c, stream)
            g = f(g) if f is adam else f(s)
        if ev is not None:
            ev.record(base + len(calls), stream)

    log(f"warmup {W} steps")
    for s in range(W):
        step(s)
    torch.cuda.synchronize()

    total_ms, upd, cycles = timed_passes(torch, stream, K, W, step, L)
    breakdown = breakdown_pass(torch, stream, K, W, calls, step, L, cycles, one_call)
    upd_cold, upd_clean = cold_passes(torch, K, W, step, L)
    copy_gbs = device_copy_gbs(torch, stream)

    # Forward gather (not part of the value): read_rows of each step's lookups.
    gathered = torch.empty((n, Cc), dtype=torch.float32, device="cuda")
    rev = HipEvents(2 * K)
    torch.cuda._sleep(cycles)
    for k, s in enumerate(range(W, W + K)):
        rev.record(2 * k, stream)
        L.read_rows(params, ids_d[s], out=gathered, stream=stream)
        rev.record(2 * k + 1, stream)
    torch.cuda.synchronize()
    rr = np.array([rev.ms(2 * k, 2 * k + 1) for k in range(K)])
    rev.close()
    rr_bytes = n * (8 + 2 * 4 * Cc)

    U = nuniq.cpu().numpy()[W:]
    coords = U * Cc
    dormancy = w.mode == "dormancy"
    # Lazy mode writes last_step but does not read it: 4 B less per coordinate
    # (per row with one last_step per row)
    if per_row:
        upd_bytes = BYTES_PER_COORD_ROW_LS * U * Cc + (BYTES_PER_ROW_ROW_LS - 4 * (not dormancy)) * U
    else:
        upd_bytes = (BYTES_PER_COORD - 4 * (not dormancy)) * U * Cc + BYTES_PER_ROW * U
    if one_call and not args.host_state:
        # the same launch also writes the CSR's row_offsets and col_indices
        # (with the state in host memory those bytes stay in HBM, off the
        # host link that bounds the launch, and are left out)
        upd_bytes = upd_bytes + (CSR_BYTES_PER_COORD * U * Cc + CSR_BYTES_PER_ROW * U
                                 + CSR_BYTES_PER_TABLE_ROW * (R + 1) + 4 * (R // 8192 + 1))
    form = "one_call" if one_call else ("two_calls" if args.two_calls else "separate_calls")
    traffic = None
    if not per_row and not args.host_state and not args.scrambled:
        traffic = traffic_for(w.name, form)
    op = (f"AdamOp<{'DormancyDecay' if dormancy else 'Lazy'}, no decay, "
          + ("last_step per row" if per_row else "last_step per coordinate") + ">")
    lpr = lanes_per_row(Cc)
    kernel = kernel_label(op, lpr, 1 if lpr == 4 else 2, one_call, "SrcCsrTouched")

    metric = METRIC if cfg == 3 else METRIC.replace("10M x 128 table", f"{R // 10**6}M x {Cc} table")
    result = result_head(w, K, W, total_ms, int(coords.sum()), metric)
    result["config"] = {"workload": w.name, "rows": R, "cols": Cc, "lookups_per_step": n,
                        "zipf_s": w.zipf_s, "mode": w.mode,
                        "state": "p,m,v float32 + last_step int32 per "
                                 + ("row" if per_row else "coordinate")
                                 + (", in mapped pinned host memory" if args.host_state
                                    else ", in HBM"),
                        "mean_unique_rows": float(U.mean()),
                        "calls": " + ".join(c for c, _ in calls)}
    result["roofline"] = roofline_block(upd, upd_cold, upd_clean, upd_bytes, coords, copy_gbs,
                                        traffic, kernel)
    result["breakdown_us"] = breakdown
    result["read_rows"] = {"us": pcts(rr), "lookups": n,
                           "achieved_GBs": float((rr_bytes / (rr * 1e-3)).mean() / 1e9),
                           "bytes_per_lookup": 8 + 2 * 4 * Cc}
    if args.host_state:
        # The state crosses the host link, not HBM: the roofline that bounds the
        # update is the link's, measured here with plain pinned copies.
        link = host_link_gbs(torch, stream)
        rf = result["roofline"]
        rf["bound"] = "host link"
        rf["peak"] = link["host_to_device"] + link["device_to_host"]
        rf["frac"] = rf["achieved"] / rf["peak"]
        for regime in ("cold", "cold_clean"):
            rf[regime]["frac"] = rf[regime]["achieved"] / rf["peak"]
        rf["host_link_copy_GBs"] = link
        rf["peak_note"] = "sum of the measured pinned copy rates, each direction"
    if args.cpu_seconds > 0:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, host_p0, batches, args.cpu_seconds, per_row)
    return result


# Partial rows: algorithmic bytes per nonzero of the update (SGD with momentum:
# read p, b, g and write p, b; Adam DormancyDecay: read p, m, v, last_step, g and
# write p, m, v, last_step), plus its column index; the update kernel without a
# touched-row list reads row_offsets over every table row (4 B per row, plus one).
PARTIAL_BYTES_PER_NNZ = {"sgd": 20, "adam": 36}
PARTIAL_COL_BYTES = 4


def cpu_baseline_partial(w, kind, host_p0, entries, budget_s: float):
    """The oracle, as it stands, on the first steps of the partial-row workload
    (COO -> CSR, then the step) until the time budget is spent; single thread."""
    import oracle

    import numpy as np

    h = w.hyper
    zeros = lambda dt=np.float32: np.zeros((w.rows, w.cols), dt)  # pages mapped lazily
    if kind == "sgd":
        opt = oracle.Sgd(host_p0, lr=h["lr"], momentum=h["momentum"],
                         weight_decay=h["weight_decay"], b=zeros())
    else:
        opt = oracle.Adam(host_p0, lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                          mode="dormancy", m=zeros(), v=zeros(), last_step=zeros(np.int32))
    nnz = 0
    steps = 0
    t_canon = 0.0
    t0 = time.perf_counter()
    # the steps' inputs in turn, again from the first once all are used, until
    # the budget is spent
    for k in range(1 << 30):
        er, ec, ev = entries[k % len(entries)]
        tc = time.perf_counter()
        lin = er * w.cols + ec
        ro, ci, cv = oracle.csr_from_coo(lin, ev, w.rows * w.cols, 1, w.rows, w.cols)
        t_canon += time.perf_counter() - tc
        opt.step_csr(ro, ci, cv)
        nnz += lin.size
        steps += 1
        if steps >= 2 and time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nnz / dt / 1e9, "unit": "G touched coords/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} steps of the same workload, its first {len(entries)} inputs in "
                      f"turn (COO -> CSR, then the step; {nnz} nonzeros in {dt:.2f} s, one thread)",
            "canonicalise_s": t_canon, "update_s": dt - t_canon,
            "host": {"cpu": cpu_model(), "nproc": os.cpu_count()}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        return ""


def run_partial(args, kind: str) -> dict:
    import numpy as np
    import torch

    import lazy_optimizer_step_amd as L
    import synth

    w = synth.WORKLOADS[4] if kind == "sgd" else synth.WORKLOAD_4_ADAM
    R, Cc = w.rows, w.cols
    K, W = args.steps, args.warmup
    h = w.hyper
    log(f"initial table {R}x{Cc} float32 (N(0, {w.init_std}))")
    host_p0 = synth.init_params(w)
    p_d = torch.from_numpy(host_p0).to("cuda")
    if kind == "sgd":
        opt = L.SparseSgd(p_d, lr=h["lr"], momentum=h["momentum"], weight_decay=h["weight_decay"])
    else:
        opt = L.SparseAdam(p_d, lr=h["lr"], beta1=h["beta1"], beta2=h["beta2"], eps=h["eps"],
                           mode="dormancy")
    log(f"inputs of {W + K} steps ({w.n_rows_touched} rows of {w.col_min}-{w.col_max} columns)")
    entries = synth.partial_rows_many(w, range(W + K))
    lin_d = [torch.from_numpy(er * Cc + ec).to("cuda") for er, ec, _ in entries]
    val_d = [torch.from_numpy(ev).to("cuda") for _, _, ev in entries]
    nnz = np.array([x.numel() for x in lin_d])
    row_offsets = torch.empty(R + 1, dtype=torch.int32, device="cuda")
    col_indices = torch.empty(int(nnz.max()), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def to_csr(s: int):
        coo = L.CooGradient(lin_d[s], val_d[s], dim=R * Cc, width=1)
        return L.csr_from_coo(coo, R, Cc, row_offsets=row_offsets, col_indices=col_indices,
                              copy_values=False, stream=stream)

    def upd(g) -> None:
        opt.step(g, stream=stream)

    step_name = "sparse_sgd_step" if kind == "sgd" else "sparse_adam_step"
    calls = [("csr_from_coo", to_csr), (step_name, upd)]

    def step(s: int, ev=None, base: int = 0) -> None:
        g = None
        for c, (name, f) in enumerate(calls):
            if ev is not None:
                ev.record(base + c, stream)
            g = f(g) if f is upd else f(s)
        if ev is not None:
            ev.record(base + len(calls), stream)

    log(f"warmup {W} steps")
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    total_ms, upd_ms, cycles = timed_passes(torch, stream, K, W, step, L)
    breakdown = breakdown_pass(torch, stream, K, W, calls, step, L, cycles, False)
    upd_cold, upd_clean = cold_passes(torch, K, W, step, L)
    copy_gbs = device_copy_gbs(torch, stream)

    nz = nnz[W:]
    upd_bytes = (PARTIAL_BYTES_PER_NNZ[kind] + PARTIAL_COL_BYTES) * nz + 4 * (R + 1)
    op = "SgdOp<momentum>" if kind == "sgd" else "AdamOp<DormancyDecay, no decay, last_step per coordinate>"
    kernel = f"k_update_csr_scan<{op}>"
    metric = METRIC.replace("10M x 128 table", f"2M x {Cc} table, partial rows")
    result = result_head(w, K, W, total_ms, int(nz.sum()), metric)
    result["config"] = {"workload": w.name, "rows": R, "cols": Cc,
                        "rows_per_step": w.n_rows_touched,
                        "cols_per_row": [w.col_min, w.col_max],
                        "optimizer": kind if kind == "sgd" else "adam dormancy",
                        "state": ("p, momentum float32" if kind == "sgd"
                                  else "p,m,v float32 + last_step int32 per coordinate")
                                 + ", in HBM",
                        "mean_nnz": float(nz.mean()),
                        "calls": " + ".join(c for c, _ in calls)}
    result["roofline"] = roofline_block(upd_ms, upd_cold, upd_clean, upd_bytes, nz, copy_gbs,
                                        traffic_for(w.name, "two_calls"), kernel)
    result["breakdown_us"] = breakdown
    if args.cpu_seconds > 0:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline_partial(w, kind, host_p0, entries, args.cpu_seconds)
    return result


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the sparse step is built and timed on a single "
              "MI355X; run it with --gpus 1", file=sys.stderr, flush=True)
        return 2

    import torch

    if args.copy_probe:
        copy_probe(args.warmup + args.steps)
        return 0

    cfg, kind = WORKLOAD_CHOICES[args.workload]
    if kind is not None and (args.two_calls or args.separate_calls or args.last_step_per_row
                             or args.scrambled or args.host_state):
        print("the partial-row workloads take none of --two-calls, --separate-calls, "
              "--last-step-per-row, --scrambled, --host-state", file=sys.stderr, flush=True)
        return 2
    torch.cuda.set_device(0)
    if kind is not None:
        result = run_partial(args, kind)
    else:
        result = run_lookups(args, cfg)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
