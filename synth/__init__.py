"""Seeded synthetic inputs for the sparse / lazy optimizer step.

This module is shared by the tests, the benchmark and the smoke check.  It
draws lookups, gradient rows, initial tables and partial-row gradients with
numpy's PCG64; it holds none of the optimizer's arithmetic (no sorting into
canonical form, no duplicate sums, no moment or parameter updates).

Every stream is keyed by ``SeedSequence([SEED, cfg, stream, index])``:

* stream 0: initial parameter values, one chunk of ``INIT_CHUNK_ROWS`` rows per
  index, so any row can be regenerated on its own chunk;
* stream 1: lookup row ids (or 1-D indices), index = step;
* stream 2: gradient values, index = step;
* stream 3: column subsets of partial-row gradients, index = step.

"N(0, x)" in a workload description means a normal with standard deviation x.
Bounded Zipf(s) over R rows gives rank k in 1..R probability k^-s / H(R, s) and
maps it to row id k-1, so row 0 is the hottest row; a workload with scramble = A
(coprime to R) maps rank k to row (k-1)*A mod R instead.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 20261202
INIT_CHUNK_ROWS = 1 << 20

STREAM_INIT = 0
STREAM_IDS = 1
STREAM_VALS = 2
STREAM_COLS = 3


def rng(cfg: int, stream: int, index: int) -> np.random.Generator:
    """Generator for one (workload, stream, index) triple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, cfg, stream, index])))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload.

    kind: "coo1d"   - 1-D vector, unique sorted indices each step;
          "lookups" - a table fed raw per-lookup row ids with duplicates;
          "csr"     - a table fed partial-row gradients.
    """

    cfg: int
    name: str
    kind: str
    rows: int
    cols: int
    steps: int
    optimizer: str            # "adam" or "sgd"
    mode: str = "dormancy"    # Adam: "lazy" or "dormancy"
    init_std: float = 0.01
    grad_std: float = 0.01
    n_lookups: int = 0        # "lookups": lookups per step
    zipf_s: float = 0.0       # "lookups": Zipf exponent
    scramble: int = 0         # "lookups": 0, or A coprime to rows: rank k -> row (k-1)*A mod rows
    n_indices: int = 0        # "coo1d": unique indices per step
    n_rows_touched: int = 0   # "csr": rows per step
    col_min: int = 0          # "csr": columns per touched row, inclusive range
    col_max: int = 0
    hyper: dict = field(default_factory=dict)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


ADAM_DEFAULTS = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.0}
SGD_CFG4 = {"lr": 0.05, "momentum": 0.9, "weight_decay": 1e-4}

WORKLOADS = {
    1: Workload(1, "vec4096_coo64_dormancy", "coo1d", rows=4096, cols=1, steps=20, optimizer="adam",
                mode="dormancy", init_std=1.0, grad_std=1.0, n_indices=64, hyper=ADAM_DEFAULTS),
    2: Workload(2, "table1Mx64_zipf1.1_lazy", "lookups", rows=1_000_000, cols=64, steps=100,
                optimizer="adam", mode="lazy", n_lookups=8192, zipf_s=1.1, hyper=ADAM_DEFAULTS),
    3: Workload(3, "table10Mx128_zipf1.05_dormancy", "lookups", rows=10_000_000, cols=128, steps=200,
                optimizer="adam", mode="dormancy", n_lookups=65536, zipf_s=1.05, hyper=ADAM_DEFAULTS),
    4: Workload(4, "table2Mx256_csr16-64_sgd", "csr", rows=2_000_000, cols=256, steps=100,
                optimizer="sgd", init_std=0.01, grad_std=1.0, n_rows_touched=16384, col_min=16,
                col_max=64, hyper=SGD_CFG4),
    5: Workload(5, "table50Mx128_zipf1.2_dormancy", "lookups", rows=50_000_000, cols=128, steps=50,
                optimizer="adam", mode="dormancy", n_lookups=262144, zipf_s=1.2, hyper=ADAM_DEFAULTS),
}
# The partial-row workload also runs Adam in DormancyDecay mode from fresh state.
WORKLOAD_4_ADAM = WORKLOADS[4].scaled(name="table2Mx256_csr16-64_dormancy", optimizer="adam",
                                      mode="dormancy", hyper=ADAM_DEFAULTS)


# --------------------------------------------------------------------------
# Initial tables
# --------------------------------------------------------------------------

def init_chunk(cfg: int, chunk: int, rows: int, cols: int, std: float) -> np.ndarray:
    """Initial values of rows [chunk*INIT_CHUNK_ROWS, ...) as float32 [nrows, cols]."""
    r0 = chunk * INIT_CHUNK_ROWS
    nr = min(INIT_CHUNK_ROWS, rows - r0)
    out = np.empty((nr, cols), dtype=np.float32)
    rng(cfg, STREAM_INIT, chunk).standard_normal(out=out.reshape(-1), dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def init_params(w: Workload, out: np.ndarray | None = None) -> np.ndarray:
    """The whole initial table, float32 [rows, cols] (cols == 1 gives [rows, 1])."""
    if out is None:
        out = np.empty((w.rows, w.cols), dtype=np.float32)
    nchunks = (w.rows + INIT_CHUNK_ROWS - 1) // INIT_CHUNK_ROWS

    def fill(c):
        r0 = c * INIT_CHUNK_ROWS
        blk = init_chunk(w.cfg, c, w.rows, w.cols, w.init_std)
        out[r0:r0 + blk.shape[0]] = blk

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    return out


def init_rows(w: Workload, row_ids: np.ndarray) -> np.ndarray:
    """Initial values of the given rows only (regenerates just their chunks)."""
    row_ids = np.asarray(row_ids, dtype=np.int64)
    out = np.empty((row_ids.size, w.cols), dtype=np.float32)
    chunks = np.unique(row_ids // INIT_CHUNK_ROWS)
    for c in chunks:
        blk = init_chunk(w.cfg, int(c), w.rows, w.cols, w.init_std)
        sel = np.nonzero(row_ids // INIT_CHUNK_ROWS == c)[0]
        out[sel] = blk[row_ids[sel] - c * INIT_CHUNK_ROWS]
    return out


# --------------------------------------------------------------------------
# Bounded Zipf lookups
# --------------------------------------------------------------------------

_ZIPF_CACHE: dict = {}


def zipf_cdf(rows: int, s: float) -> np.ndarray:
    """Cumulative weights sum_{k<=i+1} k^-s as float64 [rows] (cached)."""
    key = (rows, s)
    if key not in _ZIPF_CACHE:
        k = np.arange(1, rows + 1, dtype=np.float64)
        np.power(k, -s, out=k)
        np.cumsum(k, out=k)
        _ZIPF_CACHE.clear()
        _ZIPF_CACHE[key] = k
    return _ZIPF_CACHE[key]


def zipf_rows(g: np.random.Generator, rows: int, s: float, n: int) -> np.ndarray:
    """n row ids in [0, rows) from bounded Zipf(s) by inverse CDF."""
    cdf = zipf_cdf(rows, s)
    u = g.random(n) * cdf[-1]
    r = np.searchsorted(cdf, u, side="right")
    np.minimum(r, rows - 1, out=r)
    return r.astype(np.int64)


def lookups(w: Workload, step: int, n: int | None = None):
    """Raw lookups of one step: (ids int64[n], grads float32[n, cols])."""
    n = w.n_lookups if n is None else n
    ids = zipf_rows(rng(w.cfg, STREAM_IDS, step), w.rows, w.zipf_s, n)
    if w.scramble:
        # the same frequencies, the hot rows spread over the table
        ids = (ids * np.int64(w.scramble)) % np.int64(w.rows)
    grads = np.empty((n, w.cols), dtype=np.float32)
    rng(w.cfg, STREAM_VALS, step).standard_normal(out=grads.reshape(-1), dtype=np.float32)
    if w.grad_std != 1.0:
        grads *= np.float32(w.grad_std)
    return ids, grads


def lookups_many(w: Workload, steps, n: int | None = None):
    """lookups() for several steps, generated on a thread pool."""
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda s: lookups(w, s, n), steps))


# --------------------------------------------------------------------------
# 1-D coordinate lists and partial-row gradients
# --------------------------------------------------------------------------

def coo1d(w: Workload, step: int):
    """Sorted unique indices (uniform, without replacement) and N(0, grad_std) values."""
    g = rng(w.cfg, STREAM_IDS, step)
    idx = np.sort(g.choice(w.rows, size=w.n_indices, replace=False)).astype(np.int64)
    vals = rng(w.cfg, STREAM_VALS, step).standard_normal(w.n_indices, dtype=np.float32)
    if w.grad_std != 1.0:
        vals *= np.float32(w.grad_std)
    return idx, vals


def partial_rows(w: Workload, step: int):
    """A partial-row gradient as (row, column, value) entries in row-major order.

    n_rows_touched distinct rows (uniform, without replacement); each row gets
    k ~ U{col_min..col_max} distinct columns in ascending order; values
    N(0, grad_std).  Returns (rows int64[nnz], cols int32[nnz], values float32[nnz]).
    """
    g = rng(w.cfg, STREAM_IDS, step)
    touched = np.sort(g.choice(w.rows, size=w.n_rows_touched, replace=False)).astype(np.int64)
    gc = rng(w.cfg, STREAM_COLS, step)
    ks = gc.integers(w.col_min, w.col_max + 1, size=touched.size)
    # Column subsets: give every column a random key and keep the k smallest keys
    # of each row (a uniform k-subset); col_max candidates are found by partition.
    keys = gc.random((touched.size, w.cols))
    kmax = min(w.col_max, w.cols)
    cand = np.argpartition(keys, kmax - 1, axis=1)[:, :kmax] if kmax < w.cols else \
        np.broadcast_to(np.arange(w.cols), keys.shape).copy()
    order = np.take_along_axis(cand, np.argsort(np.take_along_axis(keys, cand, axis=1), axis=1), axis=1)
    take = np.arange(kmax)[None, :] < ks[:, None]
    cols = np.sort(np.where(take, order, w.cols), axis=1)
    mask = cols < w.cols
    ent_rows = np.broadcast_to(touched[:, None], cols.shape)[mask].astype(np.int64)
    ent_cols = cols[mask].astype(np.int32)
    vals = rng(w.cfg, STREAM_VALS, step).standard_normal(ent_cols.size, dtype=np.float32)
    if w.grad_std != 1.0:
        vals *= np.float32(w.grad_std)
    return ent_rows, ent_cols, vals


def partial_rows_many(w: Workload, steps):
    """partial_rows() for several steps, generated on a thread pool."""
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda s: partial_rows(w, s), steps))
