"""MI355X-native sparse / lazy optimizer step (Python binding of libsparseopt.so).

The functions below carry the C ABI's names (include/sparse_opt.h) and only
marshal arguments: they check dtypes, devices and contiguity, allocate
outputs (and the canonicalisation's workspace) with torch when none are
given, and call the library on torch's current stream, or on ``stream=``
(then what they allocate is allocated on that stream).  All arithmetic runs
in the library's HIP kernels.

Pages followed (see the header for the full contract): the optirs_gpu
sparse_optimizer module page (COO/CSR gradients, sparse SGD, Lazy and
DormancyDecay Adam with global-step bias correction) and, where it is silent,
the DiskSparseAdam README (duplicates summed and sorted, validated inputs).
"""
from __future__ import annotations

import contextlib
import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib
from ._lib import (FORMAT_COO, FORMAT_CSR, KIND_ADAM, KIND_SGD, MODE_DORMANCY, MODE_LAZY, TRUSTED,
                   VALIDATE, SparseOptError, check)

__all__ = ["coo_from_lookups", "csr_from_coo", "csr_from_lookups", "csr_to_coo",
           "sparse_opt_workspace_size",
           "sparse_opt_create", "sparse_adam_step", "sparse_sgd_step", "sparse_step_from_lookups",
           "sparse_step_from_lookups_noalloc",
           "set_step_events",
           "CooGradient",
           "CsrGradient", "SparseAdam", "SparseSgd", "SparseOptError", "TRUSTED", "VALIDATE",
           "read_rows", "HostArray"]


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _alloc_on(stream):
    """Context in which torch allocates on the stream the call's kernels run on.
    The caching allocator then gives memory this call allocates (its internal
    workspace, dropped on return) to no other stream until the work queued on
    `stream` has finished with it."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        if int(stream) == torch.cuda.current_stream().cuda_stream:
            return contextlib.nullcontext()
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


class HostArray:
    """Pinned host memory mapped into the device's address space, for state of
    tables larger than device memory.  ``numpy()`` is the host view (current
    after the stream is synchronised); the library's kernels use the device
    address.  Zero-filled at allocation; freed when the object goes."""

    _NP = {torch.float32: np.float32, torch.int32: np.int32}

    def __init__(self, shape, dtype=torch.float32):
        import ctypes as C

        self.shape = tuple(int(x) for x in shape)
        self.dtype = dtype
        n = 1
        for x in self.shape:
            n *= x
        self._numel = n
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        h, d = C.c_void_p(), C.c_void_p()
        check(_lib.lib().sparse_opt_host_alloc(max(nbytes, 1), C.byref(h), C.byref(d)))
        self._host, self._dev = h.value, d.value
        ct = C.c_float if dtype == torch.float32 else C.c_int32
        self._array = np.ctypeslib.as_array((ct * max(n, 1)).from_address(self._host))[:n]
        self._array = self._array.reshape(self.shape)

    def numpy(self) -> np.ndarray:
        return self._array

    def numel(self) -> int:
        return self._numel

    def data_ptr(self) -> int:
        return self._dev

    def __del__(self):
        host = getattr(self, "_host", None)
        if host:
            self._array = None
            _lib.lib().sparse_opt_host_free(host)
            self._host = None


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t, dtype, name, numel=None):
    if isinstance(t, HostArray):
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if numel is not None and t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t


def _flags(validate: bool) -> int:
    return VALIDATE if validate else TRUSTED


# ---------------------------------------------------------------------------
# Gradients
# ---------------------------------------------------------------------------

@dataclass
class CooGradient:
    """COO gradient over a dense (dim x width) object; see spopt_coo.

    nnz is the entry count, or an upper bound when d_nnz (a device int64[1])
    holds the count."""
    indices: torch.Tensor
    values: torch.Tensor
    dim: int
    width: int = 1
    nnz: int | None = None
    d_nnz: torch.Tensor | None = None

    def _c(self) -> _lib.Coo:
        nnz = self.indices.numel() if self.nnz is None else self.nnz
        _need(self.indices, torch.int64, "indices", nnz)
        _need(self.values, torch.float32, "values", nnz * self.width)
        if self.d_nnz is not None:
            _need(self.d_nnz, torch.int64, "d_nnz", 1)
        return _lib.Coo(self.dim, self.width, nnz, _ptr(self.d_nnz), _ptr(self.indices),
                        _ptr(self.values))


@dataclass
class CsrGradient:
    """CSR gradient of shape rows x cols; see spopt_csr."""
    row_offsets: torch.Tensor
    col_indices: torch.Tensor | None
    values: torch.Tensor
    rows: int
    cols: int
    touched_rows: torch.Tensor | None = None
    n_touched: int | None = None
    d_n_touched: torch.Tensor | None = None

    def _c(self) -> _lib.Csr:
        _need(self.row_offsets, torch.int32, "row_offsets", self.rows + 1)
        if self.col_indices is not None:
            _need(self.col_indices, torch.int32, "col_indices")
        _need(self.values, torch.float32, "values")
        n_touched = 0
        if self.touched_rows is not None:
            _need(self.touched_rows, torch.int64, "touched_rows")
            n_touched = self.touched_rows.numel() if self.n_touched is None else self.n_touched
        if self.d_n_touched is not None:
            _need(self.d_n_touched, torch.int64, "d_n_touched", 1)
        return _lib.Csr(self.rows, self.cols, _ptr(self.row_offsets), _ptr(self.col_indices),
                        _ptr(self.values), _ptr(self.touched_rows), n_touched,
                        _ptr(self.d_n_touched))


def _grad(g) -> _lib.Grad:
    if isinstance(g, CooGradient):
        return _lib.Grad(FORMAT_COO, g._c(), _lib.Csr())
    if isinstance(g, CsrGradient):
        return _lib.Grad(FORMAT_CSR, _lib.Coo(), g._c())
    raise TypeError("gradient must be a CooGradient or a CsrGradient")


# ---------------------------------------------------------------------------
# Canonicalisation and conversions
# ---------------------------------------------------------------------------

def sparse_opt_workspace_size(n: int, width: int, key_space: int) -> int:
    out = C.c_size_t(0)
    check(_lib.lib().sparse_opt_workspace_size(n, width, key_space, C.byref(out)))
    return out.value


def coo_from_lookups(ids: torch.Tensor, vals: torch.Tensor, key_space: int, *, out_keys=None,
                     out_vals=None, out_counts=None, d_nunique=None, workspace=None,
                     stream=None, validate: bool = False):
    """Raw lookups -> canonical COO.  Returns (keys, vals, counts, d_nunique), all
    sized by the lookup count n; the first U = d_nunique entries are the result."""
    with _alloc_on(stream):
        return _coo_from_lookups(ids, vals, key_space, out_keys, out_vals, out_counts, d_nunique,
                                 workspace, stream, validate)


def _coo_from_lookups(ids, vals, key_space, out_keys, out_vals, out_counts, d_nunique, workspace,
                      stream, validate):
    n = ids.numel()
    width = vals.numel() // n if n else (vals.shape[1] if vals.dim() == 2 else 1)
    dev = ids.device
    _need(ids, torch.int64, "ids")
    _need(vals, torch.float32, "vals", n * width)
    if out_keys is None:
        out_keys = torch.empty(max(n, 1), dtype=torch.int64, device=dev)
    if out_vals is None:
        out_vals = torch.empty((max(n, 1), width), dtype=torch.float32, device=dev)
    if out_counts is None:
        out_counts = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    if d_nunique is None:
        d_nunique = torch.empty(1, dtype=torch.int64, device=dev)
    need = sparse_opt_workspace_size(n, width, key_space)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(out_keys, torch.int64, "out_keys", n)
    _need(out_vals, torch.float32, "out_vals", n * width)
    _need(out_counts, torch.int32, "out_counts", n)
    _need(d_nunique, torch.int64, "d_nunique", 1)
    _need(workspace, torch.uint8, "workspace")
    check(_lib.lib().coo_from_lookups(_ptr(ids), _ptr(vals), n, width, key_space, _ptr(out_keys),
                                      _ptr(out_vals), _ptr(out_counts), _ptr(d_nunique),
                                      _ptr(workspace), workspace.numel(), _stream(stream),
                                      _flags(validate)))
    return out_keys, out_vals, out_counts, d_nunique


def csr_from_coo(coo: CooGradient, rows: int, cols: int, *, row_offsets=None, col_indices=None,
                 values=None, touched_rows=None, d_n_touched=None, want_col_indices=True,
                 copy_values=True, stream=None, validate: bool = False):
    """Canonical COO -> CSR.  Returns a CsrGradient.  For a full-row COO the touched
    rows are the COO's keys (no copy unless touched_rows is given), and values may
    alias the COO's (copy_values=False)."""
    with _alloc_on(stream):
        return _csr_from_coo(coo, rows, cols, row_offsets, col_indices, values, touched_rows,
                             d_n_touched, want_col_indices, copy_values, stream, validate)


def _csr_from_coo(coo, rows, cols, row_offsets, col_indices, values, touched_rows, d_n_touched,
                  want_col_indices, copy_values, stream, validate):
    c = coo._c()
    dev = coo.indices.device
    total = c.nnz * coo.width
    if row_offsets is None:
        row_offsets = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    _need(row_offsets, torch.int32, "row_offsets", rows + 1)
    full = coo.width == cols and coo.width > 1
    if col_indices is None and (want_col_indices or not full):
        col_indices = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
    if col_indices is not None:
        _need(col_indices, torch.int32, "col_indices", total)
    if values is None:
        values = torch.empty(max(total, 1), dtype=torch.float32, device=dev) if copy_values \
            else coo.values
    _need(values, torch.float32, "values", total)
    tr, dn = touched_rows, d_n_touched
    if full:
        if tr is None:
            tr = coo.indices
        if dn is None and coo.d_nnz is not None:
            dn = coo.d_nnz
    check(_lib.lib().csr_from_coo(C.byref(c), rows, cols, _ptr(row_offsets), _ptr(col_indices),
                                  _ptr(values), _ptr(tr) if full else None,
                                  _ptr(dn) if full else None, _stream(stream), _flags(validate)))
    return CsrGradient(row_offsets, col_indices, values, rows, cols,
                       touched_rows=tr if full else None,
                       n_touched=c.nnz if full else None, d_n_touched=dn if full else None)


def _lookup_outputs(ids, vals, rows, out_keys, out_vals, out_counts, d_nunique, row_offsets,
                    col_indices, want_col_indices, workspace):
    """Checks (and allocates what is not given of) the arrays of a call that
    takes raw lookups of full rows to the full-row CSR."""
    n = ids.numel()
    cols = vals.shape[1] if vals.dim() == 2 else (vals.numel() // n if n else 1)
    dev = ids.device
    _need(ids, torch.int64, "ids")
    _need(vals, torch.float32, "vals", n * cols)
    if out_keys is None:
        out_keys = torch.empty(max(n, 1), dtype=torch.int64, device=dev)
    if out_vals is None:
        out_vals = torch.empty((max(n, 1), cols), dtype=torch.float32, device=dev)
    if out_counts is None:
        out_counts = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    if d_nunique is None:
        d_nunique = torch.empty(1, dtype=torch.int64, device=dev)
    if row_offsets is None:
        row_offsets = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_indices is None and want_col_indices:
        col_indices = torch.empty(max(n * cols, 1), dtype=torch.int32, device=dev)
    need = sparse_opt_workspace_size(n, cols, rows)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(out_keys, torch.int64, "out_keys", n)
    _need(out_vals, torch.float32, "out_vals", n * cols)
    _need(out_counts, torch.int32, "out_counts", n)
    _need(d_nunique, torch.int64, "d_nunique", 1)
    _need(row_offsets, torch.int32, "row_offsets", rows + 1)
    if col_indices is not None:
        _need(col_indices, torch.int32, "col_indices", n * cols)
    _need(workspace, torch.uint8, "workspace")
    return n, cols, out_keys, out_vals, out_counts, d_nunique, row_offsets, col_indices, workspace


def csr_from_lookups(ids: torch.Tensor, vals: torch.Tensor, rows: int, *, out_keys=None,
                     out_vals=None, out_counts=None, d_nunique=None, row_offsets=None,
                     col_indices=None, want_col_indices=True, workspace=None, stream=None,
                     validate: bool = False):
    """Raw lookups of full table rows -> full-row CSR gradient in one call: the
    result of coo_from_lookups then csr_from_coo(copy_values=False), bit for bit.
    vals: (n, cols).  Returns (csr, counts, d_nunique): csr.touched_rows holds the
    distinct ids and csr.values their summed rows (first U = d_nunique entries)."""
    with _alloc_on(stream):
        (n, cols, out_keys, out_vals, out_counts, d_nunique, row_offsets, col_indices,
         workspace) = _lookup_outputs(ids, vals, rows, out_keys, out_vals, out_counts, d_nunique,
                                      row_offsets, col_indices, want_col_indices, workspace)
        check(_lib.lib().csr_from_lookups(_ptr(ids), _ptr(vals), n, rows, cols, _ptr(out_keys),
                                          _ptr(out_vals), _ptr(out_counts), _ptr(d_nunique),
                                          _ptr(row_offsets), _ptr(col_indices), _ptr(workspace),
                                          workspace.numel(), _stream(stream), _flags(validate)))
    csr = CsrGradient(row_offsets, col_indices, out_vals, rows, cols, touched_rows=out_keys,
                      n_touched=n, d_n_touched=d_nunique)
    return csr, out_counts, d_nunique


def sparse_step_from_lookups(h: "_Handle", ids: torch.Tensor, vals: torch.Tensor, *,
                             out_keys=None, out_vals=None, out_counts=None, d_nunique=None,
                             row_offsets=None, col_indices=None, want_col_indices=True,
                             workspace=None, stream=None, validate: bool = False):
    """Raw lookups of full rows -> one step of the handle's optimizer in one call:
    the outputs of csr_from_lookups and the table of the step on that CSR, bit for
    bit.  vals: (n, cols) with the handle's cols.  Returns (csr, counts,
    d_nunique) as csr_from_lookups."""
    n = ids.numel()
    if vals.numel() != n * h.cols or (vals.dim() == 2 and vals.shape[1] != h.cols):
        raise ValueError(f"vals: shape {tuple(vals.shape)}, the handle's table takes "
                         f"({n}, {h.cols})")
    vals = vals if vals.dim() == 2 else vals.view(n, h.cols)
    with _alloc_on(stream):
        (n, cols, out_keys, out_vals, out_counts, d_nunique, row_offsets, col_indices,
         workspace) = _lookup_outputs(ids, vals, h.rows, out_keys, out_vals, out_counts,
                                      d_nunique, row_offsets, col_indices, want_col_indices,
                                      workspace)
        check(h._L.sparse_step_from_lookups(h._h, _ptr(ids), _ptr(vals), n, _ptr(out_keys),
                                            _ptr(out_vals), _ptr(out_counts), _ptr(d_nunique),
                                            _ptr(row_offsets), _ptr(col_indices),
                                            _ptr(workspace), workspace.numel(), _stream(stream),
                                            _flags(validate)))
    csr = CsrGradient(row_offsets, col_indices, out_vals, h.rows, cols, touched_rows=out_keys,
                      n_touched=n, d_n_touched=d_nunique)
    return csr, out_counts, d_nunique


def sparse_step_from_lookups_noalloc(h: "_Handle", ids: torch.Tensor, vals: torch.Tensor, *,
                                     out_keys, out_vals, out_counts, d_nunique, row_offsets,
                                     col_indices=None, stream=None) -> None:
    """sparse_step_from_lookups for callers that cannot allocate: no workspace
    argument (the library's fixed device scratch serves instead) and nothing
    allocated here either, so every output must be given.  Trusted mode only;
    calls that overlap in time on one GPU race on the shared scratch."""
    n = ids.numel()
    _need(ids, torch.int64, "ids")
    _need(vals, torch.float32, "vals", n * h.cols)
    _need(out_keys, torch.int64, "out_keys", n)
    _need(out_vals, torch.float32, "out_vals", n * h.cols)
    _need(out_counts, torch.int32, "out_counts", n)
    _need(d_nunique, torch.int64, "d_nunique", 1)
    _need(row_offsets, torch.int32, "row_offsets", h.rows + 1)
    if col_indices is not None:
        _need(col_indices, torch.int32, "col_indices", n * h.cols)
    check(h._L.sparse_step_from_lookups_noalloc(h._h, _ptr(ids), _ptr(vals), n, _ptr(out_keys),
                                                _ptr(out_vals), _ptr(out_counts),
                                                _ptr(d_nunique), _ptr(row_offsets),
                                                _ptr(col_indices), _stream(stream), TRUSTED))


def csr_to_coo(csr: CsrGradient, *, out_indices=None, out_values=None, nnz: int | None = None,
               stream=None, validate: bool = False) -> CooGradient:
    """CSR -> COO over the flattened rows*cols view.  nnz (the entry count) is read
    from row_offsets with a host copy when not given."""
    c = csr._c()
    dev = csr.row_offsets.device
    if nnz is None:
        nnz = int(csr.row_offsets[csr.rows].item())
    with _alloc_on(stream):
        return _csr_to_coo(csr, c, dev, out_indices, out_values, nnz, stream, validate)


def _csr_to_coo(csr, c, dev, out_indices, out_values, nnz, stream, validate):
    if out_indices is None:
        out_indices = torch.empty(max(nnz, 1), dtype=torch.int64, device=dev)
    if out_values is None:
        out_values = torch.empty(max(nnz, 1), dtype=torch.float32, device=dev)
    _need(out_indices, torch.int64, "out_indices", nnz)
    _need(out_values, torch.float32, "out_values", nnz)
    check(_lib.lib().csr_to_coo(C.byref(c), _ptr(out_indices), _ptr(out_values), _stream(stream),
                                _flags(validate)))
    return CooGradient(out_indices, out_values, csr.rows * csr.cols, 1, nnz)


# ---------------------------------------------------------------------------
# Optimizer handles
# ---------------------------------------------------------------------------

class _Handle:
    def __init__(self, kind, cfg, rows, cols, p, m, v, ls):
        self.rows, self.cols = rows, cols
        self._h = C.c_void_p()
        check(_lib.lib().sparse_opt_create(C.byref(self._h), kind, C.byref(cfg), rows, cols,
                                           _ptr(p), _ptr(m), _ptr(v), _ptr(ls)))
        self._L = _lib.lib()

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._L.sparse_opt_destroy(h)
            self._h = None

    @property
    def step_count(self) -> int:
        return int(self._L.sparse_opt_get_step(self._h))

    def set_step(self, t: int) -> None:
        check(self._L.sparse_opt_set_step(self._h, t))


def sparse_opt_create(kind: int, config, rows: int, cols: int, params, m_or_momentum=None, v=None,
                      last_step=None) -> _Handle:
    n = rows * cols
    per_row = kind == KIND_ADAM and getattr(config, "last_step_per_row", 0) != 0
    _need(params, torch.float32, "params", n)
    for t, name, dt, size in ((m_or_momentum, "m_or_momentum", torch.float32, n),
                              (v, "v", torch.float32, n),
                              (last_step, "last_step", torch.int32, rows if per_row else n)):
        if t is not None:
            _need(t, dt, name, size)
    return _Handle(kind, config, rows, cols, params, m_or_momentum, v, last_step)


def sparse_adam_step(h: _Handle, grad, *, stream=None, validate: bool = False) -> None:
    g = _grad(grad)
    check(h._L.sparse_adam_step(h._h, C.byref(g), _stream(stream), _flags(validate)))


def sparse_sgd_step(h: _Handle, grad, *, stream=None, validate: bool = False) -> None:
    g = _grad(grad)
    check(h._L.sparse_sgd_step(h._h, C.byref(g), _stream(stream), _flags(validate)))


def set_step_events(begin=None, end=None) -> None:
    """Have the calling thread's step calls record the two HIP events (raw
    hipEvent_t handles, as ints or ctypes pointers) just before and just after
    the launch that updates the table; no arguments stop it."""
    check(_lib.lib().sparse_opt_set_step_events(begin, end))


def read_rows(params: torch.Tensor, indices: torch.Tensor, *, out=None, stream=None,
              validate: bool = False) -> torch.Tensor:
    """Forward gather: out[k] = params[indices[k]] (rows of a 2-D float32 table)."""
    rows = params.shape[0]
    cols = params.shape[1] if len(params.shape) == 2 else 1
    _need(params, torch.float32, "params", rows * cols)
    _need(indices, torch.int64, "indices")
    n = indices.numel()
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((n, cols), dtype=torch.float32, device=indices.device)
    _need(out, torch.float32, "out", n * cols)
    check(_lib.lib().read_rows(_ptr(params), rows, cols, _ptr(indices), n, _ptr(out),
                               _stream(stream), _flags(validate)))
    return out


class SparseAdam:
    """Sparse / lazy Adam over a (rows x cols) float32 table that this object
    allocates on the device (m = v = 0, last_step = 0)."""

    def __init__(self, params: torch.Tensor, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                 mode="dormancy", weight_decay=0.0, weight_decay_mode="l2",
                 last_step_per_row=False):
        self.params = params
        rows = params.shape[0]
        cols = params.shape[1] if params.dim() == 2 else 1
        self.m = torch.zeros_like(params)
        self.v = torch.zeros_like(params)
        shape = (rows,) if last_step_per_row else params.shape
        self.last_step = torch.zeros(shape, dtype=torch.int32, device=params.device)
        self._init_handle(rows, cols, lr=lr, beta1=beta1, beta2=beta2, eps=eps, mode=mode,
                          weight_decay=weight_decay, weight_decay_mode=weight_decay_mode,
                          last_step_per_row=last_step_per_row)

    def _init_handle(self, rows, cols, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                     mode="dormancy", weight_decay=0.0, weight_decay_mode="l2",
                     last_step_per_row=False):
        if weight_decay_mode not in ("l2", "decoupled"):
            raise ValueError(f"weight_decay_mode {weight_decay_mode!r}: 'l2' or 'decoupled'")
        self.rows, self.cols = rows, cols
        cfg = _lib.AdamConfig(lr, beta1, beta2, eps,
                              MODE_DORMANCY if mode == "dormancy" else MODE_LAZY, weight_decay,
                              _lib.WD_DECOUPLED if weight_decay_mode == "decoupled" else _lib.WD_L2,
                              1 if last_step_per_row else 0)
        self.handle = sparse_opt_create(KIND_ADAM, cfg, rows, cols, self.params, self.m, self.v,
                                        self.last_step)

    @property
    def t(self) -> int:
        return self.handle.step_count

    def step(self, grad, *, stream=None, validate=False) -> None:
        sparse_adam_step(self.handle, grad, stream=stream, validate=validate)

    def step_lookups(self, ids: torch.Tensor, vals: torch.Tensor, **kw):
        """One step from raw lookups of full rows (ids (n,), vals (n, cols));
        keywords and result as sparse_step_from_lookups."""
        return sparse_step_from_lookups(self.handle, ids, vals, **kw)

    def read_rows(self, indices: torch.Tensor, *, out=None, stream=None, validate=False):
        """The current rows of the table for a batch of lookups (forward pass)."""
        return read_rows(self.params, indices, out=out, stream=stream, validate=validate)

    @classmethod
    def host_resident(cls, params_init, **kw) -> "SparseAdam":
        """Adam whose table and state live in mapped pinned host memory: only the
        touched rows cross the host link on each step.  params_init: a (rows x
        cols) array of initial values, copied in.  Gradients and the
        canonicalisation stay in device memory."""
        p0 = np.ascontiguousarray(np.asarray(params_init, dtype=np.float32))
        if p0.ndim == 1:
            p0 = p0.reshape(-1, 1)
        self = cls.__new__(cls)
        rows, cols = p0.shape
        per_row = kw.get("last_step_per_row", False)
        self.params = HostArray((rows, cols))
        self.params.numpy()[...] = p0
        self.m = HostArray((rows, cols))
        self.v = HostArray((rows, cols))
        self.last_step = HostArray((rows,) if per_row else (rows, cols), torch.int32)
        self._init_handle(rows, cols, **kw)
        return self


class SparseSgd:
    """Sparse SGD (coupled weight decay, lazy momentum) over a float32 table."""

    def __init__(self, params: torch.Tensor, lr, momentum=0.0, weight_decay=0.0):
        self.params = params
        self.rows = params.shape[0]
        self.cols = params.shape[1] if params.dim() == 2 else 1
        self.momentum_buf = torch.zeros_like(params) if momentum != 0.0 else None
        cfg = _lib.SgdConfig(lr, momentum, weight_decay)
        self.handle = sparse_opt_create(KIND_SGD, cfg, self.rows, self.cols, params,
                                        self.momentum_buf)

    @property
    def t(self) -> int:
        return self.handle.step_count

    def step(self, grad, *, stream=None, validate=False) -> None:
        sparse_sgd_step(self.handle, grad, stream=stream, validate=validate)

    def step_lookups(self, ids: torch.Tensor, vals: torch.Tensor, **kw):
        """One step from raw lookups of full rows; as SparseAdam.step_lookups."""
        return sparse_step_from_lookups(self.handle, ids, vals, **kw)
