"""CPU oracle of the sparse / lazy optimizer step (TEST INFRASTRUCTURE).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``oracle.c`` (plain C, double arithmetic) with
numpy arrays and keeps the global step counter ``t`` the way the optimizer
page defines it: the number of step calls so far, incremented before the
update, so the first call runs with t = 1.

It imports nothing from the HIP library and the HIP library imports nothing
from it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, ERANGE, ENOTCANON, ESHAPE, ENONFINITE, EOVERFLOW, EWORKSPACE, EDEVICE, ENOMEM = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
ERROR_NAMES = {OK: "OK", EINVAL: "EINVAL", ERANGE: "ERANGE", ENOTCANON: "ENOTCANON",
               ESHAPE: "ESHAPE", ENONFINITE: "ENONFINITE", EOVERFLOW: "EOVERFLOW",
               EWORKSPACE: "EWORKSPACE", EDEVICE: "EDEVICE", ENOMEM: "ENOMEM"}
MODE_LAZY, MODE_DORMANCY = 0, 1
WD_L2, WD_DECOUPLED = 0, 1
CHECK_FINITE = 1


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERROR_NAMES.get(code, code)}")
        self.code = code


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no intrinsics)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _AdamCfg(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("mode", C.c_int), ("weight_decay", C.c_double),
                ("wd_mode", C.c_int)]


def _adam_cfg(lr, beta1, beta2, eps, mode, weight_decay, weight_decay_mode):
    if weight_decay_mode not in ("l2", "decoupled"):
        raise ValueError(f"weight_decay_mode {weight_decay_mode!r}: 'l2' or 'decoupled'")
    return _AdamCfg(lr, beta1, beta2, eps, MODE_DORMANCY if mode == "dormancy" else MODE_LAZY,
                    weight_decay, WD_DECOUPLED if weight_decay_mode == "decoupled" else WD_L2)


class _SgdCfg(C.Structure):
    _fields_ = [("lr", C.c_double), ("momentum", C.c_double), ("weight_decay", C.c_double)]


_lib = None
# A test that plants mistakes in a copy of oracle.c (tests/test_oracle_mutations.py)
# points this at the copy's library, in a child process of its own.
_LIB_ENV = "SPOPT_ORACLE_LIB"


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(os.environ.get(_LIB_ENV) or build())
        P = C.c_void_p
        I64 = C.c_int64
        L.orc_coo_from_lookups.argtypes = [P, P, I64, I64, I64, P, P, P, P, C.c_int]
        L.orc_csr_from_coo.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, P]
        L.orc_csr_to_coo.argtypes = [P, P, P, I64, I64, P, P]
        L.orc_adam_coo_f32.argtypes = [P, P, P, P, I64, I64, P, P, I64, I64, P, C.c_int]
        L.orc_adam_csr_f32.argtypes = [P, P, P, P, I64, I64, P, P, P, I64, P, C.c_int]
        L.orc_adam_rows_csr_f32.argtypes = [P, P, P, P, I64, I64, P, P, P, I64, P, C.c_int]
        L.orc_read_rows.argtypes = [P, I64, I64, P, I64, P, C.c_int]
        L.orc_adam_coo_f64.argtypes = [P, P, P, P, I64, P, P, I64, I64, P]
        L.orc_sgd_coo_f32.argtypes = [P, P, I64, I64, P, P, I64, P, C.c_int]
        L.orc_sgd_csr_f32.argtypes = [P, P, I64, I64, P, P, P, P, C.c_int]
        L.orc_sgd_coo_f64.argtypes = [P, P, I64, P, P, I64, P]
        for f in ("orc_coo_from_lookups", "orc_csr_from_coo", "orc_csr_to_coo", "orc_adam_coo_f32",
                  "orc_adam_csr_f32", "orc_adam_coo_f64", "orc_sgd_coo_f32", "orc_sgd_csr_f32",
                  "orc_sgd_coo_f64"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _arr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != OK:
        raise OracleError(rc, what)


# --------------------------------------------------------------------------
# Canonicalisation and conversions
# --------------------------------------------------------------------------

def coo_from_lookups(ids, vals, key_space: int, check_finite: bool = False):
    """Raw lookups -> (keys int64[U], vals float32[U, width], counts int32[U])."""
    ids = _arr(ids, np.int64).reshape(-1)
    n = ids.size
    vals = _arr(vals, np.float32).reshape(n, -1) if n else np.zeros((0, 1), np.float32)
    width = vals.shape[1] if vals.ndim == 2 and vals.shape[1] > 0 else 1
    keys = np.empty(max(n, 1), np.int64)
    out = np.empty((max(n, 1), width), np.float32)
    counts = np.empty(max(n, 1), np.int32)
    u = C.c_int64(0)
    rc = lib().orc_coo_from_lookups(_p(ids), _p(vals), n, width, key_space, _p(keys), _p(out),
                                    _p(counts), C.byref(u), CHECK_FINITE if check_finite else 0)
    _check(rc, "coo_from_lookups")
    U = u.value
    return keys[:U].copy(), out[:U].copy(), counts[:U].copy()


def csr_from_coo(idx, vals, dim: int, width: int, rows: int, cols: int):
    """Canonical COO -> (row_offsets int32[rows+1], col_indices int32[nnz], values float32[nnz])."""
    idx = _arr(idx, np.int64).reshape(-1)
    vals = _arr(vals, np.float32).reshape(-1)
    total = idx.size * width
    ro = np.empty(rows + 1, np.int32)
    ci = np.empty(max(total, 1), np.int32)
    ov = np.empty(max(total, 1), np.float32)
    rc = lib().orc_csr_from_coo(_p(idx), _p(vals), idx.size, dim, width, rows, cols, _p(ro),
                                _p(ci), _p(ov))
    _check(rc, "csr_from_coo")
    return ro, ci[:total].copy(), ov[:total].copy()


def csr_to_coo(row_offsets, col_indices, vals, rows: int, cols: int):
    """CSR -> (linear indices int64[nnz], values float32[nnz])."""
    ro = _arr(row_offsets, np.int32)
    ci = _arr(col_indices, np.int32)
    vals = _arr(vals, np.float32)
    nnz = int(ro[rows])
    idx = np.empty(max(nnz, 1), np.int64)
    ov = np.empty(max(nnz, 1), np.float32)
    rc = lib().orc_csr_to_coo(_p(ro), _p(ci), _p(vals), rows, cols, _p(idx), _p(ov))
    _check(rc, "csr_to_coo")
    return idx[:nnz].copy(), ov[:nnz].copy()


# --------------------------------------------------------------------------
# Optimizers (float32 state, double arithmetic)
# --------------------------------------------------------------------------

def read_rows(params, idx, check_finite=False):
    """Forward gather of table rows (duplicates allowed)."""
    params = _arr(params, np.float32)
    rows = params.shape[0]
    cols = params.shape[1] if params.ndim == 2 else 1
    idx = _arr(idx, np.int64).reshape(-1)
    out = np.zeros((idx.size, cols), np.float32)
    rc = lib().orc_read_rows(_p(params), rows, cols, _p(idx), idx.size, _p(out),
                             CHECK_FINITE if check_finite else 0)
    _check(rc, "read_rows")
    return out


class Adam:
    """Sparse / lazy Adam over a dense (rows x cols) float32 state.

    State arrays may be supplied (e.g. lazily allocated zero pages for a huge
    table of which only a few rows are ever touched)."""

    def __init__(self, params, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, mode="dormancy",
                 m=None, v=None, last_step=None, weight_decay=0.0, weight_decay_mode="l2"):
        self.p = params
        self.rows = params.shape[0]
        self.cols = params.shape[1] if params.ndim == 2 else 1
        self.m = np.zeros_like(params) if m is None else m
        self.v = np.zeros_like(params) if v is None else v
        self.ls = np.zeros(params.shape, np.int32) if last_step is None else last_step
        self.cfg = _adam_cfg(lr, beta1, beta2, eps, mode, weight_decay, weight_decay_mode)
        self.t = 0

    def _state(self):
        return _p(self.p), _p(self.m), _p(self.v), _p(self.ls)

    def step_coo(self, idx, vals, width: int = 1, check_finite=False):
        """COO gradient; width == 1 indexes the flattened view, width == cols gives full rows."""
        idx = _arr(idx, np.int64).reshape(-1)
        vals = _arr(vals, np.float32).reshape(-1)
        dim = self.p.size // width
        rc = lib().orc_adam_coo_f32(*self._state(), dim, width, _p(idx), _p(vals), idx.size,
                                    self.t + 1, C.byref(self.cfg),
                                    CHECK_FINITE if check_finite else 0)
        _check(rc, "adam_coo")
        self.t += 1

    def step_csr(self, row_offsets, col_indices, vals, check_finite=False):
        ro = _arr(row_offsets, np.int32)
        ci = _arr(col_indices, np.int32)
        vals = _arr(vals, np.float32)
        rc = lib().orc_adam_csr_f32(*self._state(), self.rows, self.cols, _p(ro), _p(ci),
                                    _p(vals), self.t + 1, C.byref(self.cfg),
                                    CHECK_FINITE if check_finite else 0)
        _check(rc, "adam_csr")
        self.t += 1


class AdamRows(Adam):
    """Sparse / lazy Adam with one last_step per row (full-row gradients only)."""

    def __init__(self, params, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, mode="dormancy",
                 m=None, v=None, last_step=None, weight_decay=0.0, weight_decay_mode="l2"):
        rows = params.shape[0]
        super().__init__(params, lr, beta1, beta2, eps, mode, m, v,
                         np.zeros(rows, np.int32) if last_step is None else last_step,
                         weight_decay, weight_decay_mode)

    def step_coo(self, idx, vals, width: int = 1, check_finite=False):
        """Full-row COO (width == cols): keys are row ids."""
        if width != self.cols:
            raise ValueError("a row-granular table takes full-row gradients only")
        idx = _arr(idx, np.int64).reshape(-1)
        vals = _arr(vals, np.float32).reshape(-1)
        ro, ci, cv = csr_from_coo(idx, vals, self.rows, self.cols, self.rows, self.cols)
        self.step_csr(ro, ci, cv, check_finite)

    def step_csr(self, row_offsets, col_indices, vals, check_finite=False):
        ro = _arr(row_offsets, np.int32)
        ci = _arr(col_indices, np.int32)
        vals = _arr(vals, np.float32)
        rc = lib().orc_adam_rows_csr_f32(*self._state(), self.rows, self.cols, _p(ro), _p(ci),
                                         _p(vals), self.t + 1, C.byref(self.cfg),
                                         CHECK_FINITE if check_finite else 0)
        _check(rc, "adam_rows_csr")
        self.t += 1


class Sgd:
    """Sparse SGD (coupled weight decay, lazy heavy-ball momentum), float32 state."""

    def __init__(self, params, lr, momentum=0.0, weight_decay=0.0, b=None):
        self.p = params
        self.rows = params.shape[0]
        self.cols = params.shape[1] if params.ndim == 2 else 1
        self.b = (np.zeros_like(params) if b is None else b) if momentum != 0.0 else None
        self.cfg = _SgdCfg(lr, momentum, weight_decay)
        self.t = 0

    def step_coo(self, idx, vals, width: int = 1, check_finite=False):
        idx = _arr(idx, np.int64).reshape(-1)
        vals = _arr(vals, np.float32).reshape(-1)
        dim = self.p.size // width
        rc = lib().orc_sgd_coo_f32(_p(self.p), _p(self.b), dim, width, _p(idx), _p(vals),
                                   idx.size, C.byref(self.cfg), CHECK_FINITE if check_finite else 0)
        _check(rc, "sgd_coo")
        self.t += 1

    def step_csr(self, row_offsets, col_indices, vals, check_finite=False):
        ro = _arr(row_offsets, np.int32)
        ci = _arr(col_indices, np.int32)
        vals = _arr(vals, np.float32)
        rc = lib().orc_sgd_csr_f32(_p(self.p), _p(self.b), self.rows, self.cols, _p(ro), _p(ci),
                                   _p(vals), C.byref(self.cfg), CHECK_FINITE if check_finite else 0)
        _check(rc, "sgd_csr")
        self.t += 1


# --------------------------------------------------------------------------
# Double-storage variants (used by the pins to check the formulas exactly)
# --------------------------------------------------------------------------

class Adam64:
    """1-D sparse / lazy Adam with double state."""

    def __init__(self, params, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, mode="dormancy",
                 weight_decay=0.0, weight_decay_mode="l2"):
        self.p = np.array(params, dtype=np.float64)
        self.m = np.zeros_like(self.p)
        self.v = np.zeros_like(self.p)
        self.ls = np.zeros(self.p.shape, np.int32)
        self.cfg = _adam_cfg(lr, beta1, beta2, eps, mode, weight_decay, weight_decay_mode)
        self.t = 0

    def step(self, idx, vals):
        idx = _arr(idx, np.int64)
        vals = _arr(vals, np.float64)
        rc = lib().orc_adam_coo_f64(_p(self.p), _p(self.m), _p(self.v), _p(self.ls), self.p.size,
                                    _p(idx), _p(vals), idx.size, self.t + 1, C.byref(self.cfg))
        _check(rc, "adam_coo_f64")
        self.t += 1


class Sgd64:
    """1-D sparse SGD with double state."""

    def __init__(self, params, lr, momentum=0.0, weight_decay=0.0):
        self.p = np.array(params, dtype=np.float64)
        self.b = np.zeros_like(self.p)
        self.cfg = _SgdCfg(lr, momentum, weight_decay)

    def step(self, idx, vals):
        idx = _arr(idx, np.int64)
        vals = _arr(vals, np.float64)
        rc = lib().orc_sgd_coo_f64(_p(self.p), _p(self.b), self.p.size, _p(idx), _p(vals),
                                   idx.size, C.byref(self.cfg))
        _check(rc, "sgd_coo_f64")
