"""ctypes view of the C ABI in include/sparse_opt.h (argument marshalling only).

torch is imported first so that its HIP runtime is the one the library binds
to (both carry the soname libamdhip64.so.7); the library itself must exist,
built in-tree for gfx950: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (loads the process's HIP runtime before the library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparseopt.so")

OK, EINVAL, ERANGE, ENOTCANON, ESHAPE, ENONFINITE, EOVERFLOW, EWORKSPACE, EDEVICE, ENOMEM = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
ERROR_NAMES = {OK: "OK", EINVAL: "EINVAL", ERANGE: "ERANGE", ENOTCANON: "ENOTCANON",
               ESHAPE: "ESHAPE", ENONFINITE: "ENONFINITE", EOVERFLOW: "EOVERFLOW",
               EWORKSPACE: "EWORKSPACE", EDEVICE: "EDEVICE", ENOMEM: "ENOMEM"}

TRUSTED, VALIDATE = 0, 1
KIND_ADAM, KIND_SGD = 0, 1
MODE_LAZY, MODE_DORMANCY = 0, 1
WD_L2, WD_DECOUPLED = 0, 1
FORMAT_COO, FORMAT_CSR = 0, 1


class AdamConfig(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("mode", C.c_int32), ("weight_decay", C.c_double),
                ("weight_decay_mode", C.c_int32), ("last_step_per_row", C.c_int32)]


class SgdConfig(C.Structure):
    _fields_ = [("lr", C.c_double), ("momentum", C.c_double), ("weight_decay", C.c_double)]


class Coo(C.Structure):
    _fields_ = [("dim", C.c_int64), ("width", C.c_int64), ("nnz", C.c_int64),
                ("d_nnz", C.c_void_p), ("indices", C.c_void_p), ("values", C.c_void_p)]


class Csr(C.Structure):
    _fields_ = [("rows", C.c_int64), ("cols", C.c_int64), ("row_offsets", C.c_void_p),
                ("col_indices", C.c_void_p), ("values", C.c_void_p),
                ("touched_rows", C.c_void_p), ("n_touched", C.c_int64),
                ("d_n_touched", C.c_void_p)]


class Grad(C.Structure):
    _fields_ = [("format", C.c_int32), ("coo", Coo), ("csr", Csr)]


class SparseOptError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with lazy_optimizer_step_amd.build.build() "
                "(hipcc, gfx950); there is no CPU fallback")
        L = C.CDLL(LIB_PATH)
        P, I64, U32, I32 = C.c_void_p, C.c_int64, C.c_uint32, C.c_int32
        L.sparse_opt_create.argtypes = [C.POINTER(P), I32, P, I64, I64, P, P, P, P]
        L.sparse_opt_create.restype = C.c_int
        L.sparse_opt_destroy.argtypes = [P]
        L.sparse_opt_destroy.restype = None
        L.sparse_opt_get_step.argtypes = [P]
        L.sparse_opt_get_step.restype = I64
        L.sparse_opt_set_step.argtypes = [P, I64]
        L.sparse_opt_set_step.restype = C.c_int
        L.sparse_opt_last_error.argtypes = []
        L.sparse_opt_last_error.restype = C.c_char_p
        L.sparse_opt_workspace_size.argtypes = [I64, I64, I64, C.POINTER(C.c_size_t)]
        L.sparse_opt_workspace_size.restype = C.c_int
        L.coo_from_lookups.argtypes = [P, P, I64, I64, I64, P, P, P, P, P, C.c_size_t, P, U32]
        L.coo_from_lookups.restype = C.c_int
        L.csr_from_coo.argtypes = [C.POINTER(Coo), I64, I64, P, P, P, P, P, P, U32]
        L.csr_from_coo.restype = C.c_int
        L.csr_from_lookups.argtypes = [P, P, I64, I64, I64, P, P, P, P, P, P, P, C.c_size_t, P,
                                       U32]
        L.csr_from_lookups.restype = C.c_int
        L.csr_to_coo.argtypes = [C.POINTER(Csr), P, P, P, U32]
        L.csr_to_coo.restype = C.c_int
        L.sparse_adam_step.argtypes = [P, C.POINTER(Grad), P, U32]
        L.sparse_adam_step.restype = C.c_int
        L.sparse_sgd_step.argtypes = [P, C.POINTER(Grad), P, U32]
        L.read_rows.restype = C.c_int
        L.read_rows.argtypes = [P, I64, I64, P, I64, P, P, U32]
        L.sparse_opt_host_alloc.restype = C.c_int
        L.sparse_opt_host_alloc.argtypes = [C.c_size_t, C.POINTER(P), C.POINTER(P)]
        L.sparse_opt_host_free.restype = None
        L.sparse_opt_host_free.argtypes = [P]
        L.sparse_opt_host_device_pointer.restype = C.c_int
        L.sparse_opt_host_device_pointer.argtypes = [P, C.POINTER(P)]
        L.sparse_sgd_step.restype = C.c_int
        L.sparse_step_from_lookups.argtypes = [P, P, P, I64, P, P, P, P, P, P, P, C.c_size_t, P,
                                               U32]
        L.sparse_step_from_lookups.restype = C.c_int
        L.sparse_step_from_lookups_noalloc.argtypes = [P, P, P, I64, P, P, P, P, P, P, P, U32]
        L.sparse_step_from_lookups_noalloc.restype = C.c_int
        L.sparse_opt_set_step_events.argtypes = [P, P]
        L.sparse_opt_set_step_events.restype = C.c_int
        _lib = L
    return _lib


def check(rc: int) -> None:
    if rc != OK:
        raise SparseOptError(rc, lib().sparse_opt_last_error().decode(errors="replace"))


EXPORTED = ("sparse_opt_create", "sparse_opt_destroy", "sparse_opt_get_step", "sparse_opt_set_step",
            "sparse_opt_last_error", "sparse_opt_workspace_size", "coo_from_lookups",
            "csr_from_coo", "csr_from_lookups", "csr_to_coo", "sparse_adam_step",
            "sparse_sgd_step", "sparse_step_from_lookups", "sparse_step_from_lookups_noalloc",
            "sparse_opt_set_step_events", "read_rows",
            "sparse_opt_host_alloc", "sparse_opt_host_free", "sparse_opt_host_device_pointer")
