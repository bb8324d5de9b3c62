"""CPU-side checks of the C ABI: the library loads, exports every entry point
declared in include/*.h, and rejects bad host-side arguments without touching
a device."""
import ctypes as C
import glob
import os
import re
import subprocess
import sys

import pytest

import lazy_optimizer_step_amd as L
from lazy_optimizer_step_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^SPOPT_API\s+[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    lib = C.CDLL(_lib.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert names == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == names


def test_workspace_size():
    assert L.sparse_opt_workspace_size(65536, 128, 10_000_000) > 65536 * 16
    assert L.sparse_opt_workspace_size(0, 1, 1) >= 0
    for bad in [(-1, 1, 1), (10, 0, 5), (10, 1, 0), (1 << 30, 1, 1 << 40)]:
        with pytest.raises(L.SparseOptError) as e:
            L.sparse_opt_workspace_size(*bad)
        assert e.value.code == _lib.EINVAL


FAKE = 256  # a non-NULL address that create() stores but never dereferences


@pytest.mark.parametrize("cfg", [
    _lib.AdamConfig(1e-3, 1.0, 0.999, 1e-8, 1), _lib.AdamConfig(1e-3, 0.9, -0.1, 1e-8, 1),
    _lib.AdamConfig(1e-3, 0.9, 0.999, 0.0, 1), _lib.AdamConfig(-1.0, 0.9, 0.999, 1e-8, 1),
    _lib.AdamConfig(1e-3, 0.9, 0.999, 1e-8, 7),
    _lib.AdamConfig(1e-3, 0.9, 0.999, 1e-8, 1, -0.1, _lib.WD_L2),
    _lib.AdamConfig(1e-3, 0.9, 0.999, 1e-8, 1, float("nan"), _lib.WD_DECOUPLED),
    _lib.AdamConfig(1e-3, 0.9, 0.999, 1e-8, 1, 0.01, 5)])
def test_create_rejects_bad_adam_config(cfg):
    h = C.c_void_p()
    rc = _lib.lib().sparse_opt_create(C.byref(h), _lib.KIND_ADAM, C.byref(cfg), 10, 4, FAKE, FAKE,
                                      FAKE, FAKE)
    assert rc == _lib.EINVAL and not h.value
    assert _lib.lib().sparse_opt_last_error()


@pytest.mark.parametrize("cfg", [_lib.SgdConfig(-0.1, 0.9, 0.0), _lib.SgdConfig(0.1, 1.0, 0.0),
                                 _lib.SgdConfig(0.1, 0.5, -1e-4)])
def test_create_rejects_bad_sgd_config(cfg):
    h = C.c_void_p()
    rc = _lib.lib().sparse_opt_create(C.byref(h), _lib.KIND_SGD, C.byref(cfg), 10, 4, FAKE, FAKE,
                                      None, None)
    assert rc == _lib.EINVAL


def test_handle_step_counter_and_shape_errors():
    # An SGD handle needs no device memory of its own (an Adam handle uploads a
    # table of beta powers at creation), so this runs without a GPU.
    L_ = _lib.lib()
    h = C.c_void_p()
    cfg = _lib.SgdConfig(0.1, 0.9, 0.0)
    assert L_.sparse_opt_create(C.byref(h), _lib.KIND_SGD, C.byref(cfg), 10, 4, FAKE, FAKE, None,
                                None) == 0
    try:
        assert L_.sparse_opt_get_step(h) == 0
        assert L_.sparse_opt_set_step(h, 41) == 0 and L_.sparse_opt_get_step(h) == 41
        assert L_.sparse_opt_set_step(h, -1) == _lib.EINVAL
        assert L_.sparse_opt_set_step(h, 1 << 31) == _lib.EINVAL
        # Shape errors are found on the host, before any device work.
        g = _lib.Grad(_lib.FORMAT_COO, _lib.Coo(11, 4, 0, None, FAKE, FAKE), _lib.Csr())
        assert L_.sparse_sgd_step(h, C.byref(g), None, 0) == _lib.ESHAPE
        g = _lib.Grad(_lib.FORMAT_CSR, _lib.Coo(), _lib.Csr(10, 5, FAKE, None, FAKE, None, 0, None))
        assert L_.sparse_sgd_step(h, C.byref(g), None, 0) == _lib.ESHAPE
        g = _lib.Grad(9, _lib.Coo(), _lib.Csr())
        assert L_.sparse_sgd_step(h, C.byref(g), None, 0) == _lib.EINVAL
        assert L_.sparse_adam_step(h, C.byref(g), None, 0) == _lib.EINVAL   # wrong kind
        assert L_.sparse_opt_get_step(h) == 41
        assert L_.sparse_opt_set_step(h, (1 << 31) - 2) == 0
        g = _lib.Grad(_lib.FORMAT_COO, _lib.Coo(10, 4, 0, None, FAKE, FAKE), _lib.Csr())
        assert L_.sparse_sgd_step(h, C.byref(g), None, 0) == _lib.EINVAL   # t would hit 2^31
    finally:
        L_.sparse_opt_destroy(h)


def test_csr_from_lookups_host_errors():
    """Argument errors of the fused call are found before any device work."""
    f = _lib.lib().csr_from_lookups
    args = lambda n=10, rows=100, cols=4, ro=FAKE, ws=1 << 20: (
        FAKE, FAKE, n, rows, cols, FAKE, FAKE, FAKE, FAKE, ro, None, FAKE, ws, None, 0)
    assert f(*args(ro=None)) == _lib.EINVAL
    assert f(*args(rows=0)) == _lib.EINVAL
    assert f(*args(n=1 << 24, cols=128)) == _lib.EOVERFLOW      # n * cols >= 2^31
    assert f(*args(n=1 << 30, cols=1)) == _lib.EOVERFLOW        # n >= 2^30
    assert f(*args(ws=16)) == _lib.EWORKSPACE


def test_step_from_lookups_host_errors():
    """The step from raw lookups checks its handle before any device work; the
    timing hook takes two events or none."""
    L_ = _lib.lib()
    f = L_.sparse_step_from_lookups
    assert f(None, FAKE, FAKE, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None,
             0) == _lib.EINVAL
    h = C.c_void_p()
    cfg = _lib.SgdConfig(0.1, 0.0, 0.0)
    assert L_.sparse_opt_create(C.byref(h), _lib.KIND_SGD, C.byref(cfg), 100, 4, FAKE, None, None,
                                None) == 0
    try:
        args = lambda n=10, ro=FAKE, ws=1 << 20: (h, FAKE, FAKE, n, FAKE, FAKE, FAKE, FAKE, ro,
                                                  None, FAKE, ws, None, 0)
        assert f(*args(ro=None)) == _lib.EINVAL
        assert b"sparse_step_from_lookups" in L_.sparse_opt_last_error()
        assert f(*args(n=1 << 30)) == _lib.EOVERFLOW        # n * cols >= 2^31
        assert f(*args(ws=16)) == _lib.EWORKSPACE
        assert b"sparse_step_from_lookups" in L_.sparse_opt_last_error()
        assert L_.sparse_opt_get_step(h) == 0               # no step taken
        assert L_.sparse_opt_set_step(h, (1 << 31) - 2) == 0
        assert f(*args()) == _lib.EINVAL                    # t would reach 2^31
    finally:
        L_.sparse_opt_destroy(h)
    ev = L_.sparse_opt_set_step_events
    assert ev(FAKE, None) == _lib.EINVAL
    assert ev(None, FAKE) == _lib.EINVAL
    assert ev(None, None) == _lib.OK


def test_step_from_lookups_noalloc_host_errors():
    """The allocation-free step refuses, before any device work: a NULL handle,
    validated calls, and lookups whose workspace exceeds its fixed 16 MiB."""
    L_ = _lib.lib()
    f = L_.sparse_step_from_lookups_noalloc
    assert f(None, FAKE, FAKE, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0) == _lib.EINVAL
    h = C.c_void_p()
    cfg = _lib.SgdConfig(0.1, 0.0, 0.0)
    rows, cols = 1000, 1024
    assert L_.sparse_opt_create(C.byref(h), _lib.KIND_SGD, C.byref(cfg), rows, cols, FAKE, None,
                                None, None) == 0
    try:
        args = lambda n, flags=0: (h, FAKE, FAKE, n, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                   flags)
        assert f(*args(10, _lib.VALIDATE)) == _lib.EINVAL
        assert b"trusted" in L_.sparse_opt_last_error()
        assert f(*args(-1)) == _lib.EINVAL
        big = 200_000
        assert L.sparse_opt_workspace_size(big, cols, rows) > 16 << 20
        assert f(*args(big)) == _lib.EWORKSPACE
        assert b"16777216" in L_.sparse_opt_last_error()
        assert L_.sparse_opt_get_step(h) == 0
    finally:
        L_.sparse_opt_destroy(h)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_header_is_plain_c_and_callable_from_c(tmp_path):
    """include/sparse_opt.h compiles as C99 and C++11 with warnings as errors, and
    a C program linked against the library gets the workspace size and the
    argument errors that need no device."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(ROOT, "include")
    hdr = os.path.join(inc, "sparse_opt.h")
    for cmd in ([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                 "-x", "c", hdr],
                ["g++", "-std=c++11", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++", hdr]):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    src = tmp_path / "use.c"
    src.write_text(r'''
#include <stdio.h>
#include "sparse_opt.h"
int main(void) {
    size_t a = 0, b = 0;
    if (sparse_opt_workspace_size(65536, 128, 10000000, &a) != SPOPT_OK) return 1;
    if (sparse_opt_workspace_size(1024, 128, 10000000, &b) != SPOPT_OK) return 2;
    if (!(a > b && b > 0)) return 3;
    if (sparse_opt_workspace_size(-1, 128, 10, &a) != SPOPT_EINVAL) return 4;
    if (csr_from_lookups(0, 0, 10, 0, 4, 0, 0, 0, 0, 0, 0, 0, 0, 0, SPOPT_TRUSTED) != SPOPT_EINVAL)
        return 5;
    printf("%s\n", sparse_opt_last_error());
    return 0;
}
''')
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = tmp_path / "use"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", str(src), "-I", inc, "-L", libdir,
                        "-lsparseopt", f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "csr_from_lookups" in r.stdout
