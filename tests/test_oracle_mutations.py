"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (a dropped term, a
wrong sign or index, a swapped operand, a missing store), builds the copy
with gcc, and runs the oracle's CPU pins (tests/test_oracle_*.py) against it
in a child process: at least one pin must fail.  The committed oracle is
never changed; nothing here touches the HIP library.

Where each mistake departs from the pages:
  page "optirs_gpu::sparse_optimizer" (docs.rs), sections Sparse SGD (coupled
  weight decay, lazy heavy-ball momentum on touched coordinates),
  LazyAdamMode::Lazy / LazyAdamMode::DormancyDecay (one decay per touch /
  beta^gap, global-t bias correction, eps after the root, last_step = t), and
  Sparse gradient representations (CSR row_offsets and columns, row*cols+col);
  the DiskSparseAdam README, Safe Duplicate Aggregation & Sorted I/O
  (duplicates summed, multiplicity), Explicit Weight Decay Semantics, and the
  API reference's read_rows.
"""
import glob
import os
from concurrent.futures import ThreadPoolExecutor
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement).  Each text occurs exactly once.
MUTATIONS = [
    ("sgd_f32_momentum_not_stored",
     "if (b != NULL && c->momentum != 0.0) b[i] = (float)bb;", "(void)bb;"),
    ("sgd_weight_decay_sign",
     "double gg = g + c->weight_decay * *p;", "double gg = g - c->weight_decay * *p;"),
    ("sgd_dampened_momentum",
     "*b = c->momentum * *b + gg;", "*b = c->momentum * *b + (1.0 - c->momentum) * gg;"),
    ("sgd_csr_column_by_entry",
     "sgd_f32(p, b, r * cols + col_indices[j], (double)g[j], cfg);",
     "sgd_f32(p, b, r * cols + (j - row_offsets[r]), (double)g[j], cfg);"),
    ("adam_gap_off_by_one",
     "double gap = (double)(t - (int64_t)*ls);", "double gap = (double)(t - (int64_t)*ls - 1);"),
    ("adam_lazy_decays_by_gap",
     "if (c->mode == ORC_MODE_DORMANCY) {\n        double gap",
     "if (c->mode == c->mode) {\n        double gap"),
    ("adam_eps_inside_root",
     "(sqrt(v_hat) + c->eps)", "sqrt(v_hat + c->eps)"),
    ("adam_bias_correction_by_gap",
     "double m_hat = *m / (1.0 - pow(c->beta1, (double)t));",
     "double m_hat = *m / (1.0 - pow(c->beta1, (double)(t - (int64_t)*ls)));"),
    ("adam_second_moment_uses_beta1",
     "*v = d2 * *v + (1.0 - c->beta2) * (g * g);", "*v = d2 * *v + (1.0 - c->beta1) * (g * g);"),
    ("adam_last_step_not_t",
     "*ls = (int32_t)t;", "*ls = (int32_t)(t - 1);"),
    ("adam_f32_m_not_stored",
     "    m[i] = (float)mm;\n    v[i] = (float)vv;\n}", "    v[i] = (float)vv;\n}"),
    ("adam_l2_half",
     "g = g + c->weight_decay * p0;", "g = g + 0.5 * c->weight_decay * p0;"),
    ("adam_decoupled_uses_new_p",
     "*p = *p - (c->lr * c->weight_decay) * p0;", "*p = *p - (c->lr * c->weight_decay) * *p;"),
    ("adam_rows_last_step_not_t",
     "        ls[r] = (int32_t)t;", "        ls[r] = (int32_t)(t - 1);"),
    ("canon_count_plus_one",
     "out_counts[u] = (int32_t)(j - i);", "out_counts[u] = (int32_t)(j - i + 1);"),
    ("canon_sum_in_float",
     "acc[c] += (double)row[c];", "acc[c] = (double)(float)(acc[c] + (double)row[c]);"),
    ("canon_drops_first_duplicate",
     "for (int64_t c = 0; c < width; ++c) acc[c] = 0.0;\n        /* one run",
     "for (int64_t c = 0; c < width; ++c) acc[c] = -(double)vals[kp[i].pos * width + c];\n"
     "        /* one run"),
    ("csr_offsets_one_row_early",
     "row_offsets[row + 1] += (int32_t)width;", "row_offsets[row] += (int32_t)width;"),
    ("csr_column_off_by_one",
     "col_indices[e] = (int32_t)(idx[k] % cols);", "col_indices[e] = (int32_t)((idx[k] + 1) % cols);"),
    ("csr_to_coo_transposed",
     "idx[j] = r * cols + col_indices[j];", "idx[j] = (int64_t)col_indices[j] * rows + r;"),
    ("read_rows_first_row_only",
     "memcpy(out + k * cols, params + idx[k] * cols,", "memcpy(out + k * cols, params + idx[0] * cols,"),
]


def _pins():
    return sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def _run_pins(workdir, name, text):
    """Builds `text` as the oracle's source and runs the pins against it in a
    child process; returns the child's exit status and output."""
    d = workdir / name
    d.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(text)
    lib = str(d / "liboracle_copy.so")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", lib,
                           str(d / "oracle.c"), "-lm"])
    env = dict(os.environ, SPOPT_ORACLE_LIB=lib)
    pins = [p for p in _pins() if not p.endswith("test_oracle_mutations.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *pins], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def results(workdir):
    """Every copy's pin run (the unchanged source under "unchanged"), four child
    processes at a time."""
    src = open(SRC).read()
    jobs = {"unchanged": src}
    for name, old, new in MUTATIONS:
        if src.count(old) == 1:
            jobs[name] = src.replace(old, new)
    with ThreadPoolExecutor(4) as ex:
        futs = {name: ex.submit(_run_pins, workdir, name, text) for name, text in jobs.items()}
        return {name: f.result() for name, f in futs.items()}


def test_unchanged_copy_passes_the_pins(results):
    """Control: the same harness with the source unchanged passes, so a failure
    below is the planted mistake's and not the harness's."""
    rc, out = results["unchanged"]
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new, results):
    n = open(SRC).read().count(old)
    assert n == 1, f"{name}: the text to replace occurs {n} times"
    rc, out = results[name]
    # 1: tests ran and at least one failed (collection errors and crashes give other codes)
    assert rc == 1, f"{name}: the pins did not fail (exit {rc})\n{out}"
