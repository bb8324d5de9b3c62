"""The seeded input generators: reproducible streams, bounded Zipf ids in range,
and the scrambled placement keeping the same multiplicities (CPU only)."""
import math

import numpy as np

import synth


def test_lookups_are_reproducible_and_in_range():
    w = synth.WORKLOADS[3]
    a_ids, a_g = synth.lookups(w, 7, n=5000)
    b_ids, b_g = synth.lookups(w, 7, n=5000)
    assert np.array_equal(a_ids, b_ids) and np.array_equal(a_g, b_g)
    assert a_ids.dtype == np.int64 and a_g.dtype == np.float32 and a_g.shape == (5000, w.cols)
    assert a_ids.min() >= 0 and a_ids.max() < w.rows
    c_ids, _ = synth.lookups(w, 8, n=5000)
    assert not np.array_equal(a_ids, c_ids)


def test_zipf_rank_one_is_row_zero_and_most_frequent():
    w = synth.WORKLOADS[3]
    ids, _ = synth.lookups(w, 0, n=20000)
    u, c = np.unique(ids, return_counts=True)
    assert u[np.argmax(c)] == 0
    # P(row 0) = 1 / H(R, s); the sample frequency is within a few standard errors
    h = float(np.sum(np.arange(1, w.rows + 1, dtype=np.float64) ** -w.zipf_s))
    p0 = 1.0 / h
    f0 = c[u == 0][0] / ids.size
    assert abs(f0 - p0) < 5 * math.sqrt(p0 * (1 - p0) / ids.size)


def test_scrambled_placement_keeps_multiplicities():
    w = synth.WORKLOADS[3]
    ws = w.scaled(scramble=999983)
    assert math.gcd(ws.scramble, w.rows) == 1          # a bijection of the rows
    ids, g = synth.lookups(w, 3, n=20000)
    sids, sg = synth.lookups(ws, 3, n=20000)
    assert np.array_equal(sg, g)
    assert np.array_equal(sids, (ids * 999983) % w.rows)
    _, c = np.unique(ids, return_counts=True)
    _, sc = np.unique(sids, return_counts=True)
    assert sorted(c.tolist()) == sorted(sc.tolist())
    assert sids.min() >= 0 and sids.max() < w.rows
