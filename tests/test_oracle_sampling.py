"""Pins of the oracle's random-number path: Philox4x32-10 and Gumbel noise."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import dspark_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", _kat_rows())
def test_philox_known_answers(row):
    ctr, key, want = row[0:4], row[4:6], row[6:10]
    got = o.philox4x32_10(*ctr, *key)
    assert [int(x) for x in got] == want


def test_philox_vectorised_equals_scalar():
    ctr = np.arange(37, dtype=np.uint64) * 7919
    vec = o.philox4x32_10(ctr, 3, 5, 0, 0xDEADBEEF, 12)
    for i, c in enumerate(ctr):
        sc = o.philox4x32_10(int(c), 3, 5, 0, 0xDEADBEEF, 12)
        assert all(int(vec[w][i]) == int(sc[w]) for w in range(4))


def test_word_layout_counter_and_key():
    # word v of (seed, offset, j) is output word v%4 of counter (v//4, j, off_lo, off_hi)
    seed, offset, j = (7 << 32) | 3, (5 << 32) | 9, 4
    w = o.philox_words(seed, offset, j, 10)
    c = o.philox4x32_10(2, j, 9, 5, 3, 7)
    assert [int(w[8]), int(w[9])] == [int(c[0]), int(c[1])]


def test_uniform_is_exact_in_binary32_and_open_interval():
    w = o.philox_words(11, 0, 0, 200000)
    u = ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23
    assert np.all(u > 0) and np.all(u < 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    # extremes of the map
    assert (0 + 0.5) * 2.0 ** -23 > 0 and ((2 ** 23 - 1) + 0.5) * 2.0 ** -23 < 1
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_gumbel_moments_and_distribution():
    g = np.concatenate([o.gumbel(s, 0, j, 50000) for s in range(4) for j in range(5)])
    n = g.size
    euler_gamma = 0.5772156649015329
    assert abs(g.mean() - euler_gamma) < 5 * math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-3


def test_streams_differ_by_request_position_and_offset():
    a = o.gumbel(1, 0, 0, 64)
    assert not np.array_equal(a, o.gumbel(2, 0, 0, 64))
    assert not np.array_equal(a, o.gumbel(1, 0, 1, 64))
    assert not np.array_equal(a, o.gumbel(1, 1, 0, 64))
    assert np.array_equal(a, o.gumbel(1, 0, 0, 64))


def test_leading_requests_equal_a_fresh_draw():
    """The benchmark takes its one- and 64-request workloads as the leading
    requests of the 256-request draw; each per-tensor stream is sequential,
    so they equal fresh draws of the smaller workloads."""
    import synth
    big = synth.propose_inputs(B=9, H=64, V=520, r=32, wdtype="bf16", topk=4)
    for B in (1, 4):
        small = synth.propose_inputs(B=B, H=64, V=520, r=32, wdtype="bf16", temperature=1.0, topk=0)
        cut = synth.leading_requests(big, B, temperature=1.0, topk=0)
        for name in ("h", "w_lm", "A", "Bm", "anchor", "w_c", "teacher", "seeds"):
            assert np.array_equal(getattr(cut, name), getattr(small, name)), name
        assert (cut.B, cut.temperature, cut.topk) == (B, 1.0, 0)
