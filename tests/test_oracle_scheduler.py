"""Pins of the oracle's hardware-aware prefix scheduler ("DSpark 论文精读",
§3.2): exhaustive search over every length vector, an independent correctly
rounded summation, closed-form tables and the monotone response to a steeper
hardware curve."""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import dspark_oracle as o


def _objective(a, sps, lengths):
    """Theta of one length vector straight from its definition: tau = R plus
    each request's first l_r survival values (one correctly rounded sum),
    B = sum (1 + l_r), Theta = tau * SPS(B)."""
    R = a.shape[0]
    B = R + int(sum(lengths))
    terms = [float(R)] + [float(a[r, j]) for r in range(R) for j in range(int(lengths[r]))]
    tau = math.fsum(terms)
    return tau * float(sps[B - 1]), tau, B


@pytest.mark.parametrize("seed", range(24))
def test_greedy_scan_matches_exhaustive_search(seed):
    g = np.random.default_rng([seed, 99])
    R = int(g.integers(1, 4))
    gamma = int(g.integers(1, 5))
    a = synth.survival_rows(R, gamma, seed=seed)
    n = R * (gamma + 1) - int(g.integers(0, 3))          # sometimes cuts the last batches off
    n = max(n, R)
    sps = g.uniform(0.2, 3.0, size=n)                      # any positive table, not only monotone
    best = None
    for lens in itertools.product(range(gamma + 1), repeat=R):
        if R + sum(lens) > n:
            continue
        th, tau, B = _objective(a, sps, lens)
        key = (th, -B)
        if best is None or key > best[0]:
            best = (key, lens, tau, B)
    lengths, theta, tau, batch = o.prefix_schedule(a, sps)
    assert theta == best[0][0]
    assert batch == best[3]
    assert _objective(a, sps, lengths)[0] == theta
    assert tuple(int(x) for x in lengths) == best[1]
    assert tau == best[2]


@pytest.mark.parametrize("R,gamma,seed", [(50, 7, 1), (256, 7, 2), (9, 16, 3)])
def test_tau_is_the_correctly_rounded_sum_of_the_taken_prefixes(R, gamma, seed):
    a = synth.survival_rows(R, gamma, seed=seed)
    sps = synth.sps_table(R * (gamma + 1), knee=R + 3 * R // 2, per_token_ms=0.02)
    lengths, theta, tau, batch = o.prefix_schedule(a, sps)
    th, t, B = _objective(a, sps, lengths)       # lengths read as prefixes of each row
    assert (t, B) == (tau, batch)
    assert th == theta
    assert 0 < batch - R < R * gamma                # this table makes an interior cut


def test_flat_table_admits_every_positive_candidate():
    a = synth.survival_rows(20, 7, seed=4)
    a[3, 4:] = 0.0
    a[11, :] = 0.0
    lengths, theta, tau, batch = o.prefix_schedule(a, np.full(20 * 8, 3.0))
    assert np.array_equal(lengths, (a > 0).sum(axis=1))
    assert batch == 20 + int((a > 0).sum())


def test_inverse_batch_table_admits_nothing():
    # SPS(B) = 1/B makes Theta the mean emitted tokens per slot: every
    # candidate below 1 lowers it
    a = np.minimum(synth.survival_rows(30, 7, seed=5), np.float32(0.99))
    sps = 1.0 / np.arange(1, 30 * 8 + 1, dtype=np.float64)
    lengths, theta, tau, batch = o.prefix_schedule(a, sps)
    assert not lengths.any() and batch == 30 and tau == 30.0
    assert theta == 30.0 * sps[29]


def test_step_table_fills_exactly_to_the_knee():
    R, gamma, knee = 10, 7, 30
    a = (synth.survival_rows(R, gamma, seed=6) * np.float32(0.1)).astype(np.float32)
    sps = np.where(np.arange(1, R * (gamma + 1) + 1) <= knee, 2.0, 1.0)
    lengths, theta, tau, batch = o.prefix_schedule(a, sps)
    assert batch == knee
    top = np.sort(a.ravel())[::-1][:knee - R]
    assert np.array_equal(lengths, (a >= top[-1]).sum(axis=1))


def test_steeper_hardware_curve_never_admits_more():
    # log Theta = log tau(B) - log(1 + s (B - R)) has decreasing differences in
    # (B, s), so the chosen batch cannot grow with the slope s
    R, gamma = 64, 7
    a = synth.survival_rows(R, gamma, seed=7)
    B = np.arange(1, R * (gamma + 1) + 1, dtype=np.float64)
    prev = None
    for s in [0.0, 1e-4, 1e-3, 3e-3, 1e-2, 3e-2, 0.1, 1.0]:
        sps = 1.0 / (1.0 + s * np.maximum(B - R, 0.0))
        batch = o.prefix_schedule(a, sps)[3]
        if prev is not None:
            assert batch <= prev
        prev = batch
    assert prev == R                                      # a steep enough curve sends no drafts


def test_out_of_range_values_are_clamped():
    a = synth.survival_rows(6, 5, seed=8)
    b = a.copy()
    a[0, 0], a[2, 3], a[5, 1] = np.nan, -0.5, 7.0
    b[0, 0], b[2, 3], b[5, 1] = 0.0, 0.0, 1.0
    sps = synth.sps_table(6 * 6, knee=8, per_token_ms=0.4)
    got, want = o.prefix_schedule(a, sps), o.prefix_schedule(b, sps)
    assert np.array_equal(got[0], want[0]) and got[1:] == want[1:]


def test_table_end_caps_the_batch_and_ties_follow_the_flat_index():
    a = np.full((3, 2), 0.5, dtype=np.float32)
    lengths, theta, tau, batch = o.prefix_schedule(a, np.ones(3 + 3))
    assert batch == 6 and list(lengths) == [2, 1, 0]
    assert tau == 4.5 and theta == 4.5


def test_table_shorter_than_the_requests_is_rejected():
    with pytest.raises(ValueError):
        o.prefix_schedule(np.zeros((4, 2), np.float32), np.ones(3))
