"""Pins of the oracle's confidence/survival and overlap/tau metrics: printed
worked numbers, identities, closed forms and degenerate cases."""
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import dspark_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cumprod_golden():
    rows, ratio = [], None
    with open(os.path.join(GOLDEN, "cumprod_sensitivity.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            p = line.split()
            if p[0] == "ratio":
                ratio = (float(p[1]), float(p[2]))
            else:
                rows.append((float(p[0]), int(p[1]), float(p[2]), float(p[3])))
    return rows, ratio


def _const_conf(c, B=1, gamma=7, H=8):
    # w_c = 0 and b_c = logit(c): every slot's confidence is exactly c
    h = np.random.default_rng(0).standard_normal((B, gamma, H))
    return o.confidence_survival(h, np.zeros(H), math.log(c / (1 - c)))


def test_printed_cumprod_sensitivity_example():
    rows, (ratio, rtol) = _cumprod_golden()
    surv_at = {}
    for c, pos, printed, tol in rows:
        conf, surv = _const_conf(c)
        assert np.allclose(conf, c, atol=1e-15)
        assert abs(surv[0, pos - 1] - printed) <= tol
        surv_at[c] = surv[0, pos - 1]
    assert abs(100 * (surv_at[0.85] / surv_at[0.80] - 1) - ratio) <= rtol


def test_survival_is_monotone_and_starts_at_first_confidence():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((20, 7, 32))
    conf, surv = o.confidence_survival(h, rng.standard_normal(32), 0.3)
    assert np.all(np.diff(surv, axis=1) <= 0)
    assert np.array_equal(surv[:, 0], conf[:, 0])
    assert np.all((conf > 0) & (conf < 1))


def test_confidence_closed_form_with_markov_term():
    # h = 0, w_c = 0, A one-hot rows: s_j = b_c + w_m[k(prev_j)]
    V, r = 6, 3
    A = np.zeros((V, r))
    kk = [0, 2, 1, 1, 0, 2]
    A[np.arange(V), kk] = 1.0
    w_m = np.array([0.5, -1.0, 2.0])
    anchor, tokens = np.array([3]), np.array([[5, 0, 1, 4, 2, 2, 3]])
    conf, _ = o.confidence_survival(np.zeros((1, 7, 4)), np.zeros(4), 0.25, w_m=w_m, A=A,
                                    anchor=anchor, tokens=tokens)
    prev = [3, 5, 0, 1, 4, 2, 2]
    want = [1 / (1 + math.exp(-(0.25 + w_m[kk[p]]))) for p in prev]
    assert np.allclose(conf[0], want, atol=1e-15)


def _rows(n, V, seed=0, scale=1.0):
    return np.random.default_rng(seed).standard_normal((n, V)) * scale


def test_overlap_identity_sum_min_equals_one_minus_half_l1():
    t, d = _rows(9, 5000, 1), _rows(9, 5000, 2, 1.7)
    a, l1 = o.overlap_dense(t, d)
    assert np.allclose(a, 1 - 0.5 * l1, atol=1e-13)
    assert np.all((a > 0) & (a < 1))


def test_overlap_identical_and_disjoint():
    t = _rows(3, 700, 3)
    a, _ = o.overlap_dense(t, t.copy())
    assert np.allclose(a, 1.0, atol=1e-13)
    one_hot_p = np.full((1, 50), -1e4)
    one_hot_p[0, 3] = 0
    one_hot_q = np.full((1, 50), -1e4)
    one_hot_q[0, 8] = 0
    a, l1 = o.overlap_dense(one_hot_p, one_hot_q)
    assert a[0] == 0.0 and l1[0] == 2.0


def test_overlap_is_shift_invariant():
    t, d = _rows(2, 900, 4), _rows(2, 900, 5)
    a1, _ = o.overlap_dense(t, d)
    a2, _ = o.overlap_dense(t + 30.0, d - 7.0)
    assert np.allclose(a1, a2, atol=1e-13)


@pytest.mark.parametrize("sigma,limit", [(0.5, 0.8026), (1.0, 0.6171), (2.0, 0.3173)])
def test_overlap_closed_form_for_gaussian_noise(sigma, limit):
    # teacher = draft + N(0, sigma^2) iid over a large vocabulary: the overlap
    # tends to 2 Phi(-sigma/2) (law of large numbers over the vocabulary)
    assert abs(2 * stats.norm.cdf(-sigma / 2) - limit) < 1e-4
    V = 151936
    d = _rows(6, V, 6)
    t = d + sigma * _rows(6, V, 7)
    a, _ = o.overlap_dense(t, d)
    assert abs(a.mean() - limit) < 6e-3


def test_tau_bounds_identical_and_first_rejected():
    rng = np.random.default_rng(8)
    alpha = rng.random((50, 7))
    _, tau, _, _ = o.tau_metrics(alpha)
    assert np.all((tau >= 1) & (tau <= 8))
    _, tau1, acc1, m1 = o.tau_metrics(np.ones((4, 7)))
    assert np.all(tau1 == 8.0) and np.all(acc1 == 1.0) and m1 == 8.0
    a0 = alpha.copy()
    a0[:, 0] = 0
    _, tau0, _, _ = o.tau_metrics(a0)
    assert np.all(tau0 == 1.0)


@pytest.mark.parametrize("a", [0.1, 0.5, 0.9])
def test_tau_constant_alpha_geometric_series(a):
    _, tau, _, _ = o.tau_metrics(np.full((3, 7), a))
    assert np.allclose(tau, 1 + a * (1 - a ** 7) / (1 - a), atol=1e-14)


def test_tau_validity_truncation_and_dummy_blocks():
    alpha = np.full((4, 7), 0.5)
    valid = np.ones((4, 7), dtype=np.uint8)
    valid[1, 3:] = 0           # prefix of 3 valid slots
    valid[3, :] = 0            # padding block
    a, tau, acc, mean = o.tau_metrics(alpha, valid)
    assert np.all(a[1, 3:] == 0) and np.all(a[3] == 0)
    assert tau[0] == 1 + 0.5 * (1 - 0.5 ** 7) / 0.5
    assert tau[1] == 1 + 0.5 + 0.25 + 0.125
    assert tau[3] == 0.0
    assert math.isclose(mean, (tau[0] * 2 + tau[1]) / 3, rel_tol=1e-15)
    assert np.all(acc == 0.5)  # each position averages only its valid slots


def test_tau_clamps_alpha():
    _, tau, acc, _ = o.tau_metrics(np.array([[1.0000001, 1.2, -0.1, 0.5, 0.5, 0.5, 0.5]]))
    assert tau[0] == 3.0 and acc[0] == 1.0 and acc[2] == 0.0


def test_sparse_overlap_full_support_equals_dense():
    rng = np.random.default_rng(9)
    V = 24
    t, d = rng.standard_normal((5, V)), rng.standard_normal((5, V))
    q = o.softmax(d)
    idx = np.tile(np.arange(V), (5, 1))
    perm = rng.permutation(V)
    a_sparse = o.overlap_sparse(t, idx[:, perm], q[:, perm])
    a_dense, _ = o.overlap_dense(t, d)
    assert np.allclose(a_sparse, a_dense, atol=1e-14)


def test_sparse_overlap_ignores_mass_outside_candidates():
    t = np.zeros((1, 10))                        # p uniform, 0.1 each
    a = o.overlap_sparse(t, np.array([[2, 7]]), np.array([[0.75, 0.25]]))
    assert math.isclose(a[0], 0.2, rel_tol=1e-14)


def test_expected_tau_under_gaussian_noise():
    # independent rows: E[tau] = 1 + sum_{i=1}^{7} E[alpha]^i
    sigma, V = 1.0, 151936
    abar = 2 * stats.norm.cdf(-sigma / 2)
    want = 1 + abar * (1 - abar ** 7) / (1 - abar)
    assert abs(want - 2.557) < 1e-3
    d = _rows(2 * 7, V, 10)
    t = d + sigma * _rows(2 * 7, V, 11)
    a, _ = o.overlap_dense(t, d)
    _, tau, _, _ = o.tau_metrics(a.reshape(2, 7))
    assert abs(tau.mean() - want) < 0.05
