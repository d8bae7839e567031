"""Pins of the oracle's sequential-head variants ("DSpark 论文精读", §2.3 heads
table): SiLU-Vanilla and GatedMarkov reduce to closed forms or to the linear
chain in limiting cases, m_j is rounded to the tables' dtype, and the
teacher-forced form reproduces the chain's corrected logits."""
import math

import numpy as np
import pytest

from oracle import dspark_oracle as o


def _case(B=3, gamma=5, V=60, r=8, H=12, seed=0):
    g = np.random.default_rng([seed, 61])
    U = g.standard_normal((B, gamma, V))
    A = o.round_to_dtype(g.standard_normal((V, r)) * 0.8, "bf16")
    Bm = o.round_to_dtype(g.standard_normal((r, V)) * 0.8, "bf16")
    h = o.round_to_dtype(g.standard_normal((B, gamma, H)), "bf16")
    W_g = o.round_to_dtype(g.standard_normal((r, H + r)) * 0.3, "bf16")
    anchor = g.integers(0, V, B)
    return U, A, Bm, h, W_g, anchor


def test_silu_values_and_rounding():
    a = np.array([-50.0, 0.0, 1.0, 2.0, 50.0])
    got = o.head_vector("silu", a)
    s1 = 1.0 / (1.0 + math.exp(-1.0))                   # SiLU(1) = sigma(1) = 0.7310585786
    assert got[1] == 0.0 and got[4] == 50.0 and abs(got[0]) < 1e-20
    assert got[2] == 0.73046875                          # the bf16 neighbour of 0.73106 (8-bit mantissa)
    assert abs(got[2] - s1) <= 2.0 ** -9 * s1
    assert got[3] == o.round_to_dtype(np.array([2.0 / (1.0 + math.exp(-2.0))]), "bf16")[0]
    assert o.round_to_dtype(np.array([1.0 + 2.0 ** -8]), "bf16")[0] == 1.0       # tie to even
    assert o.round_to_dtype(np.array([1.0 + 3 * 2.0 ** -8]), "bf16")[0] == 1.0 + 2.0 ** -6


def test_zero_gate_weights_halve_the_transition():
    U, A, Bm, h, W_g, anchor = _case(seed=1)
    got = o.markov_chain(U, anchor, A, Bm, head="gated", h=h, W_g=np.zeros_like(W_g))
    want = o.markov_chain(U, anchor, A * 0.5, Bm)           # sigma(0) = 1/2, exact in bf16
    assert np.array_equal(got["tokens"], want["tokens"])
    assert np.allclose(got["lse"], want["lse"], rtol=0, atol=1e-12)


def test_saturated_gate_and_large_silu_inputs_give_the_linear_chain():
    U, A, Bm, h, W_g, anchor = _case(seed=2)
    H = h.shape[-1]
    Wsat = np.zeros_like(W_g)
    Wsat[:, :H] = 20.0 / H                                  # with h = 1: z = 20, sigma(z) = 1 - 2e-9
    ones = np.ones_like(h)
    lin = o.markov_chain(U, anchor, A, Bm)
    gated = o.markov_chain(U, anchor, A, Bm, head="gated", h=ones, W_g=Wsat)
    assert np.array_equal(gated["tokens"], lin["tokens"])
    assert np.allclose(gated["lse"], lin["lse"], rtol=0, atol=1e-12)
    Apos = o.round_to_dtype(A + 30.0, "bf16")               # SiLU(a) = a (1 - e^-a) rounds to a
    lin2 = o.markov_chain(U, anchor, Apos, Bm * 0.01)
    silu2 = o.markov_chain(U, anchor, Apos, Bm * 0.01, head="silu")
    assert np.array_equal(silu2["tokens"], lin2["tokens"])


@pytest.mark.parametrize("head", ["silu", "gated"])
def test_teacher_forced_form_reproduces_the_chain(head):
    U, A, Bm, h, W_g, anchor = _case(seed=3)
    ch = o.markov_chain(U, anchor, A, Bm, head=head, h=h, W_g=W_g, keep_logits=True)
    prev = np.concatenate([anchor[:, None], ch["tokens"][:, :-1]], axis=1)
    tf = o.teacher_forced_logits(U, prev, A, Bm, head=head, h=h, W_g=W_g)
    assert np.allclose(tf, ch["logits"], rtol=0, atol=1e-12)


def test_gated_vector_against_a_loop():
    U, A, Bm, h, W_g, anchor = _case(seed=4)
    a, hr = A[7], h[1, 2]
    x = list(hr) + list(a)
    want = []
    for k in range(a.shape[0]):
        z = sum(W_g[k, i] * x[i] for i in range(len(x)))
        want.append(a[k] / (1.0 + math.exp(-z)))
    got = o.head_vector("gated", a, h_row=hr, W_g=W_g)
    assert np.array_equal(got, o.round_to_dtype(np.array(want), "bf16"))
