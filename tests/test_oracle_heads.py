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


# ----------------------------------------------------------------------------- RNN head
# Pins from the RNN head passage's own statements: a gate of 1 writes the
# candidate, a gate of 0 keeps the old state, the state starts at zero, and
# the input concatenates [state; W_down[x_{j-1}]; h_j].

def _rnn_blocks(r, H, gate=None, cand=None, out=None):
    W = np.zeros((3 * r, 2 * r + H))
    for i, blk in enumerate((gate, cand, out)):
        if blk is not None:
            W[i * r:(i + 1) * r] = blk
    return W


def test_rnn_with_identity_output_and_no_state_is_the_silu_head():
    U, A, Bm, h, _, anchor = _case(seed=11)
    r, H = A.shape[1], h.shape[-1]
    out = np.zeros((r, 2 * r + H))
    out[:, r:2 * r] = np.eye(r)                             # W_out picks W_down[x_{j-1}]
    W = _rnn_blocks(r, H, out=out)                          # candidate 0: the state stays 0
    rnn = o.markov_chain(U, anchor, A, Bm, head="rnn", h=h, W_g=W, keep_logits=True)
    silu = o.markov_chain(U, anchor, A, Bm, head="silu", keep_logits=True)
    assert np.array_equal(rnn["tokens"], silu["tokens"])
    assert np.allclose(rnn["logits"], silu["logits"], rtol=0, atol=1e-12)


def test_rnn_open_gate_writes_the_candidate_and_closed_gate_keeps_zero_state():
    U, A, Bm, h, _, anchor = _case(seed=12)
    r, H = A.shape[1], h.shape[-1]
    ones = np.ones_like(h)
    gate = np.zeros((r, 2 * r + H))
    cand = np.zeros((r, 2 * r + H))
    cand[:, 2 * r:] = 0.5 / H                               # with h = 1: candidate tanh(0.5) everywhere
    out = np.zeros((r, 2 * r + H))
    out[:, :r] = 3.0 * np.eye(r)                            # m_j = SiLU(3 s_j)
    want_open = o.round_to_dtype(math.tanh(0.5), "f32")
    for sign, s_want in ((1.0, want_open), (-1.0, 0.0)):
        gate[:, 2 * r:] = sign * 40.0 / H                   # gate pre-activation +-40: sigma = 1 or 0 in fp64
        W = _rnn_blocks(r, H, gate, cand, out)
        s = np.zeros(r)
        for j in range(3):
            s, m = o.rnn_head_step(s, A[5], ones[0, j], W, "f32")
            assert np.allclose(s, s_want, rtol=0, atol=1e-7)
            x = 3.0 * s_want
            assert np.allclose(m, x / (1.0 + math.exp(-x)), rtol=1e-6, atol=1e-7)


def test_rnn_state_starts_at_zero_and_carries_the_previous_position():
    r, H = 4, 6
    g = np.random.default_rng(13)
    A = g.standard_normal((10, r))
    h = g.standard_normal((1, 3, H))
    cand = np.zeros((r, 2 * r + H))
    cand[:, :r] = 2.0 * np.eye(r)                           # candidate tanh(2 s_{j-1}) + tanh of the h block
    cand[:, 2 * r:2 * r + r] = np.eye(r)
    W = _rnn_blocks(r, H, None, cand, np.hstack([np.eye(r), np.zeros((r, r + H))]))
    # gate weights 0: sigma(0) = 1/2, so s_j = (s_{j-1} + tanh(2 s_{j-1} + h_j[:r])) / 2 with s_{-1} = 0
    s_ref = np.zeros(r)
    s = np.zeros(r)
    for j in range(3):
        s_ref = (s_ref + np.tanh(2.0 * s_ref + h[0, j, :r])) / 2.0
        s, _ = o.rnn_head_step(s, A[j], h[0, j], W, "f32")
        assert np.allclose(s, s_ref, rtol=1e-6, atol=1e-7)
    s0, _ = o.rnn_head_step(np.zeros(r), A[0], h[0, 0], W, "f32")
    assert np.allclose(s0, np.tanh(h[0, 0, :r]) / 2.0, rtol=1e-6)


def test_rnn_teacher_forced_form_reproduces_the_chain():
    U, A, Bm, h, _, anchor = _case(seed=14)
    r, H = A.shape[1], h.shape[-1]
    g = np.random.default_rng(15)
    W = o.round_to_dtype(g.standard_normal((3 * r, 2 * r + H)) * 0.3, "bf16")
    ch = o.markov_chain(U, anchor, A, Bm, head="rnn", h=h, W_g=W, keep_logits=True)
    prev = np.concatenate([anchor[:, None], ch["tokens"][:, :-1]], axis=1)
    tf = o.teacher_forced_logits(U, prev, A, Bm, head="rnn", h=h, W_g=W)
    assert np.allclose(tf, ch["logits"], rtol=0, atol=1e-12)
