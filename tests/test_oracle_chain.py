"""Pins of the oracle's LM head and sequential Markov chain (greedy, sampled,
top-k), by closed forms, special cases, library routines and brute force."""
import itertools

import numpy as np
import pytest
from scipy import special, stats

from oracle import dspark_oracle as o


def test_lm_head_one_hot_selects_columns():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((11, 6))
    h = np.eye(6)[[4, 0, 5]]
    U = o.lm_head(h, W)
    assert np.array_equal(U, W[:, [4, 0, 5]].T)


def test_lm_head_brute_force_loops():
    rng = np.random.default_rng(2)
    h, W = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    U = o.lm_head(h, W)
    for m in range(3):
        for v in range(4):
            s = 0.0
            for k in range(5):
                s += h[m, k] * W[v, k]
            assert abs(U[m, v] - s) < 1e-12


def _perm_case(V=8, gamma=7, c=4.0, seed=3):
    """A = I, Bm = c * P_pi: the bias after token t is c at pi(t) only, so the
    greedy chain walks the permutation from the anchor."""
    rng = np.random.default_rng(seed)
    pi = rng.permutation(V)
    A = np.eye(V)
    Bm = np.zeros((V, V))
    Bm[np.arange(V), pi] = c
    U = rng.uniform(-0.4 * c, 0.4 * c, size=(2, gamma, V))
    return pi, A, Bm, U


def test_greedy_chain_walks_a_permutation():
    pi, A, Bm, U = _perm_case()
    anchor = np.array([5, 2])
    out = o.markov_chain(U, anchor, A, Bm)
    for b in range(2):
        t = anchor[b]
        for j in range(U.shape[1]):
            t = pi[t]
            assert out["tokens"][b, j] == t


def test_zero_transition_reduces_to_parallel_argmax():
    # with no transition bias the chain is the pure-parallel product of
    # marginals ([P4] §2.2): each slot takes argmax of its own base logits
    rng = np.random.default_rng(4)
    U = rng.standard_normal((3, 7, 50))
    out = o.markov_chain(U, np.array([1, 2, 3]), np.zeros((50, 4)), rng.standard_normal((4, 50)))
    assert np.array_equal(out["tokens"], U.argmax(axis=-1))


def test_teacher_forced_form_reproduces_the_chain():
    rng = np.random.default_rng(5)
    B, g, V, r = 3, 7, 40, 6
    U = rng.standard_normal((B, g, V))
    A, Bm = rng.standard_normal((V, r)), rng.standard_normal((r, V)) * 0.5
    anchor = np.array([0, 17, 39])
    out = o.markov_chain(U, anchor, A, Bm, keep_logits=True)
    prev = np.concatenate([anchor[:, None], out["tokens"][:, :-1]], axis=1)
    tf = o.teacher_forced_logits(U, prev, A, Bm)
    assert np.allclose(tf, out["logits"], rtol=0, atol=1e-12)
    assert np.allclose(out["lse"], special.logsumexp(out["logits"], axis=-1), atol=1e-12)
    assert np.array_equal(out["tok_logit"], np.take_along_axis(out["logits"], out["tokens"][..., None], -1)[..., 0])


def test_gap_is_best_minus_second():
    U = np.zeros((1, 1, 6))
    U[0, 0, [1, 4]] = [2.0, 1.25]
    out = o.markov_chain(U, np.array([0]), np.zeros((6, 2)), np.zeros((2, 6)))
    assert out["tokens"][0, 0] == 1 and out["gap"][0, 0] == 0.75


def test_ties_go_to_lowest_index():
    U = np.zeros((1, 2, 9))
    U[0, 0, [7, 3, 5]] = 1.0
    out = o.markov_chain(U, np.array([0]), np.zeros((9, 2)), np.zeros((2, 9)), topk=4)
    assert out["tokens"][0, 0] == 3
    assert list(out["topk_idx"][0, 0]) == [3, 5, 7, 0]
    assert list(out["topk_idx"][0, 1]) == [0, 1, 2, 3]


def test_forced_prefix_is_followed():
    pi, A, Bm, U = _perm_case()
    forced = -np.ones((2, 7), dtype=np.int64)
    forced[0, 2] = 6
    out = o.markov_chain(U, np.array([5, 2]), A, Bm, forced=forced)
    assert out["tokens"][0, 2] == 6 and out["tokens"][0, 3] == pi[6]


@pytest.mark.parametrize("temperature", [1.0, 0.6])
def test_gumbel_max_samples_the_chain_distribution(temperature):
    # brute force: enumerate all V^gamma sequences of a tiny chain and compare
    # the empirical frequency of the sampled blocks by chi-square
    rng = np.random.default_rng(6)
    V, g, r = 5, 3, 2
    U1 = rng.standard_normal((g, V))
    A, Bm = rng.standard_normal((V, r)), rng.standard_normal((r, V))
    anchor = 2
    joint = {}
    for seq in itertools.product(range(V), repeat=g):
        p, prev = 1.0, anchor
        for j, x in enumerate(seq):
            z = (U1[j] + A[prev] @ Bm) / temperature
            p *= np.exp(z[x] - special.logsumexp(z))
            prev = x
        joint[seq] = p
    assert abs(sum(joint.values()) - 1) < 1e-12
    n = 12000
    U = np.broadcast_to(U1, (n, g, V))
    out = o.markov_chain(U, np.full(n, anchor), A, Bm, temperature=temperature,
                         seeds=np.arange(n, dtype=np.uint64) + 1000, offset=3)
    seqs = list(joint)
    index = {s: i for i, s in enumerate(seqs)}
    obs = np.zeros(len(seqs))
    for row in out["tokens"]:
        obs[index[tuple(int(x) for x in row)]] += 1
    exp = np.array([joint[s] for s in seqs]) * n
    big = exp >= 5
    obs_m = np.append(obs[big], obs[~big].sum())
    exp_m = np.append(exp[big], exp[~big].sum())
    assert stats.chisquare(obs_m, exp_m).pvalue > 1e-4


def test_topk_equal_to_vocab_is_the_dense_softmax():
    rng = np.random.default_rng(7)
    V = 16
    U = rng.standard_normal((2, 3, V))
    A, Bm = rng.standard_normal((V, 4)), rng.standard_normal((4, V))
    out = o.markov_chain(U, np.array([1, 9]), A, Bm, topk=V, keep_logits=True)
    q = o.softmax(out["logits"])
    dense = np.take_along_axis(q, out["topk_idx"], axis=-1)
    assert np.allclose(out["topk_prob"], dense, atol=1e-14)
    assert np.allclose(out["topk_prob"].sum(-1), 1.0)
    # candidates in descending order of U~
    vals = np.take_along_axis(out["logits"], out["topk_idx"], axis=-1)
    assert np.all(np.diff(vals, axis=-1) <= 0)


def test_topk_matches_a_stable_library_sort():
    rng = np.random.default_rng(8)
    x = np.round(rng.standard_normal(3000), 1)        # many ties
    want = np.argsort(-x, kind="stable")[:16]
    assert np.array_equal(o.topk_indices(x, 16), want)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x3C23, 0x7F7F], dtype=np.uint16)
    vals = o.widen_bf16(bits)
    assert list(vals[:3]) == [1.0, -1.0, 0.0]
    assert vals[3] == 1.2734375 * 2.0 ** -7           # 0x3C23: exponent 120, mantissa 35/128
    assert vals[4] == (2 - 2 ** -7) * 2.0 ** 127
