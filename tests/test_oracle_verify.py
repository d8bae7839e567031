"""Pins of the oracle's rejection-sampling verification ("DeepSpec 训练全流程详解",
§4.4; "DSpark 论文精读", §2.1): the emitted tokens follow the target's
distribution (the speculative-sampling theorem) at the first and at a later
position, the acceptance rate equals the distribution overlap, and the
degenerate cases (identical distributions, an empty proposal, the residual's
support)."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import dspark_oracle as o


def _probs(logits):
    e = np.exp(logits - logits.max())
    return e / e.sum()


def _trials(n, V=5, G=1, seed=0):
    """n independent requests sharing fixed target/draft rows; drafted tokens
    drawn from q with numpy's generator (independent of the verifier's Philox
    stream); seeds 0..n-1."""
    g = np.random.default_rng([seed, 31])
    tl = g.standard_normal((G + 1, V)) * 1.5
    dl = g.standard_normal((G, V)) * 1.5
    q = np.stack([_probs(dl[j]) for j in range(G)])
    toks = np.stack([g.choice(V, size=n, p=q[j]) for j in range(G)], axis=1)
    t = np.broadcast_to(tl, (n, G + 1, V))
    d = np.broadcast_to(dl, (n, G, V))
    r = o.verify_draft(t, d, toks, np.full(n, G), np.arange(n, dtype=np.uint64) + 1000 * seed)
    return tl, dl, toks, r


def test_first_emitted_token_follows_the_target():
    n, V = 30000, 5
    tl, dl, toks, r = _trials(n, V=V, seed=1)
    first = np.where(r["accepted"] >= 1, toks[:, 0], r["next_token"])
    counts = np.bincount(first, minlength=V)
    p0 = _probs(tl[0])
    chi2 = ((counts - n * p0) ** 2 / (n * p0)).sum()
    assert stats.chi2.sf(chi2, V - 1) > 1e-4, (counts, n * p0)


def test_acceptance_rate_is_the_overlap():
    n, V = 30000, 5
    tl, dl, toks, r = _trials(n, V=V, seed=2)
    alpha = np.minimum(_probs(tl[0]), _probs(dl[0])).sum()
    rate = (r["accepted"] >= 1).mean()
    assert abs(rate - alpha) <= 4 * math.sqrt(alpha * (1 - alpha) / n), (rate, alpha)


def test_second_emitted_token_follows_the_target_after_an_accept():
    # the target rows are fixed here, so given an accepted first token the
    # second emitted token must follow p_1
    n, V = 40000, 4
    tl, dl, toks, r = _trials(n, V=V, G=2, seed=3)
    sel = r["accepted"] >= 1
    second = np.where(r["accepted"][sel] >= 2, toks[sel, 1], r["next_token"][sel])
    m = sel.sum()
    counts = np.bincount(second, minlength=V)
    p1 = _probs(tl[1])
    chi2 = ((counts - m * p1) ** 2 / (m * p1)).sum()
    assert stats.chi2.sf(chi2, V - 1) > 1e-4, (counts, m * p1)


def test_identical_distributions_accept_every_token():
    g = np.random.default_rng(4)
    B, G, V = 50, 7, 30
    t = g.standard_normal((B, G + 1, V))
    toks = g.integers(0, V, (B, G))
    r = o.verify_draft(t, t[:, :G], toks, np.full(B, G), np.arange(B))
    assert (r["accepted"] == G).all()


def test_empty_proposal_draws_from_the_first_target_row():
    g = np.random.default_rng(5)
    B, G, V = 20, 7, 40
    t = g.standard_normal((B, G + 1, V))
    d = g.standard_normal((B, G, V))
    toks = g.integers(0, V, (B, G))
    seeds = np.arange(B, dtype=np.uint64) * 7919
    r = o.verify_draft(t, d, toks, np.zeros(B, int), seeds, offset=3)
    assert (r["accepted"] == 0).all()
    for b in range(B):
        want = int(np.argmax(t[b, 0] + o.gumbel(int(seeds[b]), 3, o.VERIFY_GUMBEL, V)))
        assert r["next_token"][b] == want


def test_residual_draws_stay_where_the_target_exceeds_the_draft():
    V, n = 6, 4000
    tl = np.log(np.array([0.05, 0.30, 0.05, 0.40, 0.10, 0.10]))
    dl = np.log(np.array([0.30, 0.10, 0.20, 0.05, 0.20, 0.15]))
    g = np.random.default_rng(6)
    toks = g.choice(V, size=(n, 1), p=np.exp(dl))
    t = np.broadcast_to(tl, (n, 2, V))
    d = np.broadcast_to(dl, (n, 1, V))
    r = o.verify_draft(t, d, toks, np.ones(n, int), np.arange(n))
    rej = r["accepted"] == 0
    assert rej.any()
    assert set(np.unique(r["next_token"][rej])) <= {1, 3}


def test_acceptance_uniforms_are_uniform_and_exact():
    u = np.array([o.verify_uniform(s, 0, j) for s in range(400) for j in range(7)])
    assert (u > 0).all() and (u < 1).all()
    assert np.all(np.float32(u) == u)                    # exact in binary32
    assert stats.kstest(u, "uniform").pvalue > 1e-3


def test_bonus_token_follows_the_last_target_row():
    # identical draft and target rows always accept, so the next token is the
    # draw from p_L (here L = 2: the third row)
    n, V, G = 20000, 5, 2
    g = np.random.default_rng(7)
    tl = g.standard_normal((G + 1, V)) * 1.5
    t = np.broadcast_to(tl, (n, G + 1, V))
    toks = g.integers(0, V, (n, G))
    r = o.verify_draft(t, t[:, :G], toks, np.full(n, G), np.arange(n))
    assert (r["accepted"] == G).all()
    counts = np.bincount(r["next_token"], minlength=V)
    p = _probs(tl[G])
    chi2 = ((counts - n * p) ** 2 / (n * p)).sum()
    assert stats.chi2.sf(chi2, V - 1) > 1e-4, (counts, n * p)
