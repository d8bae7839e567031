"""Helpers shared by the GPU parity tests: moving synthetic inputs to the
device and comparing the HIP results with the oracle under the stated bars.

Bars (fixed for this hot path):
  * drafted tokens bit-exact, except where the oracle's top-2 gap of the
    selection score is below 1e-3; after such a near-tie the oracle is re-run
    along the GPU's choice and the rest of the block is checked against that;
  * logits and probabilities within 2e-2 relative, read as
    |x - y| <= 2e-2 * max(|y|, rms(row));
  * alpha and tau_prob within 1e-3 absolute.
The tests also apply a tighter check where fp32 accumulation of exact bf16
inputs leaves far more margin (TIGHT * rms(row)), to catch small mistakes.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import dspark_oracle as o

TOKEN_GAP = 1e-3
REL = 2e-2
ALPHA_ABS = 1e-3
TIGHT = 1e-4


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda", 0)


def to_dev(x: np.ndarray, wdtype: str = "f32", device="cuda"):
    if wdtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def rel_check(got, want, scale, rel=REL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    lim = rel * np.maximum(np.abs(want), scale)
    err = np.abs(got - want)
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside {rel} rel (max err {err.max():.3g})"


def tight_check(got, want, scale, what="", tol=TIGHT):
    want = np.asarray(want, np.float64)
    err = np.abs(np.asarray(got, np.float64) - want)
    lim = tol * np.maximum(np.abs(want), np.asarray(scale, np.float64))
    assert (err <= lim).all(), f"{what}: max err {err.max():.3g} above {tol} x rms"


def check_chain(gpu: dict, U, anchor, A, Bm, *, temperature=0.0, seeds=None, offset=0, topk=0,
                reqs=None, check_logits=True, oracle_kw=None, tight=TIGHT):
    """Compare the GPU chain outputs (numpy dict: tokens, tok_logit, lse, and
    optionally topk_idx/topk_prob/logits) with the oracle for requests ``reqs``.
    U/A/Bm are float64.  ``tight`` is the bar of the tighter check.  Returns
    the number of near-tie divergences."""
    B, gamma, V = U.shape
    reqs = range(B) if reqs is None else reqs
    ties = 0
    for b in reqs:
        forced = -np.ones((1, gamma), dtype=np.int64)
        kw = dict(temperature=temperature, seeds=None if seeds is None else seeds[b:b + 1],
                  offset=offset, topk=topk, keep_logits=True)
        if oracle_kw:
            kw.update({k: (v[b:b + 1] if k == "h" else v) for k, v in oracle_kw.items()})
        ref = o.markov_chain(U[b:b + 1], anchor[b:b + 1], A, Bm, **kw)
        for j in range(gamma):
            gt = int(gpu["tokens"][b, j])
            if gt != ref["tokens"][0, j]:
                assert ref["gap"][0, j] < TOKEN_GAP, (
                    f"request {b} position {j}: GPU token {gt} != oracle {ref['tokens'][0, j]} "
                    f"with gap {ref['gap'][0, j]:.3g}")
                ties += 1
                forced[0, :j + 1] = gpu["tokens"][b, :j + 1]
                ref = o.markov_chain(U[b:b + 1], anchor[b:b + 1], A, Bm, forced=forced, **kw)
                assert ref["score_max"][0, j] - ref["score_tok"][0, j] < TOKEN_GAP, (
                    f"request {b} position {j}: GPU token is not a near-tie choice")
        rms = np.sqrt((ref["logits"][0] ** 2).mean(axis=-1))          # [gamma]
        rel_check(gpu["tok_logit"][b], ref["tok_logit"][0], rms, what=f"tok_logit b={b}")
        rel_check(gpu["lse"][b], ref["lse"][0], rms, what=f"lse b={b}")
        tight_check(gpu["tok_logit"][b], ref["tok_logit"][0], rms, what=f"tok_logit b={b}", tol=tight)
        tight_check(gpu["lse"][b], ref["lse"][0], rms, what=f"lse b={b}", tol=tight)
        if check_logits and "logits" in gpu:
            rel_check(gpu["logits"][b], ref["logits"][0], rms[:, None], what=f"logits b={b}")
            tight_check(gpu["logits"][b], ref["logits"][0], rms[:, None], what=f"logits b={b}", tol=tight)
        if topk:
            for j in range(gamma):
                check_topk(gpu["topk_idx"][b, j], gpu["topk_prob"][b, j], ref["logits"][0, j],
                           ref["topk_idx"][0, j], ref["topk_prob"][0, j])
    return ties


def check_topk(gidx, gprob, ut, ridx, rprob, gap=TOKEN_GAP):
    """Top-k candidates: identical ids unless the oracle's k+1 largest values
    hold a near-tie (two neighbours closer than ``gap``), in which case the
    GPU's ids must carry the same values (to the gap) in non-increasing order;
    probabilities to the bars."""
    k = len(ridx)
    gidx = np.asarray(gidx, dtype=np.int64)
    assert len(set(gidx.tolist())) == k, "duplicate candidate ids"
    top = np.sort(ut)[::-1][:k + 1]
    near = (np.diff(top) > -gap).any()
    if not near:
        assert np.array_equal(gidx, ridx), f"top-k ids differ: {gidx} vs {ridx}"
    else:
        assert np.all(np.abs(ut[gidx] - ut[ridx]) < gap)
    rel_check(gprob, rprob, np.full(k, 1.0 / k), what="topk_prob")
    assert abs(float(np.sum(gprob)) - 1.0) < 1e-5
