"""Pins of the oracle's training-loss forward ("DSpark 论文精读", §4.1;
"DeepSpec 训练全流程详解", §3.4): the printed position weights, library
routines for the cross entropy and the BCE-with-logits term, the overlap
identity for L1, degenerate distributions and the agreement of the pages'
aggregation forms when every position is valid."""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import synth
from oracle import dspark_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    rows, ratio = [], None
    with open(os.path.join(GOLDEN, "loss_decay_weights.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            p = line.split()
            if p[0] == "ratio":
                ratio = (float(p[1]), float(p[2]))
            else:
                rows.append((int(p[0]), float(p[1]), float(p[2])))
    return rows, ratio


def _case(B=3, gamma=7, V=64, seed=0, sigma=1.0):
    g = np.random.default_rng([seed, 5])
    draft = g.standard_normal((B, gamma, V))
    teacher = draft + sigma * g.standard_normal((B, gamma, V))
    target = g.integers(0, V, (B, gamma))
    conf = g.standard_normal((B, gamma))
    return draft, teacher, target, conf


def test_printed_position_weights():
    # the CE aggregate over two valid positions {0, j}: position 0 made
    # (almost) certain of its target (CE ~ 0), position j uniform (CE = log V),
    # gives w_j / w_0 = agg / (log V - agg)
    rows, (ratio, rtol) = _golden()
    V, gamma = 64, 7
    eff = {}
    for j, printed, tol in rows:
        draft = np.zeros((1, gamma, V))
        draft[0, 0, 5] = 80.0
        target = np.full((1, gamma), 5)
        valid = np.zeros((1, gamma), dtype=np.uint8)
        valid[0, 0] = 1
        valid[0, j] = 1
        _, (_, ce, _, _) = o.compute_loss(draft, draft, target, None, valid)
        w = 1.0 if j == 0 else ce / (math.log(V) - ce)
        eff[j] = w
        assert abs(w - printed) <= tol, (j, w, printed)
    assert abs(eff[0] / eff[6] - ratio) <= rtol


def test_cross_entropy_is_the_library_logsumexp_minus_the_target_logit():
    draft, teacher, target, conf = _case(seed=1)
    per_pos, _ = o.compute_loss(draft, teacher, target, conf)
    want = logsumexp(draft, axis=-1) - np.take_along_axis(draft, target[..., None], axis=-1)[..., 0]
    assert np.allclose(per_pos[..., 0], want, rtol=0, atol=1e-12)


def test_confidence_term_is_the_library_bce_with_logits():
    draft, teacher, target, conf = _case(seed=2)
    per_pos, (_, _, _, cf) = o.compute_loss(draft, teacher, target, conf)
    alpha = per_pos[..., 2]
    s = torch.from_numpy(conf)
    lib = torch.nn.functional.binary_cross_entropy_with_logits(s, torch.from_numpy(alpha), reduction="none")
    assert np.allclose(per_pos[..., 3], lib.numpy(), rtol=0, atol=1e-12)
    assert math.isclose(cf, float(lib.mean()), rel_tol=0, abs_tol=1e-12)


def test_l1_matches_the_overlap_identity_and_alpha_is_its_clamped_half():
    draft, teacher, target, conf = _case(seed=3, V=500)
    per_pos, _ = o.compute_loss(draft, teacher, target, conf)
    smin, _ = o.overlap_dense(teacher, draft)
    assert np.allclose(per_pos[..., 1], 2.0 - 2.0 * smin, atol=1e-12)
    assert np.allclose(per_pos[..., 2], np.clip(smin, 0.0, 1.0), atol=1e-12)


def test_degenerate_distributions():
    V, gamma = 32, 7
    same = np.random.default_rng(4).standard_normal((1, gamma, V))
    per_pos, (_, _, l1, _) = o.compute_loss(same, same, np.zeros((1, gamma), int))
    assert np.allclose(per_pos[..., 1], 0.0, atol=1e-12) and np.allclose(per_pos[..., 2], 1.0)
    a = np.full((1, gamma, V), -200.0)
    b = np.full((1, gamma, V), -200.0)
    a[..., 0] = 200.0
    b[..., 1] = 200.0                            # disjoint one-hot distributions
    per_pos, _ = o.compute_loss(a, b, np.zeros((1, gamma), int))
    assert np.allclose(per_pos[..., 1], 2.0) and np.allclose(per_pos[..., 2], 0.0)
    # a zero confidence logit costs log 2 whatever the label
    per_pos, _ = o.compute_loss(a, b, np.zeros((1, gamma), int), np.zeros((1, gamma)))
    assert np.allclose(per_pos[..., 3], math.log(2.0))


def test_normalised_weights_form_equals_the_masked_form_when_all_valid():
    # [P4] §4.1: normalised position weights applied to per-position batch
    # means; [P5] §3.4: masked weighted sum over the total weight
    draft, teacher, target, conf = _case(B=5, seed=6)
    per_pos, (total, ce, l1, cf) = o.compute_loss(draft, teacher, target, conf)
    w = np.exp(-np.arange(7) / 4.0)
    w = w / w.sum()
    assert math.isclose(ce, float((per_pos[..., 0].mean(axis=0) * w).sum()), rel_tol=1e-12)
    assert math.isclose(l1, float((per_pos[..., 1].mean(axis=0) * w).sum()), rel_tol=1e-12)
    assert math.isclose(total, 0.1 * ce + 0.9 * l1 + 1.0 * cf, rel_tol=1e-12)


def test_validity_masks_and_conf_weighting():
    draft, teacher, target, conf = _case(B=6, seed=7)
    valid = synth.validity(6, seed=7, trunc_frac=0.5, n_dummy=1)
    per_pos, (total, ce, l1, cf) = o.compute_loss(draft, teacher, target, conf, valid)
    assert not per_pos[5].any()                          # the dummy block reports zeros
    _, (_, ce_all, _, _) = o.compute_loss(draft[:5], teacher[:5], target[:5], conf[:5], valid[:5])
    assert math.isclose(ce, ce_all, rel_tol=1e-12)       # an all-invalid block carries no weight
    _, (_, _, _, cf_w) = o.compute_loss(draft, teacher, target, conf, valid, conf_decay=True)
    w = np.exp(-np.arange(7) / 4.0)[None, :] * valid
    assert math.isclose(cf_w, float((w * per_pos[..., 3]).sum() / w.sum()), rel_tol=1e-12)
    none = np.zeros((6, 7), dtype=np.uint8)
    _, losses = o.compute_loss(draft, teacher, target, conf, none)
    assert losses == (0.0, 0.0, 0.0, 0.0)


def test_teacher_forced_logits_are_the_block_bias():
    # apply_block_logits of [P4] §2.3: U + A[prev] Bm at every position, here
    # against a per-position loop of plain dot products
    g = np.random.default_rng(8)
    B, gamma, V, r = 2, 7, 40, 5
    U = g.standard_normal((B, gamma, V))
    A = g.standard_normal((V, r))
    Bm = g.standard_normal((r, V))
    prev = g.integers(0, V, (B, gamma))
    got = o.teacher_forced_logits(U, prev, A, Bm)
    for b in range(B):
        for j in range(gamma):
            for v in range(V):
                want = U[b, j, v] + sum(A[prev[b, j], k] * Bm[k, v] for k in range(r))
                assert abs(got[b, j, v] - want) < 1e-12
