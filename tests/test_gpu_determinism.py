"""Bit-identical reruns: every entry point, called twice on the same inputs
and workspace, returns the same bytes.  The library's reductions have a fixed
order and its only atomics act on integer order keys and counters, so no
result may depend on the order in which workgroups arrive."""
import numpy as np
import pytest
import torch

import synth
from semi_autoregressive_draft_amd import binding as bd
from tests.parity import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    a, b = a.detach().cpu().contiguous(), b.detach().cpu().contiguous()
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: reruns differ"


def _twice(fn):
    """Run fn() twice (each returns a dict of output tensors) and compare."""
    first = {k: v.clone() for k, v in fn().items()}
    torch.cuda.synchronize()
    second = fn()
    torch.cuda.synchronize()
    for k in first:
        _same(first[k], second[k], k)


@pytest.mark.parametrize("M,H,V", [(7, 2560, 20000), (448, 2560, 7000), (1792, 320, 3000)])
def test_lm_head_is_deterministic(M, H, V):
    dev = require_gpu()
    h = to_dev(synth.normal((M, H), 1.0, 41, synth.TID_H, "bf16"), "bf16")
    w = to_dev(synth.normal((V, H), 0.02, 41, synth.TID_WLM, "bf16"), "bf16")
    U = torch.empty((M, V), dtype=torch.float32, device=dev)

    def run():
        U.fill_(float("nan"))
        bd.dspark_lm_head(h, w, U)
        return {"U": U}
    _twice(run)


@pytest.mark.parametrize("N,V,k", [(1, 151936, 0),    # one launch with chunk exchanges
                                   (9, 30000, 0),     # split path
                                   (300, 4096, 0),    # many rows, each read once
                                   (160, 30004, 0),   # many rows, ragged chunks
                                   (5, 20000, 16),    # candidates, one launch
                                   (300, 4096, 16),   # candidates, one workgroup per row
                                   (64, 30004, 16)])  # candidates at 448 rows, one workgroup per row
def test_overlap_tau_is_deterministic(N, V, k):
    dev = require_gpu()
    g = synth.GAMMA
    teacher, draft = synth.overlap_inputs(N, V, 1.0, seed=43)
    t, d = to_dev(teacher), to_dev(draft)
    ci = cp = None
    if k:
        idx, prob = synth.candidates(N, V, k, seed=43)
        ci, cp, d = to_dev(idx), to_dev(prob), None
    valid = to_dev(synth.validity(N, seed=43, trunc_frac=0.3))
    alpha = torch.empty((N, g), dtype=torch.float32, device=dev)
    tau = torch.empty((N,), dtype=torch.float32, device=dev)
    acc = torch.empty((g,), dtype=torch.float64, device=dev)
    mean = torch.empty((1,), dtype=torch.float64, device=dev)
    ws = torch.zeros(bd.dspark_overlap_tau_workspace(N, g, V), dtype=torch.uint8, device=dev)

    def run():
        bd.dspark_overlap_tau(t, alpha, tau, draft=d, cand_idx=ci, cand_prob=cp, valid=valid,
                              accept_rate_at=acc, tau_mean=mean, ws=ws)
        return {"alpha": alpha, "tau": tau, "accept_rate_at": acc, "tau_mean": mean}
    _twice(run)


@pytest.mark.parametrize("N,V", [(1, 151936), (40, 5000)])
def test_compute_loss_is_deterministic(N, V):
    dev = require_gpu()
    g = synth.GAMMA
    teacher, draft = synth.overlap_inputs(N, V, 1.0, seed=47)
    t, d = to_dev(teacher), to_dev(draft)
    rng = synth.rng(47, synth.TID_CAND)
    target = to_dev(rng.integers(0, V, size=(N, g)).astype(np.int32))
    conf = to_dev(rng.standard_normal((N, g)).astype(np.float32))
    valid = to_dev(synth.validity(N, seed=47, trunc_frac=0.3))
    per = torch.empty((N, g, 4), dtype=torch.float32, device=dev)
    losses = torch.empty((4,), dtype=torch.float64, device=dev)
    ws = torch.zeros(bd.dspark_compute_loss_workspace(N, g, V), dtype=torch.uint8, device=dev)

    def run():
        bd.dspark_compute_loss(d, t, target, losses, conf_logit=conf, valid=valid, per_pos=per, ws=ws)
        return {"per_pos": per, "losses": losses}
    _twice(run)


@pytest.mark.parametrize("B,V", [(3, 20000), (64, 4096)])
def test_verify_is_deterministic(B, V):
    dev = require_gpu()
    g = synth.GAMMA
    gen = torch.Generator(device=dev)
    gen.manual_seed(53)
    draft = torch.randn((B, g, V), generator=gen, device=dev)
    target = torch.randn((B, g + 1, V), generator=gen, device=dev)
    target[:, :g].mul_(0.5).add_(draft)
    toks = torch.randint(0, V, (B, g), generator=gen, device=dev, dtype=torch.int32)
    lengths = torch.randint(0, g + 1, (B,), generator=gen, device=dev, dtype=torch.int32)
    seeds = torch.arange(B, dtype=torch.int64, device=dev).to(torch.uint64)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    prob = torch.empty((B, g), dtype=torch.float32, device=dev)
    ws = torch.empty(bd.dspark_verify_workspace(B, g, V), dtype=torch.uint8, device=dev)

    def run():
        bd.dspark_verify(target, draft, toks, seeds, acc, nxt, lengths=lengths, offset=5, accept_prob=prob, ws=ws)
        return {"accepted": acc, "next_token": nxt, "accept_prob": prob}
    _twice(run)


@pytest.mark.parametrize("R", [1, 256, 2340])
def test_prefix_schedule_is_deterministic(R):
    dev = require_gpu()
    g = synth.GAMMA
    a = to_dev(synth.survival_rows(R, g, seed=59))
    sps = to_dev(synth.sps_table(R * (g + 1), knee=R + R * g // 3, per_token_ms=20.0 / R))
    lengths = torch.empty((R,), dtype=torch.int32, device=dev)
    stats = torch.empty((3,), dtype=torch.float64, device=dev)

    def run():
        bd.dspark_prefix_schedule(a, sps, lengths, stats)
        return {"lengths": lengths, "stats": stats}
    _twice(run)


@pytest.mark.parametrize("B,V,r", [(64, 5000, 256), (3, 1000, 48)])
def test_apply_block_logits_is_deterministic(B, V, r):
    dev = require_gpu()
    g = synth.GAMMA
    U = to_dev(synth.base_logits(B, V, seed=61))
    A = to_dev(synth.normal((V, r), 0.25, 61, synth.TID_A, "bf16"), "bf16")
    Bm = to_dev(synth.normal((r, V), 0.25, 61, synth.TID_BM, "bf16"), "bf16")
    prev = to_dev(synth.rng(61, synth.TID_ANCHOR).integers(0, V, size=(B, g)).astype(np.int32))
    out = torch.empty((B, g, V), dtype=torch.float32, device=dev)

    def run():
        bd.dspark_apply_block_logits(U, prev, A, Bm, out)
        return {"logits": out}
    _twice(run)


@pytest.mark.parametrize("head", ["gated", "rnn"])
def test_head_variants_are_deterministic(head):
    dev = require_gpu()
    B, g, V, r, H = 40, synth.GAMMA, 3000, 64, 96
    U = to_dev(synth.base_logits(B, V, seed=67))
    A = to_dev(synth.normal((V, r), 0.25, 67, synth.TID_A, "bf16"), "bf16")
    Bm = to_dev(synth.normal((r, V), 0.25, 67, synth.TID_BM, "bf16"), "bf16")
    anchor = to_dev(synth.rng(67, synth.TID_ANCHOR).integers(0, V, size=B).astype(np.int32))
    h = to_dev(synth.normal((B, g, H), 1.0, 67, synth.TID_H, "bf16"), "bf16")
    rows = r if head == "gated" else 3 * r
    cols = H + r if head == "gated" else 2 * r + H
    W = to_dev(synth.normal((rows, cols), 0.1, 67, synth.TID_WG, "bf16"), "bf16")
    code = bd.HEAD_GATED if head == "gated" else bd.HEAD_RNN
    seeds = torch.arange(B, dtype=torch.int64, device=dev).to(torch.uint64)
    tokens = torch.empty((B, g), dtype=torch.int32, device=dev)
    lse = torch.empty((B, g), dtype=torch.float32, device=dev)
    ti = torch.empty((B, g, 8), dtype=torch.int32, device=dev)
    tp = torch.empty((B, g, 8), dtype=torch.float32, device=dev)
    ws = torch.zeros(bd.dspark_markov_propose_head_workspace(code, B, g, V, r, bd.BF16, 8), dtype=torch.uint8,
                     device=dev)

    def run():
        bd.dspark_markov_propose_head(code, U, anchor, A, Bm, tokens, h=h, W_g=W, temperature=0.8, seeds=seeds,
                                      topk=8, lse=lse, topk_idx=ti, topk_prob=tp, ws=ws)
        return {"tokens": tokens, "lse": lse, "topk_idx": ti, "topk_prob": tp}
    _twice(run)
