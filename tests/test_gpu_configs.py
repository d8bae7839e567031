"""GPU parity at the five workloads' full sizes, through the same DraftPath the
benchmark times.  Where the oracle cannot recompute everything in seconds the
check covers sampled outputs (rows, requests) computed one by one by the
oracle, plus properties that hold at any size."""
import numpy as np
import pytest
import torch
from scipy import stats

import synth
from oracle import dspark_oracle as o
from semi_autoregressive_draft_amd import binding as bd
from semi_autoregressive_draft_amd.path import DraftPath
from tests.parity import (ALPHA_ABS, check_chain, rel_check, require_gpu, tight_check, to_dev)

pytestmark = pytest.mark.gpu


def _device_path(inp: synth.ProposeInputs, overlap):
    wd = inp.wdtype
    return DraftPath(
        to_dev(inp.h, wd), to_dev(inp.w_lm, wd), to_dev(inp.A, wd), to_dev(inp.Bm, wd),
        to_dev(inp.anchor), to_dev(inp.w_c, wd), inp.b_c, gamma=inp.gamma,
        temperature=inp.temperature,
        seeds=to_dev(inp.seeds) if inp.temperature > 0 else None, offset=inp.offset,
        topk=inp.topk, w_m=None if inp.w_m is None else to_dev(inp.w_m, wd),
        teacher=to_dev(inp.teacher) if overlap else None, overlap=overlap)


def _oracle_U_rows(inp: synth.ProposeInputs, rows, chunk=16384):
    """Oracle U for the given rows of h, over the full vocabulary (W widened to
    float64 a chunk of vocabulary rows at a time to bound host memory)."""
    h = o.to_f64(inp.h[rows], inp.wdtype)
    out = np.empty((len(rows), inp.V))
    for v0 in range(0, inp.V, chunk):
        out[:, v0:v0 + chunk] = o.lm_head(h, o.to_f64(inp.w_lm[v0:v0 + chunk], inp.wdtype))
    return out


def _check_requests(p: DraftPath, inp: synth.ProposeInputs, reqs):
    g = inp.gamma
    rows = [b * g + j for b in reqs for j in range(g)]
    U = _oracle_U_rows(inp, rows).reshape(len(reqs), g, inp.V)
    gpu = dict(tokens=p.tokens.cpu().numpy()[reqs], tok_logit=p.tok_logit.cpu().numpy()[reqs],
               lse=p.lse.cpu().numpy()[reqs])
    if inp.topk:
        gpu["topk_idx"] = p.topk_idx.cpu().numpy()[reqs]
        gpu["topk_prob"] = p.topk_prob.cpu().numpy()[reqs]
    if p.logits is not None:
        gpu["logits"] = p.logits.cpu().numpy()[reqs]
    A, Bm = o.to_f64(inp.A, inp.wdtype), o.to_f64(inp.Bm, inp.wdtype)
    seeds = inp.seeds[reqs] if inp.temperature > 0 else None
    check_chain(gpu, U, inp.anchor[reqs], A, Bm, temperature=inp.temperature, seeds=seeds,
                offset=inp.offset, topk=inp.topk)
    # U rows from the LM head
    Ug = p.U.cpu().numpy()[reqs]
    rms = np.sqrt((U ** 2).mean(axis=-1, keepdims=True))
    rel_check(Ug, U, rms, what="U")
    tight_check(Ug, U, rms, what="U")
    # confidence along the GPU's own tokens
    toks = gpu["tokens"]
    h3 = o.to_f64(inp.h, inp.wdtype).reshape(inp.B, g, inp.H)[reqs]
    c_ref, s_ref = o.confidence_survival(
        h3, o.to_f64(inp.w_c, inp.wdtype), inp.b_c,
        w_m=None if inp.w_m is None else o.to_f64(inp.w_m, inp.wdtype), A=A,
        anchor=inp.anchor[reqs], tokens=toks)
    assert np.abs(p.conf.cpu().numpy()[reqs] - c_ref).max() < 1e-5
    assert np.abs(p.survival.cpu().numpy()[reqs] - s_ref).max() < 1e-5
    return U, A, Bm, toks


def _check_overlap_for(p, inp, reqs, U, A, Bm, toks):
    """alpha/tau of the sampled requests against the oracle, along the GPU tokens."""
    g = inp.gamma
    prev = np.concatenate([inp.anchor[reqs, None], toks[:, :-1]], axis=1)
    ut = o.teacher_forced_logits(U, prev, A, Bm)
    t = inp.teacher[reqs].astype(np.float64)
    if p.overlap == "dense":
        a_raw, _ = o.overlap_dense(t, ut)
    else:
        idx = np.stack([[o.topk_indices(ut[i, j], inp.topk) for j in range(g)] for i in range(len(reqs))])
        e = np.exp(np.take_along_axis(ut, idx, -1) - np.take_along_axis(ut, idx[..., :1], -1))
        a_raw = o.overlap_sparse(t, idx, e / e.sum(-1, keepdims=True))
    _, tau_ref, _, _ = o.tau_metrics(a_raw)
    alpha = p.alpha.cpu().numpy()[reqs]
    assert np.abs(alpha - np.clip(a_raw, 0, 1)).max() < ALPHA_ABS
    assert np.abs(p.tau.cpu().numpy()[reqs] - tau_ref).max() < ALPHA_ABS


def test_config1_tiny_fp32_end_to_end():
    require_gpu()
    inp = synth.propose_inputs(**{k: v for k, v in synth.CONFIGS["c1_tiny_fp32"].items()})
    p = _device_path(inp, "dense")
    p.run()
    p.check()                                   # device status words: no wait ran out
    reqs = list(range(inp.B))
    U, A, Bm, toks = _check_requests(p, inp, reqs)
    _check_overlap_for(p, inp, reqs, U, A, Bm, toks)
    a_ref, tau_ref, acc_ref, mean_ref = o.tau_metrics(p.alpha.cpu().numpy().astype(np.float64))
    assert abs(float(p.tau_mean.cpu()[0]) - mean_ref) < ALPHA_ABS


def test_config2_qwen3_4b_single_request_full():
    require_gpu()
    cfg = dict(synth.CONFIGS["c2_qwen3_4b_b1"])
    cfg["topk"] = 16                            # top-16 rides along; greedy tokens unchanged
    inp = synth.propose_inputs(**cfg)
    p = _device_path(inp, "dense")
    p.run()
    p.check()                                   # device status words: no wait ran out
    U, A, Bm, toks = _check_requests(p, inp, [0])
    _check_overlap_for(p, inp, [0], U, A, Bm, toks)


def _spread(B, step):
    """Every step-th request plus the last one: each 16-request group of the
    batched kernels (one wave per 16 requests) contributes at least one."""
    return sorted(set(range(0, B, step)) | {B - 1})


def test_config3_batch64_gumbel_sampled_requests():
    require_gpu()
    cfg = dict(synth.CONFIGS["c3_batch64_gumbel"])
    cfg["topk"] = 16                            # as timed: top-16 candidates and the sparse overlap
    inp = synth.propose_inputs(**cfg)
    p = _device_path(inp, "topk")
    p.run()
    p.check()                                   # device status words: no wait ran out
    reqs = _spread(inp.B, 2)                    # 33 of 64 requests
    U, A, Bm, toks = _check_requests(p, inp, reqs)
    _check_overlap_for(p, inp, reqs, U, A, Bm, toks)
    # every request's tokens are valid ids and the lse bounds its logit
    toks = p.tokens.cpu().numpy()
    assert toks.min() >= 0 and toks.max() < inp.V
    assert np.all(p.tok_logit.cpu().numpy() <= p.lse.cpu().numpy())


def test_config5_high_load_top16_sampled_requests():
    require_gpu()
    inp = synth.propose_inputs(**synth.CONFIGS["c5_flash_next_b256"])
    p = _device_path(inp, "topk")
    p.run()
    p.check()                                   # device status words: no wait ran out
    reqs = _spread(inp.B, 8)                    # 33 of 256 requests
    U, A, Bm, toks = _check_requests(p, inp, reqs)
    _check_overlap_for(p, inp, reqs, U, A, Bm, toks)
    # properties over every request: survival non-increasing, candidates sorted
    s = p.survival.cpu().numpy()
    assert np.all(np.diff(s, axis=1) <= 0)
    pr = p.topk_prob.cpu().numpy()
    assert np.allclose(pr.sum(-1), 1.0, atol=1e-5) and np.all(np.diff(pr, axis=-1) <= 1e-7)
    # the first candidate is the greedy token (up to rounding near-ties)
    assert (p.topk_idx.cpu().numpy()[..., 0] != p.tokens.cpu().numpy()).mean() < 1e-3


@pytest.mark.parametrize("sigma", [0.5, 1.0, 2.0])
def test_config4_offline_eval_full_size(sigma):
    dev = require_gpu()
    cfg = synth.CONFIGS["c4_offline_eval"]
    N, V, g = cfg["N"], cfg["V"], synth.GAMMA
    teacher, draft = synth.device_overlap_inputs(N, V, sigma, dev, seed=0)
    valid = synth.validity(N, seed=0, trunc_frac=cfg["trunc_frac"])
    alpha = torch.empty((N, g), dtype=torch.float32, device=dev)
    tau = torch.empty((N,), dtype=torch.float32, device=dev)
    acc = torch.empty((g,), dtype=torch.float64, device=dev)
    mean = torch.empty((1,), dtype=torch.float64, device=dev)
    bd.dspark_overlap_tau(teacher, alpha, tau, draft=draft, valid=to_dev(valid),
                          accept_rate_at=acc, tau_mean=mean)
    torch.cuda.synchronize()
    al, ta = alpha.cpu().numpy(), tau.cpu().numpy()
    # sampled blocks, recomputed by the oracle from the same device inputs
    blocks = np.random.default_rng(1).choice(N, size=12, replace=False)
    t = teacher[torch.as_tensor(blocks, device=dev)].cpu().numpy().astype(np.float64)
    d = draft[torch.as_tensor(blocks, device=dev)].cpu().numpy().astype(np.float64)
    a_raw, _ = o.overlap_dense(t, d)
    a_ref, tau_ref, _, _ = o.tau_metrics(a_raw, valid[blocks])
    assert np.abs(al[blocks] - a_ref).max() < ALPHA_ABS
    assert np.abs(ta[blocks] - tau_ref).max() < ALPHA_ABS
    # aggregates: exact recomputation from the GPU's own per-slot alphas...
    _, _, acc_ref, mean_ref = o.tau_metrics(al.astype(np.float64), valid)
    assert np.abs(acc.cpu().numpy() - acc_ref).max() < 1e-6
    assert abs(float(mean.cpu()[0]) - mean_ref) < 1e-5
    # ...and the large-vocabulary closed form 2 Phi(-sigma/2) for the mean overlap
    limit = 2 * stats.norm.cdf(-sigma / 2)
    assert np.abs(acc.cpu().numpy() - limit).max() < 5e-3
    full = valid.all(axis=1)
    abar = limit
    assert abs(ta[full].mean() - (1 + abar * (1 - abar ** 7) / (1 - abar))) < 0.03
    del teacher, draft
    torch.cuda.empty_cache()


def test_teacher_forced_block_logits_full_size():
    """Teacher-forced block logits at the training shape (512 blocks x 7
    positions, V = 151936, r = 256): 2.18 GB of logits, which the library
    splits into row chunks below 2 GiB.  Rows on both sides of the chunk
    boundary and random rows are recomputed by the oracle one by one."""
    dev = require_gpu()
    N, g, V, r = 512, synth.GAMMA, 151936, 256
    gen = torch.Generator(device=dev)
    gen.manual_seed(71)
    U = torch.randn((N, g, V), generator=gen, device=dev)
    A = (torch.randn((V, r), generator=gen, device=dev) * 0.25).to(torch.bfloat16)
    Bm = (torch.randn((r, V), generator=gen, device=dev) * 0.25).to(torch.bfloat16)
    prev = torch.randint(0, V, (N, g), generator=gen, device=dev, dtype=torch.int32)
    out = torch.full((N, g, V), float("nan"), dtype=torch.float32, device=dev)
    bd.dspark_apply_block_logits(U, prev, A, Bm, out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    rows_total = N * g
    chunk = (2 ** 31 - 1) // (V * 4) // 16 * 16
    rows = sorted(set([0, 1, 15, 16, chunk - 1, chunk, chunk + 1, rows_total - 1]
                      + list(np.random.default_rng(71).choice(rows_total, 8, replace=False))))
    ridx = torch.as_tensor(rows, device=dev)
    U_r = U.view(rows_total, V)[ridx].cpu().numpy().astype(np.float64)
    prev_r = prev.view(rows_total)[ridx].cpu().numpy().reshape(-1, 1)
    A64 = A.float().cpu().numpy().astype(np.float64)
    Bm64 = Bm.float().cpu().numpy().astype(np.float64)
    want = o.teacher_forced_logits(U_r[:, None, :], prev_r, A64, Bm64)[:, 0]
    got = out.view(rows_total, V)[ridx].cpu().numpy()
    tight_check(got, want, np.abs(want).max(axis=-1, keepdims=True), what="block logits")
    del U, out
    torch.cuda.empty_cache()
