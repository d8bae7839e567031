"""dspark_markov_propose_noalloc (the library's static scratch as workspace)
against dspark_markov_propose with a caller workspace: two calls in a row,
the second with a smaller input, each compared output by output.  Both entry
points run the same kernels with the same reduction order, so the outputs
must agree bit for bit."""
import numpy as np
import pytest
import torch

import synth
from semi_autoregressive_draft_amd import binding as bd
from tests.parity import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _inputs(B, V, r, seed):
    U = synth.base_logits(B, V, seed=seed)
    A = synth.normal((V, r), 0.25, seed, synth.TID_A, "bf16")
    Bm = synth.normal((r, V), 0.25, seed, synth.TID_BM, "bf16")
    anchor = synth.rng(seed, synth.TID_ANCHOR).integers(0, V, size=B).astype(np.int32)
    return to_dev(U), to_dev(anchor), to_dev(A, "bf16"), to_dev(Bm, "bf16")


def _outputs(B, gamma, V, topk, dump, dev):
    f32 = dict(dtype=torch.float32, device=dev)
    return dict(tokens=torch.full((B, gamma), -7, dtype=torch.int32, device=dev),
                tok_logit=torch.full((B, gamma), float("nan"), **f32),
                lse=torch.full((B, gamma), float("nan"), **f32),
                topk_idx=torch.full((B, gamma, topk), -7, dtype=torch.int32, device=dev) if topk else None,
                topk_prob=torch.full((B, gamma, topk), float("nan"), **f32) if topk else None,
                logits_out=torch.full((B, gamma, V), float("nan"), **f32) if dump else None,
                status=torch.full((1,), -1, dtype=torch.int32, device=dev))


def _call(fn, ins, out, T, seeds, topk, **extra):
    U, anchor, A, Bm = ins
    fn(U, anchor, A, Bm, out["tokens"], temperature=T, seeds=seeds, offset=9, topk=topk,
       tok_logit=out["tok_logit"], lse=out["lse"], topk_idx=out["topk_idx"], topk_prob=out["topk_prob"],
       logits_out=out["logits_out"], status=out["status"], **extra)


# (B, V, r, T, topk, U~ dump) of the first and the second (smaller) call
CASES = [
    # resident chain (B <= 16, r = 256), then a smaller resident chain
    ((4, 151936, 256, 0.0, 16, True), (2, 50000, 256, 0.0, 8, False)),
    # per-position chain with sampling and top-16 at the largest batch the
    # scratch holds, then a smaller per-position call
    ((64, 151936, 256, 1.0, 16, False), (20, 30000, 64, 0.7, 4, True)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_the_workspace_entry_point(first, second):
    dev = require_gpu()
    gamma = 7
    for call, (B, V, r, T, topk, dump) in enumerate((first, second)):
        print(f"noalloc call {call}: B={B} V={V} r={r} T={T} topk={topk} dump={dump}", flush=True)
        ins = _inputs(B, V, r, seed=71 + call)
        seeds = torch.arange(B, dtype=torch.int64, device=dev).to(torch.uint64) if T > 0 else None
        ref = _outputs(B, gamma, V, topk, dump, dev)
        ws = torch.zeros(bd.dspark_markov_propose_workspace(B, gamma, V, topk), dtype=torch.uint8, device=dev)
        _call(bd.dspark_markov_propose, ins, ref, T, seeds, topk, ws=ws)
        got = _outputs(B, gamma, V, topk, dump, dev)
        _call(bd.dspark_markov_propose_noalloc, ins, got, T, seeds, topk)
        torch.cuda.synchronize()
        bd.check_device_status(ref["status"], "dspark_markov_propose")
        bd.check_device_status(got["status"], "dspark_markov_propose_noalloc")
        for key, want in ref.items():
            if want is None:
                continue
            have = got[key]
            assert torch.equal(have.cpu().view(torch.uint8), want.cpu().view(torch.uint8)), (
                f"call {call}: {key} differs from dspark_markov_propose")
        toks = got["tokens"].cpu().numpy()
        assert toks.min() >= 0 and toks.max() < V


def test_noalloc_rejects_sizes_beyond_its_scratch():
    dev = require_gpu()
    B, gamma, V, r, topk = 256, 7, 151936, 256, 16
    assert bd.dspark_markov_propose_workspace(B, gamma, V, topk) > 64 << 20
    U = torch.empty((B, gamma, V), dtype=torch.float32, device=dev)
    anchor = torch.zeros((B,), dtype=torch.int32, device=dev)
    A = torch.zeros((V, r), dtype=torch.bfloat16, device=dev)
    Bm = torch.zeros((r, V), dtype=torch.bfloat16, device=dev)
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    ti = torch.empty((B, gamma, topk), dtype=torch.int32, device=dev)
    tp = torch.empty((B, gamma, topk), dtype=torch.float32, device=dev)
    with pytest.raises(bd.DsparkError) as e:
        bd.dspark_markov_propose_noalloc(U, anchor, A, Bm, tokens, topk=topk, topk_idx=ti, topk_prob=tp)
    assert e.value.status == bd.EWORKSPACE and "static scratch" in str(e.value)
