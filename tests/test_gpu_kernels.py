"""GPU parity of each C-ABI entry point against the fp64 oracle, at sizes the
oracle finishes in seconds that still span several tiles and a ragged tail,
plus degenerate cases (ties, zero transitions, invalid blocks)."""
import numpy as np
import pytest
import torch

import synth
from oracle import dspark_oracle as o
from semi_autoregressive_draft_amd import binding as bd
from tests.parity import (ALPHA_ABS, REL, TIGHT, TOKEN_GAP, check_chain, check_topk, rel_check, require_gpu, tight_check,
                          to_dev)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- S1
@pytest.mark.parametrize("M,H,V,wdtype", [
    (7, 256, 4096, "f32"),        # tiny reference config shape
    (5, 100, 333, "f32"),         # ragged everything
    (1, 256, 5000, "bf16"),       # skinny path, ragged vocabulary tail
    (7, 296, 5000, "bf16"),       # skinny, K not a multiple of 32
    (12, 2560, 1000, "bf16"),     # skinny, largest M that keeps h in 64 KB of LDS
    (13, 2560, 1000, "bf16"),     # tiled path, ragged M, fewer tiles than XCDs
    (130, 296, 5000, "bf16"),     # tiled, ragged M/K/V tiles
    (448, 320, 3000, "bf16"),
    (600, 136, 2104, "bf16"),     # several row tiles, K tail, vocabulary tail; 21 tiles over 8 XCD runs
    (257, 8, 264, "bf16"),        # tiled, one K stage that is all tail, one row past a tile
    (270, 64, 1032, "bf16"),      # tiled, exactly one full K stage
    # more tiles than compute units (several rounds of workgroups per XCD)
    (600, 136, 50000, "bf16"),    # 3 row tiles, K tail
    (300, 200, 40008, "bf16"),    # ragged M, K tail, vocabulary tail
    # 8 row tiles (the last 208 rows), a K tail of 8 and a last vocabulary tile of 8 columns: the
    # DMA of waves 0-3 (own and partner blocks), its tail zeroing and the range-checked rows at once
    (2000, 264, 40008, "bf16"),
])
def test_lm_head_parity(M, H, V, wdtype):
    dev = require_gpu()
    h = synth.normal((M, H), 1.0, 11, synth.TID_H, wdtype)
    w = synth.normal((V, H), 0.02, 11, synth.TID_WLM, wdtype)
    U = torch.full((M, V), float("nan"), dtype=torch.float32, device=dev)
    bd.dspark_lm_head(to_dev(h, wdtype), to_dev(w, wdtype), U)
    got = U.cpu().numpy()
    want = o.lm_head(o.to_f64(h, wdtype), o.to_f64(w, wdtype))
    rms = np.sqrt((want ** 2).mean(axis=1, keepdims=True))
    rel_check(got, want, rms, what="U")
    tight_check(got, want, rms, what="U")


# ----------------------------------------------------------------------------- S2-S4
def _run_markov(U, anchor, A, Bm, wdtype, *, T=0.0, seeds=None, offset=0, topk=0, dump=True, ws=None):
    dev = require_gpu()
    B, gamma, V = U.shape
    Ud = to_dev(U)
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    tl = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    ls = torch.empty_like(tl)
    ti = torch.empty((B, gamma, topk), dtype=torch.int32, device=dev) if topk else None
    tp = torch.empty((B, gamma, topk), dtype=torch.float32, device=dev) if topk else None
    lo = torch.empty((B, gamma, V), dtype=torch.float32, device=dev) if dump else None
    sd = to_dev(seeds) if seeds is not None else None
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    bd.dspark_markov_propose(Ud, to_dev(anchor), to_dev(A, wdtype), to_dev(Bm, wdtype), tokens,
                             temperature=T, seeds=sd, offset=offset, topk=topk, tok_logit=tl,
                             lse=ls, topk_idx=ti, topk_prob=tp, logits_out=lo, ws=ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == bd.OK, "the device status word must report a completed call"
    out = dict(tokens=tokens.cpu().numpy(), tok_logit=tl.cpu().numpy(), lse=ls.cpu().numpy())
    if topk:
        out["topk_idx"], out["topk_prob"] = ti.cpu().numpy(), tp.cpu().numpy()
    if dump:
        out["logits"] = lo.cpu().numpy()
    return out


def _markov_case(B, V, r, wdtype, seed=3, mstd=0.25):
    U = synth.base_logits(B, V, seed=seed)
    A = synth.normal((V, r), mstd, seed, synth.TID_A, wdtype)
    Bm = synth.normal((r, V), mstd, seed, synth.TID_BM, wdtype)
    anchor = synth.rng(seed, synth.TID_ANCHOR).integers(0, V, size=B).astype(np.int32)
    return U, anchor, A, Bm


@pytest.fixture(params=["resident", "per_position"])
def chain_path(request, monkeypatch):
    """Run each Markov case through both chain implementations (the resident
    chain only where it applies)."""
    if request.param == "per_position":
        monkeypatch.setenv("DSPARK_MARKOV_RESIDENT", "0")
    return request.param


@pytest.mark.parametrize("B,V,r,wdtype,T,topk", [
    (1, 5000, 256, "bf16", 0.0, 0),     # one request (per position: r split over 4 waves)
    (3, 5000, 64, "bf16", 0.0, 0),      # r split over 2 waves
    (5, 4096, 32, "bf16", 0.7, 0),      # sampled, no r split
    (17, 5000, 128, "bf16", 0.0, 0),    # 64-column tiles, 2 request groups, ragged
    (40, 3000, 256, "bf16", 1.0, 0),    # 3 request groups, sampled
    (70, 2000, 64, "bf16", 0.0, 16),    # 5 request groups, top-16
    (150, 3000, 128, "bf16", 0.0, 16),  # two groups of 16 per wave, ragged request block
    (300, 2000, 64, "bf16", 1.0, 0),    # two request blocks, sampled
    (64, 3000, 256, "bf16", 1.0, 0),    # 4 waves of one group, 2 Bm chunks per wave, sampled
    (129, 2008, 256, "bf16", 0.0, 16),  # 8 waves x 2 request blocks, ragged requests and last tile
    (20, 1000, 32, "bf16", 0.0, 0),     # one chunk, 2 waves
    (2, 5000, 256, "bf16", 0.0, 32),    # top-32
    (1, 1000, 64, "bf16", 1.0, 16),     # sampled with top-16
    (1, 4096, 32, "f32", 0.0, 0),       # tiny reference config
    (3, 1000, 48, "f32", 1.0, 5),       # float32 tables, any rank
])
def test_markov_parity(B, V, r, wdtype, T, topk, chain_path):
    U, anchor, A, Bm = _markov_case(B, V, r, wdtype)
    seeds = np.arange(B, dtype=np.uint64) * 7919 + 3 if T > 0 else None
    gpu = _run_markov(U, anchor, A, Bm, wdtype, T=T, seeds=seeds, offset=5, topk=topk)
    check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, wdtype), o.to_f64(Bm, wdtype),
                temperature=T, seeds=seeds, offset=5, topk=topk)


@pytest.mark.parametrize("B,V,r,T,topk,wg", [
    (1, 5000, 256, 0.0, 16, 0),         # one group per workgroup
    (1, 5000, 256, 0.0, 0, 8),          # 10 groups per workgroup: 8 in registers, 2 in LDS
    (1, 3000, 128, 1.0, 8, 4),          # r = 128: 2 register groups per wave, sampled
    (1, 2504, 64, 0.0, 16, 1),          # r = 64, one workgroup: 32 register + 8 LDS groups, ragged
    (5, 5000, 256, 0.0, 8, 8),          # several requests, LDS groups
    (16, 4104, 256, 0.7, 16, 8),        # 16 requests, sampled, top-16, ragged last group
    (2, 5000, 256, 0.0, 32, 0),         # top-32; the last workgroup has 8 live columns
])
def test_markov_resident_chain(B, V, r, T, topk, wg, monkeypatch):
    # the resident chain with the operand share spread as on smaller devices
    # (a workgroup cap puts more groups, and LDS-held groups, in each workgroup)
    require_gpu()
    if wg:
        monkeypatch.setenv("DSPARK_MARKOV_WORKGROUPS", str(wg))
    n = bd.dspark_markov_propose_plan(B, V, r)
    assert n > 0 and (wg == 0 or n == wg)
    U, anchor, A, Bm = _markov_case(B, V, r, "bf16", seed=6)
    seeds = np.arange(B, dtype=np.uint64) * 104729 + 1 if T > 0 else None
    gpu = _run_markov(U, anchor, A, Bm, "bf16", T=T, seeds=seeds, offset=2, topk=topk)
    check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, "bf16"), o.to_f64(Bm, "bf16"),
                temperature=T, seeds=seeds, offset=2, topk=topk)


@pytest.mark.parametrize("B,V,r,T,topk", [
    (32, 5000, 256, 0.0, 16),      # the copy pays off from B*gamma = 12 rows at this V
    (24, 3000, 128, 0.9, 32),      # sampled, top-32, r = 128
    (40, 2008, 64, 0.0, 8),        # ragged last tile of the transpose (2008 = 31 * 64 + 24)
])
def test_markov_topk_with_transposed_bm(B, V, r, T, topk):
    # the larger workspace turns on the transposed-Bm recompute of the top-k
    # candidates (the copy stored by position 0's step kernel when no dump is
    # asked for, else by the copy kernel); the smaller one keeps the strided
    # recompute: all exact, and the same top-k
    dev = require_gpu()
    U, anchor, A, Bm = _markov_case(B, V, r, "bf16", seed=9)
    seeds = np.arange(B, dtype=np.uint64) * 31 + 5 if T > 0 else None
    small = bd.dspark_markov_propose_workspace(B, 7, V, topk)
    big = bd.dspark_markov_propose_workspace_bmt(bd.HEAD_LINEAR, B, 7, V, r, bd.BF16, topk)
    assert big >= small + r * V * 2
    ids = []
    for n, dump in ((big, True), (big, False), (small, False)):
        ws = torch.zeros(n, dtype=torch.uint8, device=dev)
        gpu = _run_markov(U, anchor, A, Bm, "bf16", T=T, seeds=seeds, offset=4, topk=topk, ws=ws, dump=dump)
        check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, "bf16"), o.to_f64(Bm, "bf16"),
                    temperature=T, seeds=seeds, offset=4, topk=topk, check_logits=dump)
        ids.append(gpu["topk_idx"])
    # the same BmT either way: the same recompute, bit for bit
    assert np.array_equal(ids[0], ids[1])


def test_markov_workspace_is_left_ready_for_the_next_call(monkeypatch):
    # one zero-filled workspace serves resident and per-position calls of
    # different shapes in turn: each call must leave it as the next expects
    dev = require_gpu()
    ws = torch.zeros(bd.dspark_markov_propose_workspace(3, 7, 5000, 16), dtype=torch.uint8, device=dev)
    for B, r, resident, T in [(1, 256, True, 0.0), (3, 256, True, 1.0), (1, 64, False, 0.0),
                              (2, 256, True, 0.0), (1, 256, True, 0.0)]:
        monkeypatch.setenv("DSPARK_MARKOV_RESIDENT", "1" if resident else "0")
        assert (bd.dspark_markov_propose_plan(B, 5000, r) > 0) == resident
        U, anchor, A, Bm = _markov_case(B, 5000, r, "bf16", seed=B + r)
        seeds = np.arange(B, dtype=np.uint64) + 11 if T > 0 else None
        Ud = to_dev(U)
        tokens = torch.empty((B, 7), dtype=torch.int32, device=dev)
        tl = torch.empty((B, 7), dtype=torch.float32, device=dev)
        ls = torch.empty_like(tl)
        ti = torch.empty((B, 7, 16), dtype=torch.int32, device=dev)
        tp = torch.empty((B, 7, 16), dtype=torch.float32, device=dev)
        bd.dspark_markov_propose(Ud, to_dev(anchor), to_dev(A, "bf16"), to_dev(Bm, "bf16"), tokens,
                                 temperature=T, seeds=to_dev(seeds) if seeds is not None else None,
                                 topk=16, tok_logit=tl, lse=ls, topk_idx=ti, topk_prob=tp, ws=ws)
        torch.cuda.synchronize()
        gpu = dict(tokens=tokens.cpu().numpy(), tok_logit=tl.cpu().numpy(), lse=ls.cpu().numpy(),
                   topk_idx=ti.cpu().numpy(), topk_prob=tp.cpu().numpy())
        check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, "bf16"), o.to_f64(Bm, "bf16"),
                    temperature=T, seeds=seeds, topk=16)


def test_markov_plan_follows_the_shape_rules(monkeypatch):
    require_gpu()
    assert bd.dspark_markov_propose_plan(1, 151936, 256) > 0
    assert bd.dspark_markov_propose_plan(16, 151936, 256) > 0
    assert bd.dspark_markov_propose_plan(17, 151936, 256) == 0    # batched step kernels
    assert bd.dspark_markov_propose_plan(2, 5000, 64) == 0        # B > 1 needs r = 256
    assert bd.dspark_markov_propose_plan(1, 5000, 48, bd.F32) == 0
    monkeypatch.setenv("DSPARK_MARKOV_RESIDENT", "0")
    assert bd.dspark_markov_propose_plan(1, 151936, 256) == 0


def test_markov_walks_a_permutation(chain_path):
    # A = identity rows, Bm = 4 * permutation, |U| < 1.6: x_j = pi^{j+1}(anchor).
    # All values are exact in bf16, so this checks the previous-token wiring
    # (anchor at slot 0, token j-1 at slot j) independently of rounding.
    V = r = 64
    rng = np.random.default_rng(5)
    pi = rng.permutation(V)
    A = synth.bf16_bits(np.eye(V, dtype=np.float32))
    Bmf = np.zeros((r, V), dtype=np.float32)
    Bmf[np.arange(r), pi] = 4.0
    U = rng.uniform(-1.6, 1.6, size=(3, 7, V)).astype(np.float32)
    anchor = np.array([0, 17, 63], dtype=np.int32)
    gpu = _run_markov(U, anchor, A, synth.bf16_bits(Bmf), "bf16")
    for b in range(3):
        t = anchor[b]
        for j in range(7):
            t = pi[t]
            assert gpu["tokens"][b, j] == t


def test_markov_ties_take_lowest_index_and_slow_topk_path(chain_path):
    # constant logits and zero transitions: every column ties, so the token is
    # column 0 and the top-k candidate lists overflow into the exact slow path
    B, V, r, k = 2, 1024, 32, 16
    U = np.zeros((B, 7, V), dtype=np.float32)
    zeros_A = synth.bf16_bits(np.zeros((V, r), np.float32))
    zeros_B = synth.bf16_bits(np.zeros((r, V), np.float32))
    gpu = _run_markov(U, np.array([3, 9], np.int32), zeros_A, zeros_B, "bf16", topk=k)
    assert np.all(gpu["tokens"] == 0)
    assert np.all(gpu["topk_idx"] == np.arange(k))
    assert np.allclose(gpu["topk_prob"], 1.0 / k, atol=1e-7)
    assert np.allclose(gpu["lse"], np.log(V), atol=1e-5)


@pytest.mark.parametrize("B,V,r,topk", [(20, 2008, 64, 8), (3, 1024, 32, 4)])
def test_markov_nan_row_keeps_gathers_inside_the_table(B, V, r, topk):
    # per-position chain (wide step for B > 16, the small-batch step below): a
    # request whose first row is all NaN has no orderable value; its token is
    # -1 or some column, the next position gathers a table row clamped into
    # [0, V), and every other request is unaffected
    U, anchor, A, Bm = _markov_case(B, V, r, "bf16", seed=12)
    Un = U.copy()
    Un[1, 0, :] = np.nan
    ref = _run_markov(U, anchor, A, Bm, "bf16", topk=topk, dump=False)
    got = _run_markov(Un, anchor, A, Bm, "bf16", topk=topk, dump=False)
    t = got["tokens"][1]
    assert np.all((t >= -1) & (t < V)) and np.all(t[1:] >= 0)
    others = [b for b in range(B) if b != 1]
    assert np.array_equal(got["tokens"][others], ref["tokens"][others])
    assert np.array_equal(got["topk_idx"][others], ref["topk_idx"][others])
    ids = got["topk_idx"][1]                          # -1 where no candidate was ordered
    assert np.all((ids >= -1) & (ids < V))


@pytest.mark.parametrize("gamma,B,V,r,T,topk,dump", [
    (1, 40, 3000, 256, 0.0, 16, False),   # one position: the step that stores BmT is the whole chain
    (3, 40, 2008, 64, 0.8, 8, True),      # sampled, ragged last tile, with the dump
    (16, 20, 3000, 128, 0.0, 16, False),  # the longest block
    (1, 2, 5000, 256, 0.0, 16, False),    # small batch (resident chain where it applies)
    (16, 3, 5000, 256, 1.0, 0, True),
])
def test_markov_other_block_lengths(gamma, B, V, r, T, topk, dump, chain_path):
    # blocks of other lengths than 7, through both chain paths and the
    # transposed-Bm workspace
    dev = require_gpu()
    U = synth.base_logits(B, V, gamma=gamma, seed=31)
    A = synth.normal((V, r), 0.25, 31, synth.TID_A, "bf16")
    Bm = synth.normal((r, V), 0.25, 31, synth.TID_BM, "bf16")
    anchor = synth.rng(31, synth.TID_ANCHOR).integers(0, V, size=B).astype(np.int32)
    seeds = np.arange(B, dtype=np.uint64) * 5 + 2 if T > 0 else None
    n = (bd.dspark_markov_propose_workspace_bmt(bd.HEAD_LINEAR, B, gamma, V, r, bd.BF16, topk) if topk
         else bd.dspark_markov_propose_workspace(B, gamma, V, topk))
    ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    gpu = _run_markov(U, anchor, A, Bm, "bf16", T=T, seeds=seeds, offset=1, topk=topk, dump=dump, ws=ws)
    check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, "bf16"), o.to_f64(Bm, "bf16"),
                temperature=T, seeds=seeds, offset=1, topk=topk)


@pytest.mark.parametrize("T", [0.0, 0.8])
def test_markov_without_dump_matches_with_dump(T):
    # the per-position wide step has a variant that issues no U~ dump stores
    # (chain with no dump requested): the same tokens, logits, lse and top-k,
    # bit for bit
    B, V, r = 40, 5000, 256
    U, anchor, A, Bm = _markov_case(B, V, r, "bf16", seed=14)
    seeds = np.arange(B, dtype=np.uint64) * 7 + 3 if T > 0 else None
    with_dump = _run_markov(U, anchor, A, Bm, "bf16", T=T, seeds=seeds, offset=2, topk=8, dump=True)
    no_dump = _run_markov(U, anchor, A, Bm, "bf16", T=T, seeds=seeds, offset=2, topk=8, dump=False)
    for k in no_dump:
        assert np.array_equal(no_dump[k].view(np.uint8), with_dump[k].view(np.uint8)), k


def test_markov_zero_transition_is_parallel_argmax():
    B, V, r = 4, 3000, 64
    U = synth.base_logits(B, V, seed=8)
    gpu = _run_markov(U, np.zeros(B, np.int32), synth.bf16_bits(np.zeros((V, r), np.float32)),
                      synth.normal((r, V), 0.25, 8, synth.TID_BM, "bf16"), "bf16", dump=False)
    assert np.array_equal(gpu["tokens"], U.argmax(axis=-1))


@pytest.mark.parametrize("B", [1, 33])
def test_markov_is_deterministic(B):
    U, anchor, A, Bm = _markov_case(B, 5000, 256, "bf16", seed=4)
    seeds = np.arange(B, dtype=np.uint64)
    a = _run_markov(U, anchor, A, Bm, "bf16", T=1.0, seeds=seeds, topk=16)
    b = _run_markov(U, anchor, A, Bm, "bf16", T=1.0, seeds=seeds, topk=16)
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


# ----------------------------------------------------------------------------- S1 + S5
@pytest.mark.parametrize("B,gamma,H,V,wdtype", [
    (1, 7, 2560, 3000, "bf16"),     # one launch (skinny LM head, workgroup 0 adds S5)
    (2, 8, 512, 1032, "bf16"),      # one launch, M = 16
    (3, 7, 264, 520, "bf16"),       # M = 21: the GEMM and the S5 kernel
    (1, 5, 96, 300, "f32"),         # fp32: two launches
])
def test_lm_head_confidence_parity(B, gamma, H, V, wdtype):
    dev = require_gpu()
    h = synth.normal((B, gamma, H), 1.0, 5, synth.TID_H, wdtype)
    w = synth.normal((V, H), 0.05, 5, synth.TID_WLM, wdtype)
    w_c = synth.normal((H,), 0.05, 5, synth.TID_WC, wdtype)
    U = torch.empty((B, gamma, V), dtype=torch.float32, device=dev)
    conf = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    surv = torch.empty_like(conf)
    bd.dspark_lm_head_confidence(to_dev(h, wdtype), to_dev(w, wdtype), U, to_dev(w_c, wdtype), -0.2, conf, surv)
    torch.cuda.synchronize()
    h64 = o.to_f64(h, wdtype)
    u_ref = o.lm_head(h64.reshape(B * gamma, H), o.to_f64(w, wdtype)).reshape(B, gamma, V)
    rel_check(U.cpu().numpy(), u_ref, float(np.sqrt(np.mean(u_ref ** 2))), what="U")
    c_ref, s_ref = o.confidence_survival(h64, o.to_f64(w_c, wdtype), -0.2)
    assert np.abs(conf.cpu().numpy() - c_ref).max() < 1e-5
    assert np.abs(surv.cpu().numpy() - s_ref).max() < 1e-5


# ----------------------------------------------------------------------------- S5
@pytest.mark.parametrize("B,H,r,wdtype,with_wm,gamma", [
    (5, 2560, 256, "bf16", True, 7),
    (1, 256, 32, "f32", False, 7),
    (256, 2560, 256, "bf16", False, 7),
    (3, 100, 48, "f32", True, 7),
    (4, 2560, 256, "bf16", True, 1),     # one position per block
    (9, 2560, 256, "bf16", False, 16),   # the longest block: survival over 16 slots
])
def test_confidence_parity(B, H, r, wdtype, with_wm, gamma):
    dev = require_gpu()
    V = 777
    h = synth.normal((B, gamma, H), 1.0, 2, synth.TID_H, wdtype)
    w_c = synth.normal((H,), 0.02, 2, synth.TID_WC, wdtype)
    w_m = synth.normal((r,), 0.5, 2, synth.TID_WM, wdtype) if with_wm else None
    A = synth.normal((V, r), 0.25, 2, synth.TID_A, wdtype)
    anchor = synth.rng(2, synth.TID_ANCHOR).integers(0, V, size=B).astype(np.int32)
    tokens = synth.rng(3, synth.TID_ANCHOR).integers(0, V, size=(B, gamma)).astype(np.int32)
    conf = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    surv = torch.empty_like(conf)
    bd.dspark_confidence_survival(to_dev(h, wdtype), to_dev(w_c, wdtype), 0.3, conf, surv,
                                  w_m=to_dev(w_m, wdtype) if with_wm else None,
                                  A=to_dev(A, wdtype), anchor=to_dev(anchor), tokens=to_dev(tokens))
    torch.cuda.synchronize()
    c_ref, s_ref = o.confidence_survival(
        o.to_f64(h, wdtype), o.to_f64(w_c, wdtype), 0.3,
        w_m=o.to_f64(w_m, wdtype) if with_wm else None, A=o.to_f64(A, wdtype),
        anchor=anchor, tokens=tokens)
    rel_check(conf.cpu().numpy(), c_ref, 0.0, what="conf")
    rel_check(surv.cpu().numpy(), s_ref, 0.0, what="survival")
    assert np.abs(conf.cpu().numpy() - c_ref).max() < 1e-5
    assert np.abs(surv.cpu().numpy() - s_ref).max() < 1e-5


# ----------------------------------------------------------------------------- S6
def _run_overlap(teacher, *, draft=None, idx=None, prob=None, valid=None):
    dev = require_gpu()
    N, gamma, V = teacher.shape
    alpha = torch.empty((N, gamma), dtype=torch.float32, device=dev)
    tau = torch.empty((N,), dtype=torch.float32, device=dev)
    acc = torch.empty((gamma,), dtype=torch.float64, device=dev)
    mean = torch.empty((1,), dtype=torch.float64, device=dev)
    bd.dspark_overlap_tau(to_dev(teacher), alpha, tau,
                          draft=None if draft is None else to_dev(draft),
                          cand_idx=None if idx is None else to_dev(idx),
                          cand_prob=None if prob is None else to_dev(prob),
                          valid=None if valid is None else to_dev(valid),
                          accept_rate_at=acc, tau_mean=mean)
    torch.cuda.synchronize()
    return alpha.cpu().numpy(), tau.cpu().numpy(), acc.cpu().numpy(), float(mean.cpu()[0])


def _check_tau(got, alpha_raw, valid):
    a_ref, tau_ref, acc_ref, mean_ref = o.tau_metrics(alpha_raw, valid)
    alpha, tau, acc, mean = got
    assert np.abs(alpha - a_ref).max() < ALPHA_ABS
    assert np.abs(alpha - a_ref).max() < 2e-5                    # tighter: fp32 sums
    assert np.abs(tau - tau_ref).max() < ALPHA_ABS
    assert np.abs(acc - acc_ref).max() < ALPHA_ABS
    assert abs(mean - mean_ref) < ALPHA_ABS


@pytest.mark.parametrize("sigma,N,V,resident", [
    (0.5, 9, 5000, True), (1.0, 9, 5000, True), (2.0, 9, 5000, True),
    (1.0, 20, 5000, True),       # split rows, per-row finish kernel
    (1.0, 200, 5000, False),     # one workgroup per row (two passes), several tau blocks
    (1.0, 200, 5000, True),      # many rows read once: 16 chunks per row, 2 float4 per thread
    (2.0, 160, 30004, True),     # ragged last chunk
    (0.5, 150, 100000, True),    # 4 float4 per thread and array
])
def test_overlap_dense_parity(sigma, N, V, resident, monkeypatch):
    monkeypatch.setenv("DSPARK_OVERLAP_RESIDENT", "1" if resident else "0")
    teacher, draft = synth.overlap_inputs(N, V, sigma, seed=1)
    valid = synth.validity(N, seed=1, trunc_frac=0.4, n_dummy=1)
    got = _run_overlap(teacher, draft=draft, valid=valid)
    a_raw, _ = o.overlap_dense(teacher.astype(np.float64), draft.astype(np.float64))
    _check_tau(got, a_raw, valid)
    assert got[1][-1] == 0.0                                   # padding block sentinel


@pytest.mark.parametrize("gamma,N,V,mode", [
    (1, 9, 5000, "dense"),        # one launch
    (16, 3, 5000, "dense"),       # one launch, the longest block
    (3, 40, 3000, "dense"),       # split rows
    (16, 80, 2000, "dense"),      # many rows, each read once (1280 rows)
    (1, 400, 3000, "candidates"),  # one workgroup per row, one position per block
    (16, 30, 3000, "candidates"),  # one workgroup per row from 384 rows (480 rows)
    (3, 10, 3000, "candidates"),  # one launch
])
def test_overlap_other_block_lengths(gamma, N, V, mode):
    # tau, accept_rate@i and tau_mean over blocks of other lengths than 7, on
    # every overlap path, with invalid slots and an all-invalid last block
    teacher, draft = synth.overlap_inputs(N, V, 1.0, gamma=gamma, seed=8)
    g = np.random.default_rng(8)
    valid = (g.random((N, gamma)) > 0.2).astype(np.uint8)
    valid[-1] = 0
    t64 = teacher.astype(np.float64)
    if mode == "dense":
        got = _run_overlap(teacher, draft=draft, valid=valid)
        a_raw, _ = o.overlap_dense(t64, draft.astype(np.float64))
    else:
        k = 16
        teacher = teacher * 3.0
        t64 = teacher.astype(np.float64)
        idx = np.argsort(-t64, axis=-1)[..., :k].astype(np.int32)
        _, prob = synth.candidates(N, V, k, gamma=gamma, seed=8)
        got = _run_overlap(teacher.astype(np.float32), idx=idx, prob=prob, valid=valid)
        a_raw = o.overlap_sparse(t64, idx, prob.astype(np.float64))
    _check_tau(got, a_raw, valid)
    assert got[1][-1] == 0.0                                   # all-invalid block sentinel


def test_overlap_identical_rows_give_tau_eight():
    teacher, _ = synth.overlap_inputs(3, 4096, 1.0, seed=2)
    alpha, tau, acc, mean = _run_overlap(teacher, draft=teacher.copy())
    assert np.allclose(alpha, 1.0, atol=2e-5) and np.allclose(tau, 8.0, atol=2e-4)


def test_overlap_single_launch_leaves_its_workspace_ready():
    # few rows run as one launch that counts arrivals in the workspace; one
    # zero-filled workspace serves dense and candidate calls of several shapes
    # (and a many-row call on the split path) in turn
    dev = require_gpu()
    cases = [("dense", 9, 5000, 4), ("cand", 5, 5000, 5), ("dense", 2, 151936, 6),
             ("dense", 20, 5000, 7), ("dense", 160, 4096, 10), ("cand", 9, 151936, 8),
             ("dense", 150, 4096, 11), ("dense", 9, 5000, 9)]
    size = max(bd.dspark_overlap_tau_workspace(N, 7, V) for _, N, V, _ in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    for mode, N, V, seed in cases:
        teacher, draft = synth.overlap_inputs(N, V, 1.0, seed=seed)
        valid = synth.validity(N, seed=seed, trunc_frac=0.4, n_dummy=1 if N > 2 else 0)
        alpha = torch.empty((N, 7), dtype=torch.float32, device=dev)
        tau = torch.empty((N,), dtype=torch.float32, device=dev)
        acc = torch.empty((7,), dtype=torch.float64, device=dev)
        mean = torch.empty((1,), dtype=torch.float64, device=dev)
        t64 = teacher.astype(np.float64)
        if mode == "dense":
            bd.dspark_overlap_tau(to_dev(teacher), alpha, tau, draft=to_dev(draft), valid=to_dev(valid),
                                  accept_rate_at=acc, tau_mean=mean, ws=ws, status=status)
            a_raw, _ = o.overlap_dense(t64, draft.astype(np.float64))
        else:
            teacher = teacher * 3.0
            t64 = teacher.astype(np.float64)
            idx = np.argsort(-t64, axis=-1)[..., :16].astype(np.int32)
            _, prob = synth.candidates(N, V, 16, seed=seed)
            bd.dspark_overlap_tau(to_dev(teacher.astype(np.float32)), alpha, tau, cand_idx=to_dev(idx),
                                  cand_prob=to_dev(prob), valid=to_dev(valid), accept_rate_at=acc,
                                  tau_mean=mean, ws=ws, status=status)
            a_raw = o.overlap_sparse(t64, idx, prob.astype(np.float64))
        torch.cuda.synchronize()
        bd.check_device_status(status, f"overlap {mode} N={N} V={V}")
        status.fill_(-1)
        got = (alpha.cpu().numpy(), tau.cpu().numpy(), acc.cpu().numpy(), float(mean.cpu()[0]))
        _check_tau(got, a_raw, valid)


def test_overlap_many_rows_time_out_is_reported(monkeypatch):
    """The single-read path for many rows waits for the other chunks of each
    row; a wait bound of 0 (set from the host) makes those waits run out.
    The kernels still finish, and the call reports it: the status word is
    ETIMEOUT and alpha, tau and the aggregates are NaN.  The next call with
    the normal bound is correct again."""
    dev = require_gpu()
    N, V = 160, 4096
    teacher, draft = synth.overlap_inputs(N, V, 1.0, seed=12)
    valid = synth.validity(N, seed=12, trunc_frac=0.2)
    ws = torch.zeros(bd.dspark_overlap_tau_workspace(N, 7, V), dtype=torch.uint8, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    alpha = torch.empty((N, 7), dtype=torch.float32, device=dev)
    tau = torch.empty((N,), dtype=torch.float32, device=dev)
    acc = torch.empty((7,), dtype=torch.float64, device=dev)
    mean = torch.empty((1,), dtype=torch.float64, device=dev)
    t, d, v = to_dev(teacher), to_dev(draft), to_dev(valid)
    monkeypatch.setenv("DSPARK_OVERLAP_RESIDENT", "1")
    monkeypatch.setenv("DSPARK_OVERLAP_WAIT_US", "0")
    bd.dspark_overlap_tau(t, alpha, tau, draft=d, valid=v, accept_rate_at=acc, tau_mean=mean, ws=ws,
                          status=status)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == bd.ETIMEOUT
    assert np.isnan(alpha.cpu().numpy()).all() and np.isnan(tau.cpu().numpy()).all()
    assert np.isnan(float(mean.cpu()[0]))
    with pytest.raises(bd.DsparkError):
        bd.check_device_status(status, "overlap")
    monkeypatch.delenv("DSPARK_OVERLAP_WAIT_US")
    status.fill_(-1)
    bd.dspark_overlap_tau(t, alpha, tau, draft=d, valid=v, accept_rate_at=acc, tau_mean=mean, ws=ws,
                          status=status)
    torch.cuda.synchronize()
    bd.check_device_status(status, "overlap")
    a_raw, _ = o.overlap_dense(teacher.astype(np.float64), draft.astype(np.float64))
    _check_tau((alpha.cpu().numpy(), tau.cpu().numpy(), acc.cpu().numpy(), float(mean.cpu()[0])), a_raw, valid)


@pytest.mark.parametrize("k,N", [
    (16, 5), (64, 5), (16, 20),
    (16, 64),     # 448 rows: one workgroup per row (not the split path)
    (16, 200),    # 1400 rows, one tau block
    (16, 300),    # two tau blocks
])
def test_overlap_candidates_parity(k, N):
    V = 5000
    teacher, _ = synth.overlap_inputs(N, V, 1.0, seed=3)
    teacher = teacher * 3.0                           # peakier teacher: visible overlap
    idx, prob = synth.candidates(N, V, k, seed=3)
    # give the candidates the teacher's largest entries so that alpha is O(0.1)
    t64 = teacher.astype(np.float64)
    order = np.argsort(-t64, axis=-1)[..., :k]
    idx = order.astype(np.int32)
    got = _run_overlap(teacher.astype(np.float32), idx=idx, prob=prob)
    a_raw = o.overlap_sparse(t64, idx, prob.astype(np.float64))
    assert a_raw.max() > 0.05
    _check_tau(got, a_raw, None)


@pytest.mark.parametrize("N", [64, 200])
def test_overlap_candidates_with_invalid_rows(N):
    # one workgroup per row: invalid rows get alpha 0, and tau and the
    # aggregates skip them
    V, k = 5000, 16
    teacher, _ = synth.overlap_inputs(N, V, 1.0, seed=6)
    teacher = teacher * 3.0
    t64 = teacher.astype(np.float64)
    idx = np.argsort(-t64, axis=-1)[..., :k].astype(np.int32)
    _, prob = synth.candidates(N, V, k, seed=6)
    valid = synth.validity(N, seed=6, trunc_frac=0.4, n_dummy=1)
    got = _run_overlap(teacher.astype(np.float32), idx=idx, prob=prob, valid=valid)
    a_raw = o.overlap_sparse(t64, idx, prob.astype(np.float64))
    assert a_raw.max() > 0.05
    _check_tau(got, a_raw, valid)


@pytest.mark.parametrize("N", [5, 300])           # single launch; one workgroup per row
def test_overlap_candidates_skip_ids_outside_the_vocabulary(N):
    # an id outside [0, V) marks no candidate: it adds nothing, as a candidate
    # of probability 0 would, and reads no teacher entry
    V, k = 5000, 16
    teacher, _ = synth.overlap_inputs(N, V, 1.0, seed=4)
    teacher = teacher * 3.0
    t64 = teacher.astype(np.float64)
    idx = np.argsort(-t64, axis=-1)[..., :k].astype(np.int32)
    _, prob = synth.candidates(N, V, k, seed=4)
    bad = np.zeros(idx.shape, dtype=bool)
    bad[..., -3:] = True                              # the last three of every list
    idx_bad = np.where(bad, np.where(np.arange(k) % 2 == 0, -1, V), idx).astype(np.int32)
    got = _run_overlap(teacher.astype(np.float32), idx=idx_bad, prob=prob)
    a_raw = o.overlap_sparse(t64, idx, np.where(bad, 0.0, prob.astype(np.float64)))
    assert a_raw.max() > 0.05
    _check_tau(got, a_raw, None)


# ----------------------------------------------------------------------------- K5
def _schedule(a, sps):
    dev = require_gpu()
    R = a.shape[0]
    lengths = torch.full((R,), -7, dtype=torch.int32, device=dev)
    stats = torch.full((3,), -1.0, dtype=torch.float64, device=dev)
    bd.dspark_prefix_schedule(to_dev(a), to_dev(np.ascontiguousarray(sps, dtype=np.float64)), lengths, stats)
    torch.cuda.synchronize()
    return lengths.cpu().numpy(), stats.cpu().numpy()


def _check_schedule(a, sps):
    lengths, stats = _schedule(a, sps)
    want_l, theta, tau, batch = o.prefix_schedule(a, sps)
    assert np.array_equal(lengths, want_l), (lengths[:16], want_l[:16])
    assert stats[0] == theta and stats[1] == tau and stats[2] == batch, (stats, theta, tau, batch)
    return want_l, batch


@pytest.mark.parametrize("R,gamma,seed", [
    (1, 1, 0),          # one candidate
    (3, 7, 1),
    (146, 7, 2),        # 1022 candidates: one per thread
    (147, 7, 3),        # 1029: two sorted positions per thread, padding
    (256, 7, 4),        # a serving batch of 256 requests
    (100, 16, 5),       # longest block
    (2048, 8, 6),       # 16384 candidates: the largest sort
    (2340, 7, 7),       # 16380: ragged against the padding
])
def test_prefix_schedule_parity(R, gamma, seed):
    a = synth.survival_rows(R, gamma, seed=seed)
    # knee and slope chosen so that the best cut falls inside the candidates
    sps = synth.sps_table(R * (gamma + 1), knee=R + R * gamma // 3, per_token_ms=20.0 / R)
    _check_schedule(a, sps)


@pytest.mark.parametrize("kind", ["flat", "inverse", "step", "capped", "ties", "clamp", "no_room"])
def test_prefix_schedule_edge_cases(kind):
    R, gamma = 40, 7
    a = synth.survival_rows(R, gamma, seed=11)
    n = R * (gamma + 1)
    B = np.arange(1, n + 1, dtype=np.float64)
    if kind == "flat":                       # every positive candidate admitted
        a[5, 3:] = 0.0
        sps = np.full(n, 2.5)
    elif kind == "inverse":                  # SPS = 1/B: no drafts pay off
        a = np.minimum(a, np.float32(0.99))
        sps = 1.0 / B
    elif kind == "step":
        sps = np.where(B <= 90, 2.0, 1.0)
    elif kind == "capped":                   # the table ends before every candidate fits
        sps = np.full(R + 17, 1.0)
    elif kind == "ties":                     # equal values: flat index order
        a = np.full((R, gamma), 0.5, dtype=np.float32)
        a[::3, 4:] = 0.25
        sps = np.full(R + 100, 1.0)
    elif kind == "clamp":
        a[0, 0], a[7, 2], a[9, 6], a[20, 1] = np.nan, -3.0, 4.0, np.inf
        sps = synth.sps_table(n, knee=60, per_token_ms=0.3)
    else:                                    # the table stops at B = R
        sps = np.full(R, 3.0)
    lengths, batch = _check_schedule(a, sps)
    if kind == "no_room":
        assert batch == R and not lengths.any()


def test_prefix_schedule_on_survival_from_the_confidence_kernel():
    # the scheduler consumes what dspark_confidence_survival writes
    dev = require_gpu()
    B, gamma, H = 256, 7, 2560
    h = synth.normal((B, gamma, H), 1.0, 3, synth.TID_H, "bf16")
    w_c = synth.normal((H,), 0.02, 3, synth.TID_WC, "bf16")
    conf = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    surv = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    bd.dspark_confidence_survival(to_dev(h, "bf16"), to_dev(w_c, "bf16"), 0.5, conf, surv)
    sps = synth.sps_table(B * (gamma + 1), knee=B + 300, per_token_ms=0.02)
    lengths = torch.empty((B,), dtype=torch.int32, device=dev)
    stats = torch.empty((3,), dtype=torch.float64, device=dev)
    bd.dspark_prefix_schedule(surv, to_dev(sps), lengths, stats)
    torch.cuda.synchronize()
    a = surv.cpu().numpy()
    want_l, theta, tau, batch = o.prefix_schedule(a, sps)
    assert np.array_equal(lengths.cpu().numpy(), want_l)
    assert tuple(stats.cpu().numpy()) == (theta, tau, float(batch))


# ----------------------------------------------------------------------------- K7
@pytest.mark.parametrize("B,V,r,wdtype", [
    (1, 5000, 256, "bf16"),      # 7 rows: one partly filled wave
    (40, 3000, 256, "bf16"),     # 280 rows, ragged against 8 waves x 16 rows
    (19, 2008, 64, "bf16"),      # ragged last tile
    (5, 1000, 96, "bf16"),       # rank off the MFMA variants: plain kernel
    (2, 1004, 64, "bf16"),       # V % 8 != 0: plain kernel
    (3, 1000, 48, "f32"),        # float32 tables
])
def test_apply_block_logits_parity(B, V, r, wdtype):
    dev = require_gpu()
    gamma = 7
    U, anchor, A, Bm = _markov_case(B, V, r, wdtype, seed=21)
    prev = np.random.default_rng([21, 1]).integers(0, V, (B, gamma)).astype(np.int32)
    out = torch.full((B, gamma, V), float("nan"), dtype=torch.float32, device=dev)
    bd.dspark_apply_block_logits(to_dev(U), to_dev(prev), to_dev(A, wdtype), to_dev(Bm, wdtype), out)
    torch.cuda.synchronize()
    want = o.teacher_forced_logits(U.astype(np.float64), prev, o.to_f64(A, wdtype), o.to_f64(Bm, wdtype))
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    tight_check(got, want, np.abs(want).max(axis=-1, keepdims=True), what="block logits")


def _run_loss(draft, teacher, target, conf, valid, conf_decay=False):
    dev = require_gpu()
    B, gamma, V = draft.shape
    per = torch.full((B, gamma, 4), float("nan"), dtype=torch.float32, device=dev)
    losses = torch.full((4,), float("nan"), dtype=torch.float64, device=dev)
    bd.dspark_compute_loss(to_dev(draft), to_dev(teacher), to_dev(target), losses,
                           conf_logit=None if conf is None else to_dev(conf),
                           valid=None if valid is None else to_dev(valid), per_pos=per, conf_decay=conf_decay)
    torch.cuda.synchronize()
    return per.cpu().numpy(), losses.cpu().numpy()


def _check_loss(per, losses, want_per, want_losses):
    rel_check(per[..., 0], want_per[..., 0], np.abs(want_per[..., 0]), what="CE")
    assert np.abs(per[..., 1] - want_per[..., 1]).max() <= 2 * ALPHA_ABS, "L1"
    assert np.abs(per[..., 2] - want_per[..., 2]).max() <= ALPHA_ABS, "alpha"
    assert np.abs(per[..., 3] - want_per[..., 3]).max() <= ALPHA_ABS, "BCE"
    assert abs(losses[1] - want_losses[1]) <= 2e-2 * abs(want_losses[1]) + 1e-6, ("CE", losses, want_losses)
    assert abs(losses[2] - want_losses[2]) <= 2 * ALPHA_ABS, ("L1", losses, want_losses)
    assert abs(losses[3] - want_losses[3]) <= ALPHA_ABS, ("conf", losses, want_losses)
    # the weights cross the ABI as float32
    lam = [float(np.float32(x)) for x in (0.1, 0.9, 1.0)]
    tot = lam[0] * losses[1] + lam[1] * losses[2] + lam[2] * losses[3]
    assert abs(losses[0] - tot) <= 1e-12 * max(1.0, abs(tot))


@pytest.mark.parametrize("N,sigma,conf_decay", [
    (1, 0.5, False),     # 7 rows: the one-launch overlap path
    (9, 1.0, True),      # 63 rows, decay-weighted confidence term
    (20, 2.0, False),    # 140 rows: chunked rows over several launches
    (200, 1.0, False),   # 1400 rows: many rows, each read once
])
def test_compute_loss_parity(N, sigma, conf_decay):
    V, gamma = 5000, 7
    teacher, draft = synth.overlap_inputs(N, V, sigma, seed=3)
    g = np.random.default_rng([3, 9])
    target = g.integers(0, V, (N, gamma)).astype(np.int32)
    conf = g.standard_normal((N, gamma)).astype(np.float32)
    valid = synth.validity(N, seed=3, trunc_frac=0.4, n_dummy=1 if N > 1 else 0)
    per, losses = _run_loss(draft, teacher, target, conf, valid, conf_decay)
    want_per, want_losses = o.compute_loss(draft.astype(np.float64), teacher.astype(np.float64), target,
                                           conf.astype(np.float64), valid, conf_decay=conf_decay)
    _check_loss(per, losses, want_per, want_losses)


@pytest.mark.parametrize("gamma,N,conf_decay", [
    (1, 9, False),      # 9 rows: the one-launch overlap path
    (16, 5, True),      # 80 rows: chunked rows, decay weights over 16 positions
    (16, 100, False),   # 1600 rows: many rows, each read once
    (3, 30, True),
])
def test_compute_loss_other_block_lengths(gamma, N, conf_decay):
    V = 3000
    teacher, draft = synth.overlap_inputs(N, V, 1.0, gamma=gamma, seed=4)
    g = np.random.default_rng([4, gamma])
    target = g.integers(0, V, (N, gamma)).astype(np.int32)
    conf = g.standard_normal((N, gamma)).astype(np.float32)
    valid = (g.random((N, gamma)) > 0.25).astype(np.uint8)
    valid[-1] = 0
    per, losses = _run_loss(draft, teacher, target, conf, valid, conf_decay)
    want_per, want_losses = o.compute_loss(draft.astype(np.float64), teacher.astype(np.float64), target,
                                           conf.astype(np.float64), valid, conf_decay=conf_decay)
    _check_loss(per, losses, want_per, want_losses)


def test_compute_loss_without_confidence_or_mask():
    V, gamma, N = 4096, 7, 3
    teacher, draft = synth.overlap_inputs(N, V, 1.0, seed=5)
    target = np.random.default_rng([5, 9]).integers(0, V, (N, gamma)).astype(np.int32)
    per, losses = _run_loss(draft, teacher, target, None, None)
    want_per, want_losses = o.compute_loss(draft.astype(np.float64), teacher.astype(np.float64), target)
    _check_loss(per, losses, want_per, want_losses)
    assert losses[3] == 0.0 and not per[..., 3].any()


def test_teacher_forced_block_logits_then_loss():
    # the training forward of [P5] §3.3-3.4: corrected logits from the reference
    # tokens, then the loss against the teacher at those tokens
    dev = require_gpu()
    B, gamma, V, r = 6, 7, 3000, 256
    U, anchor, A, Bm = _markov_case(B, V, r, "bf16", seed=23)
    g = np.random.default_rng([23, 2])
    ref = g.integers(0, V, (B, gamma)).astype(np.int32)               # reference tokens t_1..t_gamma
    prev = np.concatenate([anchor[:, None], ref[:, :-1]], axis=1).astype(np.int32)
    teacher = (U + g.standard_normal(U.shape).astype(np.float32)).astype(np.float32)
    conf = g.standard_normal((B, gamma)).astype(np.float32)
    draft = torch.empty((B, gamma, V), dtype=torch.float32, device=dev)
    bd.dspark_apply_block_logits(to_dev(U), to_dev(prev), to_dev(A, "bf16"), to_dev(Bm, "bf16"), draft)
    per = torch.empty((B, gamma, 4), dtype=torch.float32, device=dev)
    losses = torch.empty((4,), dtype=torch.float64, device=dev)
    bd.dspark_compute_loss(draft, to_dev(teacher), to_dev(ref), losses, conf_logit=to_dev(conf), per_pos=per)
    torch.cuda.synchronize()
    d64 = o.teacher_forced_logits(U.astype(np.float64), prev, o.to_f64(A, "bf16"), o.to_f64(Bm, "bf16"))
    want_per, want_losses = o.compute_loss(d64, teacher.astype(np.float64), ref, conf.astype(np.float64))
    _check_loss(per.cpu().numpy(), losses.cpu().numpy(), want_per, want_losses)


# ----------------------------------------------------------------------------- K6
DECISION_MARGIN = 1e-4      # log-domain margin below which fp32 and fp64 may decide differently


def _verify_case(B, G, V, seed, sigma):
    g = np.random.default_rng([seed, 41])
    draft = g.standard_normal((B, G, V)).astype(np.float32)
    target = np.concatenate([draft, g.standard_normal((B, 1, V)).astype(np.float32)], axis=1)
    target += np.float32(sigma) * g.standard_normal((B, G + 1, V)).astype(np.float32)
    # drafted tokens drawn from the draft distribution (numpy's generator)
    toks = np.empty((B, G), dtype=np.int32)
    for b in range(B):
        for j in range(G):
            p = np.exp(draft[b, j].astype(np.float64) - draft[b, j].max())
            toks[b, j] = g.choice(V, p=p / p.sum())
    return target, draft, toks


def _run_verify(target, draft, toks, lengths, seeds, offset):
    dev = require_gpu()
    B, G, V = draft.shape
    acc = torch.full((B,), -9, dtype=torch.int32, device=dev)
    nxt = torch.full((B,), -9, dtype=torch.int32, device=dev)
    ap = torch.full((B, G), float("nan"), dtype=torch.float32, device=dev)
    bd.dspark_verify(to_dev(target), to_dev(draft), to_dev(toks), to_dev(seeds), acc, nxt,
                     lengths=None if lengths is None else to_dev(lengths), offset=offset, accept_prob=ap)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy(), ap.cpu().numpy()


@pytest.mark.parametrize("B,G,V,sigma,with_len", [
    (1, 7, 5000, 0.3, False),      # one request: rows chunked over many workgroups
    (6, 7, 4096, 1.0, True),       # scheduler-style lengths, including 0 and gamma
    (40, 7, 3000, 0.5, True),
    (300, 4, 2000, 2.0, False),    # many requests: few chunks per row
    (3, 16, 1000, 0.1, True),      # longest block
])
def test_verify_parity(B, G, V, sigma, with_len):
    target, draft, toks = _verify_case(B, G, V, seed=B + G, sigma=sigma)
    g = np.random.default_rng([B, 43])
    lengths = g.integers(0, G + 1, B).astype(np.int32) if with_len else None
    if lengths is not None:
        lengths[0], lengths[-1] = 0, G
    seeds = (np.arange(B, dtype=np.uint64) * np.uint64(2654435761)) + np.uint64(17)
    offset = 5
    acc, nxt, ap = _run_verify(target, draft, toks, lengths, seeds, offset)
    L = lengths if lengths is not None else np.full(B, G)
    want = o.verify_draft(target, draft, toks, L, seeds, offset)
    forced = want["accepted"].copy()
    for b in range(B):
        if acc[b] != want["accepted"][b]:
            # only where the oracle's decision at the first differing position was a near-tie
            k = min(acc[b], want["accepted"][b])
            assert abs(want["margin"][b, k]) < DECISION_MARGIN, (b, acc[b], want["accepted"][b], want["margin"][b])
            forced[b] = acc[b]
    if (forced != want["accepted"]).any():
        want = o.verify_draft(target, draft, toks, L, seeds, offset, forced=forced)
    assert np.array_equal(acc, want["accepted"])
    bad = (nxt != want["next_token"]) & (want["gap"] >= 1e-3)
    assert not bad.any(), (np.nonzero(bad), nxt[bad], want["next_token"][bad], want["gap"][bad])
    ok = want["accept_prob"] > 0
    assert np.abs(ap[ok] - want["accept_prob"][ok]).max(initial=0.0) <= 1e-4
    assert (ap[~ok] == 0).all()


def test_verify_accepts_everything_when_draft_equals_target():
    V, G, B = 2048, 7, 8
    g = np.random.default_rng(47)
    target = g.standard_normal((B, G + 1, V)).astype(np.float32)
    draft = np.ascontiguousarray(target[:, :G])
    toks = g.integers(0, V, (B, G)).astype(np.int32)
    seeds = np.arange(B, dtype=np.uint64)
    acc, nxt, ap = _run_verify(target, draft, toks, None, seeds, 0)
    assert (acc == G).all()
    want = o.verify_draft(target, draft, toks, np.full(B, G), seeds, 0)
    assert np.array_equal(nxt, want["next_token"]) or (want["gap"] < 1e-3).all()


# ----------------------------------------------------------------------------- sequential-head variants
@pytest.mark.parametrize("head,B,V,r,wdtype,T,topk,gamma", [
    ("silu", 1, 4000, 256, "bf16", 0.0, 16, 7),     # narrow step (r split over waves), top-16
    ("silu", 40, 3000, 256, "bf16", 1.0, 0, 7),     # wide step, sampled
    ("gated", 5, 3000, 128, "bf16", 0.0, 8, 7),
    ("gated", 33, 2008, 64, "bf16", 0.7, 16, 7),    # wide step, sampled, top-16, ragged tile
    ("gated", 3, 1000, 48, "f32", 0.0, 5, 7),       # float32 tables
    ("silu", 2, 1000, 32, "f32", 1.0, 0, 7),
    ("gated", 20, 3000, 128, "bf16", 0.0, 16, 1),   # one position per block
    ("silu", 3, 2000, 256, "bf16", 0.8, 8, 16),     # the longest block
])
def test_markov_head_variants_parity(head, B, V, r, wdtype, T, topk, gamma):
    dev = require_gpu()
    H, seed = 96, 29
    U, anchor, A, Bm = _markov_case(B, V, r, wdtype, seed=seed)
    U = synth.base_logits(B, V, gamma=gamma, seed=seed)
    h = synth.normal((B, gamma, H), 1.0, seed, synth.TID_H, wdtype)
    W_g = synth.normal((r, H + r), 0.1, seed, synth.TID_WG, wdtype)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(11) if T > 0 else None
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    tl = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    ls = torch.empty_like(tl)
    ti = torch.empty((B, gamma, topk), dtype=torch.int32, device=dev) if topk else None
    tp = torch.empty((B, gamma, topk), dtype=torch.float32, device=dev) if topk else None
    lo = torch.empty((B, gamma, V), dtype=torch.float32, device=dev)
    code = bd.HEAD_SILU if head == "silu" else bd.HEAD_GATED
    bd.dspark_markov_propose_head(code, to_dev(U), to_dev(anchor), to_dev(A, wdtype), to_dev(Bm, wdtype), tokens,
                                  h=to_dev(h, wdtype) if head == "gated" else None,
                                  W_g=to_dev(W_g, wdtype) if head == "gated" else None, temperature=T,
                                  seeds=None if seeds is None else to_dev(seeds), offset=3, topk=topk,
                                  tok_logit=tl, lse=ls, topk_idx=ti, topk_prob=tp, logits_out=lo)
    torch.cuda.synchronize()
    gpu = dict(tokens=tokens.cpu().numpy(), tok_logit=tl.cpu().numpy(), lse=ls.cpu().numpy(), logits=lo.cpu().numpy())
    if topk:
        gpu["topk_idx"], gpu["topk_prob"] = ti.cpu().numpy(), tp.cpu().numpy()
    kw = dict(head=head, wdtype=wdtype)
    if head == "gated":
        kw.update(h=o.to_f64(h, wdtype), W_g=o.to_f64(W_g, wdtype))
    check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, wdtype), o.to_f64(Bm, wdtype), temperature=T,
                seeds=seeds, offset=3, topk=topk, oracle_kw=kw)


@pytest.mark.gpu
@pytest.mark.parametrize("B,V,r,H,wdtype,T,topk,gamma", [
    (5, 3000, 128, 96, "bf16", 0.0, 8, 7),          # MFMA state and output kernels
    (33, 2008, 64, 96, "bf16", 0.7, 16, 7),         # wide step, sampled, top-16, ragged request block
    (1, 4000, 256, 200, "bf16", 0.0, 16, 7),        # one request, full rank
    (3, 1000, 32, 90, "bf16", 0.0, 0, 7),           # H % 8 != 0: one workgroup per request
    (3, 1000, 48, 96, "f32", 0.0, 5, 7),            # float32 tables
    (4, 3000, 128, 96, "bf16", 0.0, 8, 16),         # the state carried over 16 positions
    (20, 2000, 64, 96, "bf16", 0.0, 16, 1),         # one position: the state starts at zero
])
def test_markov_rnn_head_parity(B, V, r, H, wdtype, T, topk, gamma):
    dev = require_gpu()
    seed = 31
    print(f"rnn head B={B} V={V} r={r} H={H} {wdtype} T={T} topk={topk} gamma={gamma}", flush=True)
    U, anchor, A, Bm = _markov_case(B, V, r, wdtype, seed=seed)
    U = synth.base_logits(B, V, gamma=gamma, seed=seed)
    h = synth.normal((B, gamma, H), 1.0, seed, synth.TID_H, wdtype)
    W = synth.normal((3 * r, 2 * r + H), 0.1, seed, synth.TID_WG, wdtype)
    seeds = np.arange(B, dtype=np.uint64) + np.uint64(5) if T > 0 else None
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    tl = torch.empty((B, gamma), dtype=torch.float32, device=dev)
    ls = torch.empty_like(tl)
    ti = torch.empty((B, gamma, topk), dtype=torch.int32, device=dev) if topk else None
    tp = torch.empty((B, gamma, topk), dtype=torch.float32, device=dev) if topk else None
    lo = torch.empty((B, gamma, V), dtype=torch.float32, device=dev)
    wdt = bd.BF16 if wdtype == "bf16" else bd.F32
    ws = torch.zeros(bd.dspark_markov_propose_head_workspace(bd.HEAD_RNN, B, gamma, V, r, wdt, topk),
                     dtype=torch.uint8, device=dev)
    bd.dspark_markov_propose_head(bd.HEAD_RNN, to_dev(U), to_dev(anchor), to_dev(A, wdtype), to_dev(Bm, wdtype),
                                  tokens, h=to_dev(h, wdtype), W_g=to_dev(W, wdtype), temperature=T,
                                  seeds=None if seeds is None else to_dev(seeds), offset=2, topk=topk,
                                  tok_logit=tl, lse=ls, topk_idx=ti, topk_prob=tp, logits_out=lo, ws=ws)
    torch.cuda.synchronize()
    gpu = dict(tokens=tokens.cpu().numpy(), tok_logit=tl.cpu().numpy(), lse=ls.cpu().numpy(), logits=lo.cpu().numpy())
    if topk:
        gpu["topk_idx"], gpu["topk_prob"] = ti.cpu().numpy(), tp.cpu().numpy()
    kw = dict(head="rnn", wdtype=wdtype, h=o.to_f64(h, wdtype), W_g=o.to_f64(W, wdtype))
    # one step at a time: the workspace holds the m_j table and then the state
    # table ([B, gamma, r] each, tables' dtype); every position must be the
    # oracle's step from the GPU's own previous state and token, to within the
    # rounding of s_j and m_j to the tables' dtype
    es = 2 if wdtype == "bf16" else 4
    off = bd.dspark_markov_propose_workspace(B, gamma, V, topk)
    raw = ws[off:off + 2 * B * gamma * r * es].cpu().numpy()
    if wdtype == "bf16":
        tab = (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        tab = raw.view(np.float32).astype(np.float64)
    M_gpu, S_gpu = tab[:B * gamma * r].reshape(B, gamma, r), tab[B * gamma * r:].reshape(B, gamma, r)
    A64, h64, W64 = o.to_f64(A, wdtype), kw["h"], kw["W_g"]
    step_tol = 2.0 ** -7 if wdtype == "bf16" else 1e-5      # one bf16 ulp of the value, or fp32 accumulation
    for b in range(B):
        for j in range(gamma):
            prev = int(anchor[b]) if j == 0 else int(gpu["tokens"][b, j - 1])
            s_prev = S_gpu[b, j - 1] if j > 0 else np.zeros(r)
            s_ref, m_ref = o.rnn_head_step(s_prev, A64[prev], h64[b, j], W64, wdtype)
            for got, want, what in ((S_gpu[b, j], s_ref, "state"), (M_gpu[b, j], m_ref, "m")):
                lim = step_tol * np.maximum(np.abs(want), np.sqrt((want ** 2).mean())) + 1e-6
                err = np.abs(got - want)
                assert (err <= (2 if what == "m" else 1) * lim).all(), (
                    f"{what} b={b} j={j}: max err {err.max():.3g}")
    # the chain: tokens to the token rule along the oracle's own chain (re-run
    # along the GPU's choice after a near-tie), logits to the 2e-2 bar
    check_chain(gpu, U.astype(np.float64), anchor, o.to_f64(A, wdtype), o.to_f64(Bm, wdtype), temperature=T,
                seeds=seeds, offset=2, topk=0, oracle_kw=kw, tight=REL)
    # Oracle-referenced logits and top-k: the oracle's teacher-forced pass
    # along the GPU's tokens runs the state in float64 from zero.  Its m_j may
    # differ from the GPU's only where float32 accumulation and float64 land
    # on opposite sides of a bf16 rounding boundary; such a flip moves U~_j by
    # at most D_j = max_v sum_k |dm_k| |Bm[k, v]|.  Rows with no flip (D_j = 0)
    # get the tight bar; the others the tight bar plus D_j.  Top-k ids must be
    # the oracle's except where the oracle's k+1 largest values of U~_j are
    # closer than the token gap plus 2 D_j.
    Bm64 = o.to_f64(Bm, wdtype)
    prev = np.concatenate([anchor[:, None].astype(np.int64), gpu["tokens"][:, :-1].astype(np.int64)], axis=1)
    M_ref = np.zeros((B, gamma, r))
    for b in range(B):
        s = np.zeros(r)
        for j in range(gamma):
            s, M_ref[b, j] = o.rnn_head_step(s, A64[prev[b, j]], h64[b, j], W64, wdtype)
    ut_ref = o.teacher_forced_logits(U.astype(np.float64), prev, A64, Bm64, head="rnn", h=h64, W_g=W64,
                                     wdtype=wdtype)
    D = (np.abs(M_gpu - M_ref) @ np.abs(Bm64)).max(axis=-1)            # [B, gamma]
    exact_rows = 0
    for b in range(B):
        for j in range(gamma):
            rms = np.sqrt((ut_ref[b, j] ** 2).mean())
            err = np.abs(gpu["logits"][b, j] - ut_ref[b, j])
            lim = TIGHT * np.maximum(np.abs(ut_ref[b, j]), rms) + D[b, j]
            assert (err <= lim).all(), f"U~ b={b} j={j}: max err {err.max():.3g} (D={D[b, j]:.3g})"
            exact_rows += D[b, j] == 0.0
            if topk:
                ridx = o.topk_indices(ut_ref[b, j], topk)
                e = np.exp(ut_ref[b, j, ridx] - ut_ref[b, j, ridx[0]])
                check_topk(gpu["topk_idx"][b, j], gpu["topk_prob"][b, j], ut_ref[b, j], ridx, e / e.sum(),
                           gap=TOKEN_GAP + 2 * D[b, j])
    print(f"rnn head: {exact_rows} of {B * gamma} rows with m_j identical to the oracle's", flush=True)
