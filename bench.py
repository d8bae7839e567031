"""Benchmark of the DSpark draft-proposal hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic blocks:
LM head -> sequential Markov proposal (7 positions, top-16 candidates) ->
confidence + prefix survival -> overlap / tau_prob against a teacher.

Headline workload (the value of the JSON line): the Qwen3.8-Flash-Next-shaped
high load, B=256 requests x gamma=7 (1,792 LM-head rows), H=2560,
V=151936, r=256, bf16 weights, greedy, top-16 candidates, sparse overlap
against a full-vocabulary teacher.  The same line carries the other
workloads under "configs": one request (B=1, top-16, dense overlap over the
U~ dump), continuous batching (B=64, Philox-Gumbel sampling at T=1, top-16,
sparse overlap) and the offline teacher-forced eval (4,096 blocks = 28,672
rows, sigma=1, 10% truncated blocks).  Each workload reports the mean over
back-to-back steps, the median/p10/p90 of per-step times, and "cold" steps
run right after a 512 MiB write that evicts the 256 MB MALL and the L2s.

Prints ONE JSON line.  Durations come from HIP events recorded on the
stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
METRIC = "draft blocks/sec (γ=7, V=151936) + % HBM/MFMA roofline"
HEADLINE = "c5_flash_next_b256"

WORKLOADS = {
    # name: (requests taken from the 256-request draw, overrides, overlap mode)
    "c5_flash_next_b256": (256, dict(temperature=0.0, topk=16), "topk"),
    "c3_batch64_gumbel": (64, dict(temperature=1.0, topk=16), "topk"),
    "c2_qwen3_4b_b1": (1, dict(temperature=0.0, topk=16), "dense"),
}
C4_NAME = "c4_offline_eval"


def stage_work(B, gamma, H, V, r, topk, overlap, wbytes=2):
    """Algorithmic bytes / flops per launch of each stage (each weight, logit
    and hidden touched once per use the method defines; Bm once per position)."""
    M = B * gamma
    lm_bytes = V * H * wbytes + M * H * wbytes + M * V * 4
    lm_flops = 2.0 * M * H * V
    # per position: Bm once, U_j rows, gathered A rows; plus the U~ dump when dense overlap
    markov_bytes = gamma * (r * V * wbytes + B * V * 4 + B * r * wbytes)
    if overlap == "dense":
        markov_bytes += M * V * 4
    conf_bytes = M * H * wbytes + H * wbytes + 2 * M * 4
    if overlap == "dense":
        ov_bytes = 2 * M * V * 4
    elif overlap == "topk":
        ov_bytes = M * V * 4 + M * topk * 8
    else:
        ov_bytes = 0
    return {
        "lm_head": dict(bytes=lm_bytes, flops=lm_flops),
        "markov": dict(bytes=markov_bytes, flops=2.0 * gamma * B * r * V),
        "confidence": dict(bytes=conf_bytes, flops=2.0 * M * H),
        "overlap": dict(bytes=ov_bytes, flops=0.0),
    }


def lm_head_kernel_name(B, gamma, H):
    M = B * gamma
    return "lm_head_skinny_bf16" if (M <= 16 and M * (H + 8) * 2 <= 64 * 1024) else "lm_head_gemm_bf16"


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "semi_autoregressive_draft_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload, launches_per_step):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_digest") != source_digest(*t.get("sources", [])):
        return None
    return t["hbm_bytes_per_launch"]


def cpu_baseline(inp, overlap, budget_s=10.0, max_reps=100000):
    """The fp64 oracle timed on this host on a bounded sample: repetitions of
    the first block of the workload (the full path for one request: its 7 LM-head
    rows, the chain with top-k, confidence, overlap and tau)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import dspark_oracle as o

    wd = inp.wdtype
    g = inp.gamma
    h = o.to_f64(inp.h[:g], wd)
    W = o.to_f64(inp.w_lm, wd)
    A, Bm = o.to_f64(inp.A, wd), o.to_f64(inp.Bm, wd)
    w_c = o.to_f64(inp.w_c, wd)
    h3 = h.reshape(1, g, inp.H)
    t = inp.teacher[:1].astype(np.float64)
    anchor = inp.anchor[:1]
    seeds = inp.seeds[:1] if inp.temperature > 0 else None

    def one_block():
        U = o.lm_head(h, W).reshape(1, g, inp.V)
        ch = o.markov_chain(U, anchor, A, Bm, temperature=inp.temperature, seeds=seeds,
                            offset=inp.offset, topk=inp.topk, keep_logits=(overlap == "dense"))
        o.confidence_survival(h3, w_c, inp.b_c)
        if overlap == "dense":
            a, _ = o.overlap_dense(t, ch["logits"])
        else:
            a = o.overlap_sparse(t, ch["topk_idx"], ch["topk_prob"])
        o.tau_metrics(a)

    reps, t0 = 0, time.perf_counter()
    while reps < max_reps and (time.perf_counter() - t0) < budget_s:
        one_block()
        reps += 1
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": reps / el, "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} repetitions of one block (1 request x {g} slots) of the workload, "
                      f"full path in float64, {el:.1f} s"}


def bench_prefix_schedule(dev, stream, R=256, gamma=7, calls=200, with_oracle=True):
    """The hardware-aware prefix scheduler at a serving batch of R requests
    (not part of the step): mean time per call over back-to-back launches
    between two events, and the oracle's time for one call beside it."""
    import numpy as np
    import torch
    import synth
    from semi_autoregressive_draft_amd import binding as bd
    a = synth.survival_rows(R, gamma, seed=0)
    sps = synth.sps_table(R * (gamma + 1), knee=R + R * gamma // 3, per_token_ms=20.0 / R)
    d_a = torch.from_numpy(a).to(dev)
    d_sps = torch.from_numpy(sps).to(dev)
    lengths = torch.empty((R,), dtype=torch.int32, device=dev)
    stats = torch.empty((3,), dtype=torch.float64, device=dev)
    for _ in range(5):
        bd.dspark_prefix_schedule(d_a, d_sps, lengths, stats)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        bd.dspark_prefix_schedule(d_a, d_sps, lengths, stats)
    e1.record(stream)
    torch.cuda.synchronize()
    out = {"R": R, "gamma": gamma, "candidates": R * gamma, "us_per_call": round(e0.elapsed_time(e1) * 1e3 / calls, 2),
           "bound": "latency (one workgroup: sort, exact scan, argmax)",
           "batch_chosen": int(stats[2].item()), "calls": calls}
    if with_oracle:
        from oracle import dspark_oracle as o
        t = time.perf_counter()
        o.prefix_schedule(a, sps)
        out["oracle_ms_per_call"] = round((time.perf_counter() - t) * 1e3, 2)
    return out


def bench_teacher_forced_loss(dev, stream, N=512, gamma=7, V=151936, r=256, reps=10):
    """Teacher-forced block logits plus the loss forward at one sequence's
    offline-eval blocks (N anchors, block 7): mean time per call of each entry
    point over back-to-back launches, and the HBM fraction of the pair against
    its algorithmic bytes (U read and U~ written once, Bm and A rows once;
    U~ and the teacher read once by the loss)."""
    import numpy as np
    import torch
    import synth
    from semi_autoregressive_draft_amd import binding as bd
    M = N * gamma
    g = torch.Generator(device=dev)
    g.manual_seed(29)
    U = torch.randn((N, gamma, V), generator=g, device=dev, dtype=torch.float32)
    teacher = torch.randn((N, gamma, V), generator=g, device=dev, dtype=torch.float32).add_(U)
    A = torch.from_numpy(synth.normal((V, r), 0.02, 0, synth.TID_A, "bf16").view("int16")).view(torch.bfloat16).to(dev)
    Bm = torch.from_numpy(synth.normal((r, V), 0.02, 0, synth.TID_BM, "bf16").view("int16")).view(torch.bfloat16).to(dev)
    prev = torch.randint(0, V, (N, gamma), generator=g, device=dev, dtype=torch.int32)
    target = torch.randint(0, V, (N, gamma), generator=g, device=dev, dtype=torch.int32)
    conf = torch.randn((N, gamma), generator=g, device=dev, dtype=torch.float32)
    draft = torch.empty_like(U)
    per = torch.empty((N, gamma, 4), dtype=torch.float32, device=dev)
    losses = torch.empty((4,), dtype=torch.float64, device=dev)
    ws = torch.zeros(bd.dspark_compute_loss_workspace(N, gamma, V), dtype=torch.uint8, device=dev)

    def blk():
        bd.dspark_apply_block_logits(U, prev, A, Bm, draft)

    def loss():
        bd.dspark_compute_loss(draft, teacher, target, losses, conf_logit=conf, per_pos=per, ws=ws)

    out = {"blocks": N, "rows": M, "V": V, "r": r}
    for name, fn in (("apply_block_logits", blk), ("compute_loss", loss)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
    blk_bytes = 8.0 * M * V + 2.0 * r * V + 2.0 * M * r
    loss_bytes = 8.0 * M * V
    out["apply_block_logits_GBps"] = round(blk_bytes / (out["apply_block_logits_ms"] * 1e-3) / 1e9, 1)
    out["compute_loss_GBps"] = round(loss_bytes / (out["compute_loss_ms"] * 1e-3) / 1e9, 1)
    tot_ms = out["apply_block_logits_ms"] + out["compute_loss_ms"]
    out["hbm_frac"] = round((blk_bytes + loss_bytes) / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    out["bound"] = "hbm"
    out["loss_total"] = round(float(losses[0].item()), 6)
    del U, teacher, draft, ws
    torch.cuda.empty_cache()
    return out


def bench_verify(dev, stream, B=256, gamma=7, V=151936, reps=20):
    """Rejection-sampling verification of B drafted blocks (serving shape):
    mean time per call over back-to-back launches and the HBM fraction
    against its algorithmic bytes (every needed target and draft row once)."""
    import numpy as np
    import torch
    from semi_autoregressive_draft_amd import binding as bd
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    draft = torch.randn((B, gamma, V), generator=g, device=dev, dtype=torch.float32)
    target = torch.randn((B, gamma + 1, V), generator=g, device=dev, dtype=torch.float32)
    target[:, :gamma].mul_(0.5).add_(draft)
    toks = torch.randint(0, V, (B, gamma), generator=g, device=dev, dtype=torch.int32)
    seeds = torch.arange(B, dtype=torch.int64, device=dev).to(torch.uint64)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = torch.empty(bd.dspark_verify_workspace(B, gamma, V), dtype=torch.uint8, device=dev)
    for _ in range(3):
        bd.dspark_verify(target, draft, toks, seeds, acc, nxt, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        bd.dspark_verify(target, draft, toks, seeds, acc, nxt, offset=i, ws=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    byt = 4.0 * B * (2 * gamma + 1) * V
    out = {"B": B, "gamma": gamma, "V": V, "ms_per_call": round(ms, 4),
           "GBps": round(byt / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "bound": "hbm", "mean_accepted": round(float(acc.float().mean().item()), 3)}
    del draft, target, ws
    torch.cuda.empty_cache()
    return out


def bench_heads(dev, stream, B=256, gamma=7, V=151936, r=256, H=2560, reps=5):
    """The Markov chain with each sequential head at a serving batch (greedy,
    no top-k): mean time per call over back-to-back calls; the HBM fraction is
    against gamma * (2rV + 4BV) bytes (Bm and U_j once per position)."""
    import numpy as np
    import torch
    import synth
    from semi_autoregressive_draft_amd import binding as bd
    g = torch.Generator(device=dev)
    g.manual_seed(37)
    U = torch.randn((B, gamma, V), generator=g, device=dev, dtype=torch.float32)

    def bf(x):
        return torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)

    A = bf(synth.normal((V, r), 0.02, 0, synth.TID_A, "bf16"))
    Bm = bf(synth.normal((r, V), 0.02, 0, synth.TID_BM, "bf16"))
    h = bf(synth.normal((B, gamma, H), 1.0, 0, synth.TID_H, "bf16"))
    Wg = bf(synth.normal((r, H + r), 0.02, 0, synth.TID_WG, "bf16"))
    Wrnn = bf(synth.normal((3 * r, 2 * r + H), 0.02, 1, synth.TID_WG, "bf16"))
    anchor = torch.randint(0, V, (B,), generator=g, device=dev, dtype=torch.int32)
    tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    out = {"B": B, "gamma": gamma, "V": V, "r": r, "H": H}
    byt = gamma * (2.0 * r * V + 4.0 * B * V)
    weights = {bd.HEAD_GATED: Wg, bd.HEAD_RNN: Wrnn}
    for name, code in (("linear", bd.HEAD_LINEAR), ("silu", bd.HEAD_SILU), ("gated", bd.HEAD_GATED),
                       ("rnn", bd.HEAD_RNN)):
        ws = torch.zeros(bd.dspark_markov_propose_head_workspace(code, B, gamma, V, r), dtype=torch.uint8,
                         device=dev)

        def call():
            bd.dspark_markov_propose_head(code, U, anchor, A, Bm, tokens, h=h if code in weights else None,
                                          W_g=weights.get(code), ws=ws)

        for _ in range(2):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name + "_ms"] = round(ms, 4)
        out[name + "_hbm_frac"] = round(byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        del ws
    del U
    torch.cuda.empty_cache()
    return out


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def time_steps(run, stream, K, flush, cold_reps, lm_events=False):
    """K back-to-back steps with an event at every step start (and, with
    lm_events, one right after the LM-head kernel), then cold_reps steps each
    right after a write of the flush buffer (not timed).  Returns the mean
    step, the per-step distribution, the cold distribution and the mean
    LM-head event window."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev_lm = [torch.cuda.Event(enable_timing=True) for _ in range(K)] if lm_events else None
    t_wall = time.perf_counter()
    for s in range(K):
        ev[s].record(stream)
        if lm_events:
            run(lm_done=ev_lm[s])
        else:
            run()
    ev[K].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(K)]
    out = {"ms_mean": ev[0].elapsed_time(ev[K]) / K, "steps": percentiles(per), "wall_s": wall}
    if lm_events:
        out["lm_ms"] = sum(ev[s].elapsed_time(ev_lm[s]) for s in range(K)) / K
    cold = []
    for i in range(cold_reps):
        flush.fill_(i + 1)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        run()
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    out["cold"] = percentiles(cold) if cold else None
    return out


def roofline_lm(work, lm_ms, kernel, workload):
    """The LM head's roofline: HBM-bound below the ridge (few rows), MFMA-bound above."""
    intensity = work["lm_head"]["flops"] / work["lm_head"]["bytes"]
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        ach = work["lm_head"]["bytes"] / (lm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = work["lm_head"]["flops"] / (lm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = kernel
    roof["traffic"] = traffic_for(kernel, workload, 1)
    roof["algorithmic_bytes_per_launch"] = work["lm_head"]["bytes"]
    roof["algorithmic_flops_per_launch"] = work["lm_head"]["flops"]
    return roof


def bench_propose(name, inp, overlap, weights, dev, stream, K, W, flush, cold_reps):
    """One propose workload through DraftPath: timing, the LM head's roofline
    and a stage breakdown (a separate pass with an event around every stage)."""
    import torch
    from semi_autoregressive_draft_amd.path import DraftPath

    def to_dev(x):
        return torch.from_numpy(x).to(dev)

    def to_bf(x):
        return torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)

    w_lm, A, Bm, w_c = weights
    path = DraftPath(to_bf(inp.h), w_lm, A, Bm, to_dev(inp.anchor), w_c, inp.b_c, gamma=inp.gamma,
                     temperature=inp.temperature,
                     seeds=to_dev(inp.seeds) if inp.temperature > 0 else None, offset=inp.offset,
                     topk=inp.topk, teacher=to_dev(inp.teacher), overlap=overlap)
    for _ in range(W):
        path.run(stream)
    torch.cuda.synchronize()
    path.check()
    t = time_steps(lambda lm_done=None: path.run(stream, lm_done=lm_done), stream, K, flush, cold_reps,
                   lm_events=True)
    path.check()

    stages = [("lm_head", path.lm_head), ("markov", path.propose), ("overlap", path.overlap_tau)]
    D = min(K, 20)
    evd = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(D)]
    for s in range(D):
        evd[s][0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn(stream)
            evd[s][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {n: sum(evd[s][i].elapsed_time(evd[s][i + 1]) for s in range(D)) / D
                for i, (n, _) in enumerate(stages)}
    stage_ms["lm_head"] = t["lm_ms"]
    work = stage_work(inp.B, inp.gamma, inp.H, inp.V, inp.r, inp.topk, overlap)
    M = inp.B * inp.gamma
    kern = lm_head_kernel_name(inp.B, inp.gamma, inp.H)
    info = {}
    for n, ms in stage_ms.items():
        gbs = work[n]["bytes"] / (ms * 1e-3) / 1e9
        info[n] = {"ms": round(ms, 5), "GB/s": round(gbs, 1),
                   "TFLOP/s": round(work[n]["flops"] / (ms * 1e-3) / 1e12, 2),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    info["lm_head"]["note"] = "kernel: " + kern + (" (+ the confidence head in its first workgroup)"
                                                   if kern == "lm_head_skinny_bf16" else "")
    if path.markov_plan > 0:
        # The resident chain keeps Bm on chip across the 7 positions: its time is
        # seven grid-wide exchanges, not a stream of Bm.  The byte count above counts
        # Bm once per position (what a streaming kernel would move); the measured
        # HBM bytes come from the committed rocprofv3 counter summary.
        mk = info["markov"]
        mk["bound"] = "latency (resident chain: Bm held on chip, 7 grid-wide exchanges)"
        mk["effective_GBps_if_streamed"] = mk.pop("GB/s")
        mk.pop("hbm_frac")
        tr = traffic_for("markov_resident", name, 1)
        mk["measured_hbm_bytes"] = tr
        mk["measured_GBps"] = round(tr / (mk["ms"] * 1e-3) / 1e9, 1) if tr else None
    else:
        mk = info["markov"]
        mk["bound"] = "hbm (Bm and U_j streamed once per position)"
        # the per-position wide step's own HBM bytes (rocprofv3 counters), for
        # its share of the stage (the top-k recompute and merges are the rest)
        tr = traffic_for("markov_step_wide", name, 1)
        mk["wide_step_measured_hbm_bytes_per_position"] = tr
    roof = roofline_lm(work, t["lm_ms"], kern, name)
    out = {
        "B": inp.B, "gamma": inp.gamma, "H": inp.H, "V": inp.V, "r": inp.r, "topk": inp.topk,
        "sampling": "gumbel T=%g" % inp.temperature if inp.temperature > 0 else "greedy",
        "overlap": overlap,
        "blocks_per_s": round(inp.B / (t["ms_mean"] * 1e-3), 2),
        "ms_per_step": round(t["ms_mean"], 5),
        "ms_per_step_dist": t["steps"],
        "blocks_per_s_median": round(inp.B / (t["steps"]["median"] * 1e-3), 2),
        "cold_ms_per_step": t["cold"],
        "roofline": roof, "stages": info,
        "stages_note": "lm_head from the timed region (event right after its kernel); the others from a "
                       "separate pass with an event around every stage",
        "wall_s_timed": round(t["wall_s"], 4),
    }
    del path
    return out


def bench_offline_eval(dev, stream, K, flush, cold_reps, sigma=1.0):
    """The offline teacher-forced eval at full size: 4,096 blocks (28,672 rows
    x V) of draft logits and teacher = draft + sigma N(0,1), 10% of the blocks
    truncated, dense overlap and tau in one call."""
    import torch
    import synth
    from semi_autoregressive_draft_amd import binding as bd
    cfg = synth.CONFIGS[C4_NAME]
    N, V, g = cfg["N"], cfg["V"], synth.GAMMA
    teacher, draft = synth.device_overlap_inputs(N, V, sigma, dev, seed=0)
    valid = torch.from_numpy(synth.validity(N, seed=0, trunc_frac=cfg["trunc_frac"])).to(dev)
    alpha = torch.empty((N, g), dtype=torch.float32, device=dev)
    tau = torch.empty((N,), dtype=torch.float32, device=dev)
    acc = torch.empty((g,), dtype=torch.float64, device=dev)
    mean = torch.empty((1,), dtype=torch.float64, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)
    ws = torch.zeros(bd.dspark_overlap_tau_workspace(N, g, V), dtype=torch.uint8, device=dev)

    def run(lm_done=None):
        bd.dspark_overlap_tau(teacher, alpha, tau, draft=draft, valid=valid, accept_rate_at=acc,
                              tau_mean=mean, ws=ws, status=status, stream=stream)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    t = time_steps(run, stream, K, flush, cold_reps)
    bd.check_device_status(status, "overlap")
    # the rows whose logits the call reads (invalid slots read nothing)
    rows_read = int(valid.sum().item())
    byt = 8.0 * rows_read * V
    ach = byt / (t["ms_mean"] * 1e-3) / 1e9
    out = {"N_blocks": N, "rows": N * g, "rows_read": rows_read, "V": V, "sigma": sigma,
           "trunc_frac": cfg["trunc_frac"],
           "blocks_per_s": round(N / (t["ms_mean"] * 1e-3), 2), "ms_per_call": round(t["ms_mean"], 5),
           "ms_per_call_dist": t["steps"], "blocks_per_s_median": round(N / (t["steps"]["median"] * 1e-3), 2),
           "cold_ms_per_call": t["cold"],
           "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4), "kernel": "overlap_rows_resident",
                        "algorithmic_bytes_per_launch": byt,
                        "traffic": traffic_for("overlap_rows_resident", C4_NAME, 1)},
           "tau_mean": round(float(mean.item()), 5)}
    del teacher, draft, ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS) + [C4_NAME],
                    help="the workload of the headline value (default: the 256-request high load)")
    ap.add_argument("--only", action="store_true",
                    help="run the chosen workload alone (no other configs, no next rows): for profiling")
    ap.add_argument("--cold-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy_) 5 times; its "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE per dispatch calibrate the counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; running on several GPUs is not supported "
              "(requests would shard across GPUs with no exchange). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)   # evicts the 256 MB MALL
    results = {}
    big = None
    if args.workload != C4_NAME or not args.only:
        # one draw of the 256-request workload; the smaller workloads are its leading requests
        big = synth.propose_inputs(**synth.CONFIGS[HEADLINE])

        def to_bf(x):
            return torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)

        weights = (to_bf(big.w_lm), to_bf(big.A), to_bf(big.Bm), to_bf(big.w_c))
        names = [args.workload] if args.only else [args.workload] + [n for n in WORKLOADS if n != args.workload]
        for n in names:
            if n not in WORKLOADS:
                continue
            B, over, overlap = WORKLOADS[n]
            inp = synth.leading_requests(big, B, **over)
            print(f"bench: {n}", file=sys.stderr, flush=True)
            results[n] = bench_propose(n, inp, overlap, weights, dev, stream, K, W, flush, args.cold_reps)
        del weights
        torch.cuda.empty_cache()
    if args.workload == C4_NAME or not args.only:
        print(f"bench: {C4_NAME}", file=sys.stderr, flush=True)
        results[C4_NAME] = bench_offline_eval(dev, stream, K, flush, min(args.cold_reps, 3))

    head = results[args.workload]
    cpu = None
    if not args.no_cpu_baseline and args.workload in WORKLOADS:
        B, over, overlap = WORKLOADS[args.workload]
        cpu = cpu_baseline(synth.leading_requests(big, B, **over), overlap, budget_s=15.0)
    next_rows = None
    if not args.only:
        print("bench: next rows", file=sys.stderr, flush=True)
        next_rows = {"prefix_schedule": bench_prefix_schedule(dev, stream, with_oracle=not args.no_cpu_baseline),
                     "teacher_forced_loss": bench_teacher_forced_loss(dev, stream),
                     "verify": bench_verify(dev, stream), "heads": bench_heads(dev, stream)}

    if args.workload == C4_NAME:
        cfg = {"workload": C4_NAME, "N_blocks": head["N_blocks"], "rows": head["rows"], "V": head["V"],
               "sigma": head["sigma"], "parallelism": "single GPU"}
        value, ms = head["blocks_per_s"], head["ms_per_call"]
    else:
        cfg = {"workload": args.workload, **{k: head[k] for k in ("B", "gamma", "H", "V", "r", "topk",
                                                                  "sampling", "overlap")},
               "parallelism": "single GPU"}
        value, ms = head["blocks_per_s"], head["ms_per_step"]
    out = {
        "metric": METRIC, "value": value, "unit": "blocks/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hidden states and teacher logits)",
        "config": cfg,
        "roofline": head["roofline"],
        "ms_per_step_dist": head.get("ms_per_step_dist", head.get("ms_per_call_dist")),
        "cold_ms_per_step": head.get("cold_ms_per_step", head.get("cold_ms_per_call")),
        "stages": head.get("stages"),
        "cpu_baseline": cpu,
        "configs": {n: r for n, r in results.items() if n != args.workload},
        "next_rows": next_rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
