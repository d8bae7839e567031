"""Benchmark of the DSpark draft-proposal hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic blocks:
LM head -> sequential Markov proposal (7 positions, top-16 candidates, U~
dump) -> confidence + prefix survival -> overlap / tau_prob against a teacher.
Default workload: one request of the Qwen3-4B-shaped draft head (B=1, gamma=7,
H=2560, V=151936, r=256, bf16 weights, greedy).

Prints ONE JSON line.  Per-stage durations come from HIP events recorded on
the stream the kernels run on, inside the timed region.
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

WORKLOADS = {
    # name: (synth config, overrides, overlap mode)
    "c2_qwen3_4b_b1": ("c2_qwen3_4b_b1", dict(topk=16), "dense"),
    "c3_batch64_gumbel": ("c3_batch64_gumbel", dict(topk=16), "topk"),
    "c5_flash_next_b256": ("c5_flash_next_b256", dict(), "topk"),
}


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
    the first block of the workload (the full path for one request)."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2_qwen3_4b_b1", choices=sorted(WORKLOADS))
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
    from semi_autoregressive_draft_amd.path import DraftPath

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return

    cfg_name, over, overlap = WORKLOADS[args.workload]
    cfg = dict(synth.CONFIGS[cfg_name])
    cfg.update(over)
    inp = synth.propose_inputs(**cfg)
    dev = torch.device("cuda", 0)

    def to_dev(x, wd="f32"):
        if wd == "bf16":
            return torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    wd = inp.wdtype
    path = DraftPath(to_dev(inp.h, wd), to_dev(inp.w_lm, wd), to_dev(inp.A, wd), to_dev(inp.Bm, wd),
                     to_dev(inp.anchor), to_dev(inp.w_c, wd), inp.b_c, gamma=inp.gamma,
                     temperature=inp.temperature,
                     seeds=to_dev(inp.seeds) if inp.temperature > 0 else None, offset=inp.offset,
                     topk=inp.topk, teacher=to_dev(inp.teacher), overlap=overlap)
    stream = torch.cuda.current_stream()
    # the hidden-only confidence head runs inside the LM-head call (path.lm_head)
    stages = [("lm_head", path.lm_head), ("markov", path.propose)]
    if path.w_m is not None:
        stages.append(("confidence", path.confidence))
    stages.append(("overlap", path.overlap_tau))

    for _ in range(args.warmup):
        path.run()
    torch.cuda.synchronize()

    # Timed region: one event at each step start and one after the LM-head
    # launch (its duration gives the roofline figure); every event record
    # costs a few microseconds of GPU time, so the stages are not bracketed here.
    K = args.steps
    ev_step = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    ev_lm = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t_wall = time.perf_counter()
    for s in range(K):
        ev_step[s].record(stream)
        path.run(stream, lm_done=ev_lm[s])
    ev_step[K].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_per_step = ev_step[0].elapsed_time(ev_step[K]) / K
    lm_ms_live = sum(ev_step[s].elapsed_time(ev_lm[s]) for s in range(K)) / K
    blocks_per_s = inp.B / (ms_per_step / 1e3)

    # Stage breakdown (diagnostic, after the timed region): the same steps with
    # an event around every stage.
    D = min(K, 20)
    evd = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(D)]
    for s in range(D):
        evd[s][0].record(stream)
        for i, (_, fn) in enumerate(stages):
            fn()
            evd[s][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {name: sum(evd[s][i].elapsed_time(evd[s][i + 1]) for s in range(D)) / D
                for i, (name, _) in enumerate(stages)}
    stage_ms["lm_head"] = lm_ms_live

    work = stage_work(inp.B, inp.gamma, inp.H, inp.V, inp.r, inp.topk, overlap)
    dom = max(stage_ms, key=stage_ms.get)
    M = inp.B * inp.gamma
    stage_info = {}
    for name, ms in stage_ms.items():
        gbs = work[name]["bytes"] / (ms * 1e-3) / 1e9
        tfl = work[name]["flops"] / (ms * 1e-3) / 1e12
        stage_info[name] = {"ms": round(ms, 5), "GB/s": round(gbs, 1), "TFLOP/s": round(tfl, 2),
                            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    # the LM head runs as one kernel launch; its bound is HBM at small M and MFMA at large M
    lm_ms = stage_ms["lm_head"]
    lm_kernel = lm_head_kernel_name(inp.B, inp.gamma, inp.H)
    lm_intensity = work["lm_head"]["flops"] / work["lm_head"]["bytes"]
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if lm_intensity < ridge:
        ach = work["lm_head"]["bytes"] / (lm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = work["lm_head"]["flops"] / (lm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = lm_kernel
    roof["traffic"] = traffic_for(lm_kernel, args.workload, 1)
    roof["algorithmic_bytes_per_launch"] = work["lm_head"]["bytes"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, overlap)
    sched = bench_prefix_schedule(dev, stream, with_oracle=not args.no_cpu_baseline)
    tfl = bench_teacher_forced_loss(dev, stream)
    ver = bench_verify(dev, stream)
    heads = bench_heads(dev, stream)

    out = {
        "metric": METRIC, "value": round(blocks_per_s, 2), "unit": "blocks/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) hidden states and teacher logits)",
        "config": {"workload": args.workload, "B": inp.B, "gamma": inp.gamma, "H": inp.H,
                   "V": inp.V, "r": inp.r, "topk": inp.topk,
                   "sampling": "gumbel T=%g" % inp.temperature if inp.temperature > 0 else "greedy",
                   "overlap": overlap, "parallelism": "single GPU"},
        "roofline": roof,
        "dominant_stage": dom,
        "stages": stage_info,
        "stages_note": "lm_head from the timed region; the others from a separate pass with an event around every stage",
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": cpu,
        "next_rows": {"prefix_schedule": sched, "teacher_forced_loss": tfl, "verify": ver, "heads": heads},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
