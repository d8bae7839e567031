"""Seeded synthetic inputs for the DSpark draft-proposal hot path.

This module only draws random numbers and encodes them (fp32 -> bf16 bit
patterns).  It holds none of the method's arithmetic: the oracle and the HIP
path both receive exactly the arrays produced here.

Recipe (one generator per tensor): ``numpy.random.default_rng([seed, tid])``
(PCG64) with the tensor ids below; normals are drawn as float32, scaled, and
rounded to bf16 by round-to-nearest-even where the workload is bf16.  The
shapes follow the pages' draft configurations: block size 7 (anchor slot plus
six MASK slots), hidden 2560, vocabulary 151,936 and Markov rank 256
("Qwen3.8-Flash-Next DSpark 训练实验", 实验设置 table; "DeepSpec 训练全流程详解",
§5.1 model config).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# tensor ids of the per-tensor generators
TID_H, TID_WLM, TID_A, TID_BM, TID_ANCHOR, TID_TEACHER, TID_WC, TID_VALID, \
    TID_DRAFT, TID_U, TID_WM, TID_CAND, TID_SURV, TID_WG = range(14)

GAMMA = 7
QWEN_H = 2560
QWEN_V = 151936
QWEN_R = 256


def rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tid)])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal(shape, std: float, seed: int, tid: int, wdtype: str) -> np.ndarray:
    """N(0, std^2) as float32 ('f32') or as bf16 bit patterns ('bf16')."""
    n = int(np.prod(shape))
    x = rng(seed, tid).standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    x = x.reshape(shape)
    return bf16_bits(x) if wdtype == "bf16" else x


@dataclasses.dataclass
class ProposeInputs:
    """Inputs of one propose call: LM head, Markov chain, confidence, overlap."""
    B: int
    gamma: int
    H: int
    V: int
    r: int
    wdtype: str                  # 'f32' or 'bf16' (h, W_lm, A, Bm, w_c, w_m)
    h: np.ndarray                # [B*gamma, H]
    w_lm: np.ndarray             # [V, H]
    A: np.ndarray                # [V, r]  (Markov down table, W_1)
    Bm: np.ndarray               # [r, V]  (Markov up projection, W_2)
    anchor: np.ndarray           # [B] int32
    w_c: np.ndarray              # [H]
    b_c: float
    w_m: Optional[np.ndarray]    # [r] or None
    teacher: np.ndarray          # [B, gamma, V] float32
    temperature: float
    seeds: np.ndarray            # [B] uint64
    offset: int
    topk: int

    @property
    def M(self) -> int:
        return self.B * self.gamma


def propose_inputs(B: int, H: int, V: int, r: int, wdtype: str, *, gamma: int = GAMMA,
                   seed: int = 0, h_std: float = 1.0, w_std: float = 0.02,
                   markov_std: float = 0.02, temperature: float = 0.0,
                   topk: int = 0, with_wm: bool = False, offset: int = 0,
                   teacher: bool = True) -> ProposeInputs:
    """Draw one propose workload.

    ``markov_std`` sets the scale of both Markov tables; the pages' recipe is
    0.02, and tests raise it so that the transition bias is O(1) and visible.
    """
    M = B * gamma
    h = normal((M, H), h_std, seed, TID_H, wdtype)
    w_lm = normal((V, H), w_std, seed, TID_WLM, wdtype)
    A = normal((V, r), markov_std, seed, TID_A, wdtype)
    Bm = normal((r, V), markov_std, seed, TID_BM, wdtype)
    anchor = rng(seed, TID_ANCHOR).integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    w_c = normal((H,), w_std, seed, TID_WC, wdtype)
    w_m = normal((r,), w_std, seed, TID_WM, wdtype) if with_wm else None
    t = normal((B, gamma, V), 1.0, seed, TID_TEACHER, "f32") if teacher else None
    seeds = np.arange(B, dtype=np.uint64)
    return ProposeInputs(B, gamma, H, V, r, wdtype, h, w_lm, A, Bm, anchor, w_c, 0.0,
                         w_m, t, float(temperature), seeds, int(offset), int(topk))


def leading_requests(inp: ProposeInputs, B: int, **overrides) -> ProposeInputs:
    """The first B requests of a drawn workload.  Every per-request tensor is
    drawn as one sequential stream per tensor, so these are the arrays that
    ``propose_inputs`` draws for B requests with the same seed; the weights
    are shared, not copied.  ``overrides`` replace scalar fields
    (temperature, topk, offset)."""
    g = inp.gamma
    out = dataclasses.replace(inp, B=B, h=inp.h[:B * g], anchor=inp.anchor[:B],
                              teacher=None if inp.teacher is None else inp.teacher[:B],
                              seeds=inp.seeds[:B])
    return dataclasses.replace(out, **overrides)


def base_logits(B: int, V: int, *, gamma: int = GAMMA, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """Synthetic LM-head output U [B, gamma, V] float32, for testing the chain alone."""
    return normal((B, gamma, V), std, seed, TID_U, "f32")


def validity(N: int, gamma: int = GAMMA, *, seed: int = 0, trunc_frac: float = 0.1,
             n_dummy: int = 0) -> np.ndarray:
    """[N, gamma] uint8: ~trunc_frac of the blocks keep only a prefix of length
    L ~ U{1..gamma-1}; the last ``n_dummy`` blocks are all invalid (padding
    blocks)."""
    g = rng(seed, TID_VALID)
    v = np.ones((N, gamma), dtype=np.uint8)
    cut = g.random(N) < trunc_frac
    L = g.integers(1, gamma, size=N)
    pos = np.arange(gamma)[None, :]
    v[cut] = (pos < L[cut, None]).astype(np.uint8)
    if n_dummy:
        v[N - n_dummy:] = 0
    return v


def overlap_inputs(N: int, V: int, sigma: float, *, gamma: int = GAMMA, seed: int = 0):
    """Teacher-forced offline eval rows: draft ~ N(0,1), teacher = draft + sigma*N(0,1).
    Returns (teacher, draft) float32 [N, gamma, V]."""
    draft = normal((N, gamma, V), 1.0, seed, TID_DRAFT, "f32")
    noise = normal((N, gamma, V), 1.0, seed, TID_TEACHER, "f32")
    teacher = draft + np.float32(sigma) * noise
    return teacher, draft


def candidates(N: int, V: int, k: int, *, gamma: int = GAMMA, seed: int = 0):
    """Random sparse draft distributions: k distinct indices per row (ordered
    arbitrarily) with positive probabilities summing to one."""
    g = rng(seed, TID_CAND)
    rows = N * gamma
    idx = np.empty((rows, k), dtype=np.int32)
    for i in range(rows):
        idx[i] = g.choice(V, size=k, replace=False)
    w = g.random((rows, k)) + 0.05
    prob = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx.reshape(N, gamma, k), prob.reshape(N, gamma, k)


def device_overlap_inputs(N: int, V: int, sigma: float, device, *, gamma: int = GAMMA, seed: int = 0):
    """Full-size offline-eval rows drawn on the device with torch's seeded
    generator (host generation of 2 x 17 GB would take minutes).  Returns
    (teacher, draft) float32 device tensors [N, gamma, V]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + 17)
    draft = torch.randn((N, gamma, V), generator=g, device=device, dtype=torch.float32)
    teacher = torch.randn((N, gamma, V), generator=g, device=device, dtype=torch.float32)
    teacher.mul_(float(sigma)).add_(draft)
    return teacher, draft


# The five workloads (B requests x gamma slots; N offline blocks).
CONFIGS = {
    "c1_tiny_fp32": dict(B=1, H=256, V=4096, r=32, wdtype="f32", h_std=0.02,
                         temperature=0.0, topk=0),
    "c2_qwen3_4b_b1": dict(B=1, H=QWEN_H, V=QWEN_V, r=QWEN_R, wdtype="bf16",
                           temperature=0.0, topk=0),
    "c3_batch64_gumbel": dict(B=64, H=QWEN_H, V=QWEN_V, r=QWEN_R, wdtype="bf16",
                              temperature=1.0, topk=0),
    "c4_offline_eval": dict(N=4096, V=QWEN_V, sigmas=(0.5, 1.0, 2.0), trunc_frac=0.1),
    "c5_flash_next_b256": dict(B=256, H=QWEN_H, V=QWEN_V, r=QWEN_R, wdtype="bf16",
                               temperature=0.0, topk=16),
}


def survival_rows(R: int, gamma: int = GAMMA, *, seed: int = 0) -> np.ndarray:
    """[R, gamma] float32 prefix-survival stand-ins: uniform draws in [0, 1)
    sorted in descending order along each row (the scheduler's inputs are
    non-increasing along the block)."""
    u = rng(seed, TID_SURV).random((R, gamma), dtype=np.float32)
    return -np.sort(-u, axis=1)


def sps_table(n: int, *, knee: int = 64, base_ms: float = 10.0, per_token_ms: float = 0.05) -> np.ndarray:
    """Synthetic steps-per-second table [n] float64, entry B - 1 for a
    verification batch of B tokens: flat while the target model's step is
    memory-bound (B <= knee), then falling as the step time grows linearly
    with B.  A roofline-shaped stand-in for a table measured offline on the
    serving GPU ("DSpark 论文精读", §7.2 checklist item 3)."""
    B = np.arange(1, n + 1, dtype=np.float64)
    return 1000.0 / (base_ms + per_token_ms * np.maximum(0.0, B - knee))
