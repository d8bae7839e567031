"""fp64 CPU oracle of the DSpark semi-autoregressive draft-proposal hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It shares no
code with the HIP library; it receives the same input arrays (from ``synth``)
and computes every step from its plain definition, in float64, on the CPU.

Sources (the pages), cited by title and section:
  [P1] "Qwen3.8-Flash-Next DSpark 训练实验" (xpengzhao.github.io dl-note):
       评估口径/离线指标 (overlap a_i, tau_prob, validity rules, top-16 rule),
       Baseline 架构/Markov 顺序修正 (m_i, b_i, l_i, greedy),
       Confidence head 与训练目标 (s_i, sigmoid).
  [P4] "DSpark 论文精读：置信度调度推测解码、半自回归生成与大模型推理加速"
       (zzqdeco.github.io): §2.2 (U = W_lm h, corrected logits U~_j, chain vs
       parallel factorisation), §2.3 (teacher-forced vs sequential Markov),
       §3.1 (alpha identity, prefix survival cumprod and its 0.85^6 example).
  [P5] "DeepSpec 训练全流程详解（以 Qwen3 + DSpark 为例）" (wangjunjian.com):
       §4.3 propose (compute_logits, sample_draft_tokens with the anchor as
       first previous token, predict_confidence_step).
  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
       Easy as 1, 2, 3", SC'11 (the pages name no sampler).
  [P4] §4.1 (training loss: per-position CE and full-vocabulary L1, the
       accept-rate soft label, position weights exp(-j / gamma_decay)).
  [P5] §3.4 (the same loss aggregated over masked positions divided by the
       total weight; prev_token_ids = [anchor, t_1, ...] for the block bias).
  [P5] §4.4 (verify_draft_tokens: accept probability min(1, p/q) at the
       drafted token, the prefix cumprod of accept flags, a residual draw
       from max(p - q, 0) after a rejection, a draw from the last target
       distribution when every token is accepted); [P4] §2.1 (the rejection
       step keeps the output distribution exactly the target's).
  [P4] §3.2 (hardware-aware prefix scheduler: B(l), tau(l), Theta = tau *
       SPS(B), the greedy scan over candidates sorted by survival) and §7.2
       (SPS(B) as an offline-measured monotone lookup table; the sort is
       O(R gamma log(R gamma))).

Readings where the pages are silent or disagree (each is listed in the design
notes as well):
  * the Markov bias is linear, b = Bm^T A[prev] ([P1] Markov 顺序修正); the
    SiLU variant shown in [P4] §2.3 is not used;
  * every slot, including slot 0, is biased; slot 0 uses the anchor as its
    previous token ([P1] m_1 = W_1[D]; [P5] §4.3 first_prev_token_ids=anchor);
  * ties in argmax and top-k go to the lowest vocabulary index;
  * sampling is Gumbel-max with Philox4x32-10 words; see ``gumbel``;
  * the confidence head is w_c.h + b_c, plus w_m.A[prev] when w_m is given
    ([P1] s_i = w_c^T [h_i; m_i] + b_c); no calibration is applied;
  * alpha is clamped to [0, 1] and set to 0 at invalid slots; a block with no
    valid slot reports tau = 0 and is left out of the mean ([P1] 离线指标);
  * the prefix scheduler: see ``prefix_schedule`` for its four readings;
  * the training loss: see ``compute_loss`` for how its terms are aggregated;
  * verification draws its uniforms and Gumbel noise from Philox4x32-10 with
    counters kept apart from the draft sampler's: see ``verify_draft``.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# inputs


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, wdtype: str) -> np.ndarray:
    return widen_bf16(x) if wdtype == "bf16" else np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# S1: LM head.  [P4] §2.2: U_1..U_gamma = W_lm [h_1..h_gamma]; [P1] the frozen
# LM head maps the final hidden states to full-vocabulary logits (no bias).


def lm_head(h: np.ndarray, w_lm: np.ndarray) -> np.ndarray:
    """U[m, v] = sum_k h[m, k] * w_lm[v, k]   (h [M,H], w_lm [V,H], float64)."""
    return np.matmul(h, w_lm.T)


# --------------------------------------------------------------------------
# Philox4x32-10 (SC'11): a 10-round Feistel-like bijection of a 128-bit
# counter under a 64-bit key.  Each round multiplies words 0 and 2 by the
# round constants, and swaps and xors the high halves with the other words
# and the key; the key is bumped by the Weyl constants between rounds.

_MASK32 = np.uint64(0xFFFFFFFF)
_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint64(0x9E3779B9)
_PHILOX_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Arguments are arrays (or scalars) holding
    32-bit values; returns the four 32-bit output words as uint64 arrays."""
    c0, c1, c2, c3, k0, k1 = (np.asarray(x, dtype=np.uint64) & _MASK32
                              for x in (c0, c1, c2, c3, k0, k1))
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _PHILOX_W0) & _MASK32
            k1 = (k1 + _PHILOX_W1) & _MASK32
        p0 = _PHILOX_M0 * c0          # < 2^64: exact in uint64
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox_words(seed: int, offset: int, j: int, V: int) -> np.ndarray:
    """The V random words of one (request, position): word v is output word
    (v mod 4) of Philox4x32-10 with key (lo32(seed), hi32(seed)) and counter
    (v div 4, j, lo32(offset), hi32(offset))."""
    n4 = (V + 3) // 4
    ctr = np.arange(n4, dtype=np.uint64)
    s, o = int(seed), int(offset)
    w = philox4x32_10(ctr, j, o & 0xFFFFFFFF, (o >> 32) & 0xFFFFFFFF,
                      s & 0xFFFFFFFF, (s >> 32) & 0xFFFFFFFF)
    return np.stack(w, axis=1).reshape(-1)[:V]


def gumbel(seed: int, offset: int, j: int, V: int) -> np.ndarray:
    """Standard Gumbel noise G = -log(-log u), u = (floor(w / 2^9) + 1/2) 2^-23.

    u uses the top 23 bits of the word, lies in (0, 1) and is exact in both
    binary32 and binary64, so both sides start from the same u."""
    w = philox_words(seed, offset, j, V)
    u = ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23
    return -np.log(-np.log(u))


# --------------------------------------------------------------------------
# Sequential-head variants.  [P4] §2.3 heads table: VanillaMarkov
# b_j = W_up SiLU(W_down[x_{j-1}]); GatedMarkovHead g_j = sigma(W_g [h_j;
# W_down[x_{j-1}]]), b_j = W_up (g_j * W_down[x_{j-1}]).  With A = W_down and
# Bm = W_up^T, each variant changes only the r-vector m_j that the
# up-projection receives; 'linear' is the reading used by the main chain
# ([P1] b_i = W_2 m_i).  A module computing in the tables' dtype hands the
# up-projection m_j rounded to that dtype, so the variants round it (bf16:
# to nearest, ties to even, through float32).


def round_to_dtype(x: np.ndarray, wdtype: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if wdtype != "bf16":
        return x32.astype(np.float64)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def head_vector(head: str, a_row: np.ndarray, *, h_row: Optional[np.ndarray] = None,
                W_g: Optional[np.ndarray] = None, wdtype: str = "bf16") -> np.ndarray:
    """m_j for A[x_{j-1}] = a_row (and h_j, W_g [r, H + r] for the gated head)."""
    if head == "linear":
        return a_row
    if head == "silu":
        v = a_row / (1.0 + np.exp(-a_row))
    elif head == "gated":
        z = W_g @ np.concatenate([h_row, a_row])
        v = a_row / (1.0 + np.exp(-z))
    else:
        raise ValueError(head)
    return round_to_dtype(v, wdtype)


# RNN head ("DSpark 论文精读", §2.3 heads table row RNNHead, and the RNN head
# passage of "Baseline 架构"): the head keeps a state s_j of rank r, zero
# before the block's first position, and at each position reads the input
# z_j = [s_{j-1}; W_down[x_{j-1}]; h_j] (width 2r + H, in that order).  A
# sigmoid gate g_j = sigma(W_gate z_j) mixes the old state with the tanh
# candidate c_j = tanh(W_cand z_j) (with the convention chosen below, gate 1
# writes the candidate and gate 0 keeps the old state).  The output re-reads the input with the updated state,
# z'_j = [s_j; W_down[x_{j-1}]; h_j], projects it to rank r and applies the
# activation; W_up maps the result to the vocabulary.  Readings where the
# pages' formulas did not survive extraction: the state update is a convex
# mix of the old state and the candidate under the gate, as the passage's two
# limiting cases describe (one gate value keeps the old state, the other
# writes the candidate), but the gate values themselves are missing from the
# extracted text, so which end writes the candidate is a chosen convention,
# not one the page fixes: here s_j = (1 - g) * s_{j-1} + g * c_j (gate 1
# writes).  The opposite convention is the same model with W_gate negated.
# The unnamed output activation is SiLU, the activation of the pages'
# SiLU-Vanilla head; the state, like m_j, is handed on in the tables' dtype.
# W_rnn stacks [W_gate; W_cand; W_out] as [3r, 2r + H].


def rnn_head_step(s_prev: np.ndarray, a_row: np.ndarray, h_row: np.ndarray, W_rnn: np.ndarray,
                  wdtype: str = "bf16"):
    """(s_j, m_j) from s_{j-1}, A[x_{j-1}] = a_row, h_j and W_rnn [3r, 2r + H]."""
    r = a_row.shape[0]
    z = np.concatenate([s_prev, a_row, h_row])
    gate = 1.0 / (1.0 + np.exp(-(W_rnn[:r] @ z)))
    cand = np.tanh(W_rnn[r:2 * r] @ z)
    s_new = round_to_dtype((1.0 - gate) * s_prev + gate * cand, wdtype)
    o = W_rnn[2 * r:] @ np.concatenate([s_new, a_row, h_row])
    return s_new, round_to_dtype(o / (1.0 + np.exp(-o)), wdtype)


# --------------------------------------------------------------------------
# S2-S4: the sequential Vanilla-Markov stage.
# [P1] Markov 顺序修正: m_i = W_1[t_{i-1}] (t_0 = anchor), b_i = W_2 m_i,
# l_i = l_i^0 + b_i, q_i = softmax(l_i); inference selects t_i from l_i and
# feeds it to position i+1.  [P4] §2.2: x_j ~ softmax(U~_j), U~_j = U_j + b.


def markov_chain(U: np.ndarray, anchor: np.ndarray, A: np.ndarray, Bm: np.ndarray, *,
                 temperature: float = 0.0, seeds: Optional[np.ndarray] = None,
                 offset: int = 0, topk: int = 0, forced: Optional[np.ndarray] = None,
                 keep_logits: bool = False, head: str = "linear", h: Optional[np.ndarray] = None,
                 W_g: Optional[np.ndarray] = None, wdtype: str = "bf16") -> dict:
    """Run the chain for every request.

    U [B, gamma, V] base logits; anchor [B]; A [V, r]; Bm [r, V] (all float64).
    temperature 0 selects greedily; otherwise token = argmax(U~/T + G).
    ``forced`` [B, gamma] (int, -1 = free) overrides the selected token at a
    position (used to continue a chain along another valid choice).
    ``head`` selects the sequential head (see ``head_vector`` and
    ``rnn_head_step``; h [B, gamma, H] and W_g for 'gated', or W_g = W_rnn
    [3r, 2r + H] for 'rnn'; wdtype the tables' dtype for the rounding of m_j).

    Returns tokens [B,gamma], tok_logit (U~ at the token), lse (log-sum-exp of
    U~), gap (best minus second-best of the selection score), score_max and
    score_tok (the selection score's maximum and its value at the token),
    argmax (the oracle's own choice), optionally top-k indices/probabilities (softmax of
    U~ over the k largest, ties to the lower index) and U~ itself.
    """
    B, gamma, V = U.shape
    out = {k: np.zeros((B, gamma), dtype=np.float64)
           for k in ("tok_logit", "lse", "gap", "score_max", "score_tok")}
    out["tokens"] = np.zeros((B, gamma), dtype=np.int64)
    out["argmax"] = np.zeros((B, gamma), dtype=np.int64)
    if topk:
        out["topk_idx"] = np.zeros((B, gamma, topk), dtype=np.int64)
        out["topk_prob"] = np.zeros((B, gamma, topk), dtype=np.float64)
    if keep_logits:
        out["logits"] = np.zeros((B, gamma, V), dtype=np.float64)
    for b in range(B):
        prev = int(anchor[b])
        s = np.zeros(A.shape[1])                            # RNN state before the block
        for j in range(gamma):
            if head == "rnn":
                s, m = rnn_head_step(s, A[prev], h[b, j], W_g, wdtype)
            else:
                m = head_vector(head, A[prev], h_row=None if h is None else h[b, j], W_g=W_g, wdtype=wdtype)
            ut = U[b, j] + m @ Bm                           # U~_j = U_j + W_2 m_j
            mx = ut.max()
            out["lse"][b, j] = mx + math.log(np.exp(ut - mx).sum())
            if temperature == 0.0:
                score = ut
            else:
                score = ut / temperature + gumbel(int(seeds[b]), offset, j, V)
            x = int(np.argmax(score))                       # first maximum = lowest index
            rest = np.delete(score, x)
            out["gap"][b, j] = score[x] - rest.max() if rest.size else np.inf
            out["argmax"][b, j] = x
            if forced is not None and forced[b, j] >= 0:
                x = int(forced[b, j])
            out["tokens"][b, j] = x
            out["tok_logit"][b, j] = ut[x]
            out["score_max"][b, j] = score.max()
            out["score_tok"][b, j] = score[x]
            if topk:
                idx = topk_indices(ut, topk)
                out["topk_idx"][b, j] = idx
                e = np.exp(ut[idx] - ut[idx[0]])
                out["topk_prob"][b, j] = e / e.sum()
            if keep_logits:
                out["logits"][b, j] = ut
            prev = x
    return out


def topk_indices(x: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries, by value descending, ties to the
    lower index."""
    thr = np.partition(x, x.size - k)[x.size - k]
    cand = np.nonzero(x >= thr)[0]
    order = np.lexsort((cand, -x[cand]))
    return cand[order[:k]]


def teacher_forced_logits(U: np.ndarray, prev_tokens: np.ndarray, A: np.ndarray,
                          Bm: np.ndarray, head: str = "linear", h: Optional[np.ndarray] = None,
                          W_g: Optional[np.ndarray] = None, wdtype: str = "bf16") -> np.ndarray:
    """All positions at once from known previous tokens ([P4] §2.3: training
    applies the Markov bias to the whole block in one batched step).
    prev_tokens [B, gamma] = [anchor, t_0, ..., t_{gamma-2}]."""
    if head == "linear":
        return U + np.einsum("bjr,rv->bjv", A[prev_tokens], Bm)
    B, gamma = prev_tokens.shape
    if head == "rnn":                                       # the state runs along the known tokens
        M = np.zeros((B, gamma, A.shape[1]))
        for b in range(B):
            s = np.zeros(A.shape[1])
            for j in range(gamma):
                s, M[b, j] = rnn_head_step(s, A[prev_tokens[b, j]], h[b, j], W_g, wdtype)
        return U + np.einsum("bjr,rv->bjv", M, Bm)
    M = np.stack([np.stack([head_vector(head, A[prev_tokens[b, j]], h_row=None if h is None else h[b, j],
                                        W_g=W_g, wdtype=wdtype) for j in range(gamma)]) for b in range(B)])
    return U + np.einsum("bjr,rv->bjv", M, Bm)


# --------------------------------------------------------------------------
# S5: confidence head and prefix survival.
# [P1] s_i = w_c^T [h_i; m_i] + b_c, a^_i = sigma(s_i); [P4] §3.1 prefix
# survival a_{r,j} = prod_{i<=j} c_{r,i}.


def confidence_survival(h: np.ndarray, w_c: np.ndarray, b_c: float, *,
                        w_m: Optional[np.ndarray] = None, A: Optional[np.ndarray] = None,
                        anchor: Optional[np.ndarray] = None,
                        tokens: Optional[np.ndarray] = None):
    """h [B, gamma, H] -> (conf, survival) [B, gamma]."""
    s = h @ w_c + b_c
    if w_m is not None:
        prev = np.concatenate([anchor[:, None], tokens[:, :-1]], axis=1)
        s = s + A[prev] @ w_m
    conf = 1.0 / (1.0 + np.exp(-s))
    surv = np.empty_like(conf)
    run = np.ones(conf.shape[0])
    for j in range(conf.shape[1]):
        run = run * conf[:, j]
        surv[:, j] = run
    return conf, surv


# --------------------------------------------------------------------------
# S6: overlap and probabilistic acceptance length.
# [P1] 离线指标: a_i = sum_v min(p_i(v), q_i(v)) = 1 - ||p_i - q_i||_1 / 2;
# tau_prob = 1 + sum_{i=0}^{6} prod_{j<=i} a_j per valid block; invalid
# slots get a_i = 0; accept_rate@i is aggregated over valid tokens.


def softmax(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def overlap_dense(teacher: np.ndarray, draft: np.ndarray):
    """Row-wise (sum min(p, q), sum |p - q|) for p = softmax(teacher),
    q = softmax(draft)."""
    p, q = softmax(teacher), softmax(draft)
    return np.minimum(p, q).sum(axis=-1), np.abs(p - q).sum(axis=-1)


def overlap_sparse(teacher: np.ndarray, idx: np.ndarray, prob: np.ndarray) -> np.ndarray:
    """sum_v min(p(v), q'(v)) where q' is zero outside the candidate set
    ([P1]: the teacher keeps its full-vocabulary probabilities)."""
    p = softmax(teacher)
    pc = np.take_along_axis(p, idx.astype(np.int64), axis=-1)
    return np.minimum(pc, prob).sum(axis=-1)


def tau_metrics(alpha: np.ndarray, valid: Optional[np.ndarray] = None):
    """alpha [N, gamma] raw overlaps -> (alpha_used, tau [N], accept_rate [gamma],
    tau_mean)."""
    N, gamma = alpha.shape
    v = np.ones((N, gamma), dtype=bool) if valid is None else valid.astype(bool)
    a = np.where(v, np.clip(alpha, 0.0, 1.0), 0.0)
    tau = np.ones(N)
    run = np.ones(N)
    for i in range(gamma):
        run = run * a[:, i]
        tau = tau + run
    has = v.any(axis=1)
    tau = np.where(has, tau, 0.0)
    cnt = v.sum(axis=0)
    acc = np.where(cnt > 0, (a * v).sum(axis=0) / np.maximum(cnt, 1), 0.0)
    tau_mean = float(tau[has].mean()) if has.any() else 0.0
    return a, tau, acc, tau_mean


# --------------------------------------------------------------------------
# K5: hardware-aware prefix scheduler.  [P4] §3.2: a request r that sends its
# first l_r draft tokens to verification costs 1 + l_r batch slots, so the
# verification batch is B(l) = sum_r (1 + l_r); it is expected to emit
# 1 + sum_{j<=l_r} a_{r,j} tokens, so tau(l) = sum_r (1 + sum_{j<=l_r} a_{r,j});
# the objective is Theta(l) = tau(l) * SPS(B(l)).  Every extra candidate adds
# one slot to B whatever it is, so for each B the best choice is the B - R
# largest survival values, and since a_{r,j} falls with j, taking candidates in
# descending order of a keeps every request's choice a prefix.  The algorithm:
# start from l = 0, B = R, tau = R, Theta_max = R * SPS(R); visit all (r, j)
# in descending order of a, each time B += 1, tau += a_{r,j}, Theta = tau *
# SPS(B); return the lengths at the cut where Theta was largest.


def prefix_schedule(survival: np.ndarray, sps: np.ndarray):
    """survival a [R, gamma] (column j holds the pages' position j + 1),
    sps [n] with sps[B - 1] = SPS(B) for B = 1..n (n >= R)
    -> (lengths [R] int64, theta, tau, batch).

    Readings where [P4] §3.2 leaves a step open:
      * a is a probability: values are clamped to [0, 1], NaN read as 0;
      * equal survival values are taken in order of the flat index r*gamma + j
        (within a request the earlier position first, so lengths stay prefixes);
      * tau is the exact sum, rounded once to float64, and Theta one float64
        product tau * SPS(B); the first cut (smallest B) attaining the largest
        Theta is returned;
      * the table ends at the largest batch the engine accepts: cuts with
        B > n are not considered.
    """
    a = np.asarray(survival, dtype=np.float32)
    sps = np.asarray(sps, dtype=np.float64)
    R, gamma = a.shape
    n = sps.shape[0]
    if n < R:
        raise ValueError("the SPS table must cover B = R")
    cands = []
    for r in range(R):
        for j in range(gamma):
            v = float(a[r, j])
            v = min(v, 1.0) if v > 0.0 else 0.0          # NaN > 0 is false
            cands.append((v, r * gamma + j))
    cands.sort(key=lambda c: (-c[0], c[1]))
    B = R
    tau = Fraction(R)
    theta_max, k_best, tau_best = float(R) * float(sps[R - 1]), 0, float(R)
    for k, (v, _) in enumerate(cands, start=1):
        if B + 1 > n:
            break
        B += 1
        tau += Fraction(v)
        t = float(tau)                                   # correctly rounded
        theta = t * float(sps[B - 1])
        if theta > theta_max:
            theta_max, k_best, tau_best = theta, k, t
    lengths = np.zeros(R, dtype=np.int64)
    for _, m in cands[:k_best]:
        lengths[m // gamma] += 1
    return lengths, theta_max, tau_best, R + k_best


# --------------------------------------------------------------------------
# Teacher-forced block logits and the training loss (forward).  [P4] §2.3 and
# [P5] §3.3: with the reference tokens known, every position's bias comes from
# its known previous token in one batched step (``teacher_forced_logits``
# above).  [P4] §4.1: per position j, CE_j = -log q_j(x*_j) and
# L1_j = sum_v |p_j(v) - q_j(v)| with p = softmax(teacher), q = softmax(draft);
# the soft label alpha_j = clamp(1 - L1_j / 2, 0, 1) supervises the confidence
# logit through BCE-with-logits; weights w_j = exp(-j / gamma_decay);
# total = l_ce * CE + l_l1 * L1 + l_conf * conf.  [P1] Baseline loss: the same
# three terms with weights exp(-i/4).


def compute_loss(draft: np.ndarray, teacher: np.ndarray, target: np.ndarray,
                 conf_logit: Optional[np.ndarray] = None, valid: Optional[np.ndarray] = None, *,
                 lambda_ce: float = 0.1, lambda_l1: float = 0.9, lambda_conf: float = 1.0,
                 decay_gamma: float = 4.0, conf_decay: bool = False):
    """draft, teacher [B, gamma, V]; target [B, gamma] int; conf_logit
    [B, gamma] or None (no confidence term); valid [B, gamma] or None (all)
    -> (per_pos [B, gamma, 4] = (CE, L1, alpha, BCE), (total, ce, l1, conf)).

    Aggregation (the pages give it three ways that agree when every position
    is valid: [P4] §4.1 normalises the weights and averages over the batch,
    [P5] §3.4 divides the masked weighted sum by the total weight, [P1] weights
    valid response positions):
      * CE and L1: sum over valid (b, j) of w_j * term / sum of w_j over the
        same positions;
      * conf: the plain mean of BCE over valid positions, as both code excerpts
        ([P4] §4.1, [P5] §3.4) compute it; ``conf_decay`` weights it like CE
        and L1 instead, as [P1]'s prose says all three terms are;
      * invalid positions report zeros and carry no weight; with no valid
        position every aggregate is 0.
    """
    B, gamma, V = draft.shape
    v = np.ones((B, gamma), dtype=bool) if valid is None else valid.astype(bool)
    p = softmax(np.asarray(teacher, dtype=np.float64))
    q = softmax(np.asarray(draft, dtype=np.float64))
    l1 = np.abs(p - q).sum(axis=-1)
    alpha = np.clip(1.0 - 0.5 * l1, 0.0, 1.0)
    d = np.asarray(draft, dtype=np.float64)
    m = d.max(axis=-1)
    lse = m + np.log(np.exp(d - m[..., None]).sum(axis=-1))
    ce = lse - np.take_along_axis(d, np.asarray(target, dtype=np.int64)[..., None], axis=-1)[..., 0]
    if conf_logit is not None:
        s = np.asarray(conf_logit, dtype=np.float64)
        bce = np.maximum(s, 0.0) - s * alpha + np.log1p(np.exp(-np.abs(s)))
    else:
        bce = np.zeros((B, gamma))
    w = np.exp(-np.arange(gamma, dtype=np.float64) / decay_gamma)[None, :] * v
    per_pos = np.stack([ce, l1, alpha, bce], axis=-1) * v[..., None]
    W = w.sum()
    ce_a = float((w * ce).sum() / W) if W > 0 else 0.0
    l1_a = float((w * l1).sum() / W) if W > 0 else 0.0
    if conf_logit is None or not v.any():
        cf_a = 0.0
    elif conf_decay:
        cf_a = float((w * bce).sum() / W)
    else:
        cf_a = float(bce[v].mean())
    total = lambda_ce * ce_a + lambda_l1 * l1_a + lambda_conf * cf_a
    return per_pos, (total, ce_a, l1_a, cf_a)


# --------------------------------------------------------------------------
# Rejection-sampling verification.  [P5] §4.4: for the proposal x_0..x_{L-1}
# with draft distributions q_j and target distributions p_0..p_L (p_j is the
# target's distribution for position j given the prefix up to x_{j-1}), token
# j is accepted when u_j < min(1, p_j(x_j) / q_j(x_j)); only the leading run of
# accepts counts (the cumprod of the accept flags); after a rejection at n the
# next token is drawn from the residual max(p_n - q_n, 0) normalised, and when
# all L are accepted it is drawn from p_L.  [P4] §2.1: this keeps the emitted
# tokens distributed exactly as the target's.

VERIFY_UNIFORM = 0x40000000   # counter word 1 of an acceptance uniform: this | j
VERIFY_GUMBEL = 0x80000000    # counter word 1 of the final draw's noise: this | n


def verify_uniform(seed: int, offset: int, j: int) -> float:
    """u_j = (floor(w / 2^9) + 1/2) 2^-23 with w word 0 of Philox4x32-10 under key
    (lo32 seed, hi32 seed) and counter (0, VERIFY_UNIFORM | j, lo32 offset,
    hi32 offset): the draft sampler's u mapping on its own counter stream."""
    w = philox_words(seed, offset, VERIFY_UNIFORM | j, 1)[0]
    return (float(w >> np.uint64(9)) + 0.5) * 2.0 ** -23


def verify_draft(target_logits: np.ndarray, draft_logits: np.ndarray, draft_tokens: np.ndarray,
                 lengths: np.ndarray, seeds: np.ndarray, offset: int = 0, forced=None):
    """target_logits [B, G+1, V], draft_logits [B, G, V], draft_tokens [B, G],
    lengths [B] in 0..G, seeds [B] -> dict(accepted [B], next_token [B],
    accept_prob [B, G] = min(1, p/q) at the decided positions (0 past them),
    margin [B, G] = log-domain decision margins, gap [B] = top-2 gap of the
    final draw's score, residual_empty [B]).

    Readings: p = softmax(target row), q = softmax(draft row) at temperature 1;
    token j is accepted iff log u_j < min(0, log p_j(x_j) - log q_j(x_j))
    (the same event as u_j < min(1, p/q)); the final draw is Gumbel-max,
    argmax_v log r(v) + G_v with G_v from ``gumbel`` on counter word 1
    VERIFY_GUMBEL | n, over r = max(p_n - q_n, 0) after a rejection at n and
    over r = p_L otherwise; a rejection whose residual has no mass (p_n = q_n
    up to rounding) draws from p_n instead.  ``forced`` [B] (optional)
    overrides the accepted count, to continue along another valid decision."""
    t = np.asarray(target_logits, dtype=np.float64)
    d = np.asarray(draft_logits, dtype=np.float64)
    B, G1, V = t.shape
    G = G1 - 1

    def lse(x):
        m = x.max()
        return m + math.log(np.exp(x - m).sum())

    accepted = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    acc = np.zeros((B, G))
    margin = np.full((B, G), np.inf)
    gap = np.zeros(B)
    empty = np.zeros(B, dtype=bool)
    for b in range(B):
        L = int(lengths[b])
        seed = int(seeds[b])
        n = L
        for j in range(L):
            x = int(draft_tokens[b, j])
            delta = (t[b, j, x] - lse(t[b, j])) - (d[b, j, x] - lse(d[b, j]))
            lu = math.log(verify_uniform(seed, offset, j))
            margin[b, j] = min(0.0, delta) - lu
            acc[b, j] = min(1.0, math.exp(delta))
            if not lu < min(0.0, delta):
                n = j
                break
        if forced is not None:
            n = int(forced[b])
        accepted[b] = n
        g = gumbel(seed, offset, VERIFY_GUMBEL | n, V)
        logp = t[b, n] - lse(t[b, n])
        if n < L:
            r = np.exp(logp) - np.exp(d[b, n] - lse(d[b, n]))
            pos = r > 0.0
            if pos.any():
                score = np.where(pos, np.log(np.where(pos, r, 1.0)) + g, -np.inf)
            else:
                empty[b] = True
                score = logp + g
        else:
            score = logp + g
        k = int(np.argmax(score))                   # first index of the maximum
        nxt[b] = k
        srt = np.sort(score)
        gap[b] = srt[-1] - srt[-2] if V > 1 else np.inf
    return dict(accepted=accepted, next_token=nxt, accept_prob=acc, margin=margin, gap=gap,
                residual_empty=empty)
