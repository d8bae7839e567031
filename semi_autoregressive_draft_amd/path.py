"""One pass of the draft-proposal hot path over a batch of blocks.

Sequences the C-ABI calls on one stream with every output and workspace
allocated once up front:
  dspark_lm_head -> dspark_markov_propose -> dspark_confidence_survival
  -> dspark_overlap_tau (against a teacher; dense over U~, or over the top-k
  candidate distribution when topk > 0)
With the hidden-only confidence head (no w_m) the first and third are one
call, dspark_lm_head_confidence, which at small batch is one launch.
(Issuing the hidden-only confidence head on a second stream, beside the LM
head, measured slower: the cross-stream events cost more than the kernel.)
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as bd


class DraftPath:
    def __init__(self, h, w_lm, A, Bm, anchor, w_c, b_c: float, *, gamma: int,
                 temperature: float = 0.0, seeds=None, offset: int = 0, topk: int = 0,
                 w_m=None, teacher=None, overlap: Optional[str] = None):
        """h [B*gamma, H]; w_lm [V, H]; A [V, r]; Bm [r, V]; anchor [B] int32;
        w_c [H]; teacher [B, gamma, V] float32 or None.
        overlap: None (no S6), 'dense' (q = softmax U~) or 'topk' (q' on candidates)."""
        dev = h.device
        M, H = h.shape
        V = w_lm.shape[0]
        B = M // gamma
        self.B, self.gamma, self.H, self.V = B, gamma, H, V
        self.h, self.w_lm, self.A, self.Bm = h, w_lm, A, Bm
        self.anchor, self.w_c, self.b_c, self.w_m = anchor, w_c, float(b_c), w_m
        self.temperature, self.seeds, self.offset, self.topk = temperature, seeds, offset, topk
        self.teacher, self.overlap = teacher, overlap
        f32 = dict(dtype=torch.float32, device=dev)
        self.U = torch.empty((B, gamma, V), **f32)
        self.tokens = torch.empty((B, gamma), dtype=torch.int32, device=dev)
        self.tok_logit = torch.empty((B, gamma), **f32)
        self.lse = torch.empty((B, gamma), **f32)
        self.topk_idx = torch.empty((B, gamma, topk), dtype=torch.int32, device=dev) if topk else None
        self.topk_prob = torch.empty((B, gamma, topk), **f32) if topk else None
        self.logits = torch.empty((B, gamma, V), **f32) if overlap == "dense" else None
        # zero-filled once; every propose call leaves it ready for the next.
        # With top-k it also holds the transposed Bm that the recompute uses
        # where that pays off.
        ws = (bd.dspark_markov_propose_workspace_bmt(bd.HEAD_LINEAR, B, gamma, V, A.shape[1], bd._dtype(A), topk)
              if topk else bd.dspark_markov_propose_workspace(B, gamma, V, topk))
        self.ws_markov = torch.zeros(ws, dtype=torch.uint8, device=dev)
        # workgroups of the resident chain for these sizes (0: one step kernel per position)
        self.markov_plan = bd.dspark_markov_propose_plan(B, V, A.shape[1], bd._dtype(A))
        # device status words of the propose and overlap calls (see check())
        self.status = torch.zeros((2,), dtype=torch.int32, device=dev)
        self.conf = torch.empty((B, gamma), **f32)
        self.survival = torch.empty((B, gamma), **f32)
        if overlap:
            if overlap == "topk" and not topk:
                raise ValueError("overlap='topk' needs topk > 0")
            self.alpha = torch.empty((B, gamma), **f32)
            self.tau = torch.empty((B,), **f32)
            self.accept_rate = torch.empty((gamma,), dtype=torch.float64, device=dev)
            self.tau_mean = torch.empty((1,), dtype=torch.float64, device=dev)
            self.ws_overlap = torch.zeros(bd.dspark_overlap_tau_workspace(B, gamma, V),
                                          dtype=torch.uint8, device=dev)

    def lm_head(self, stream=None):
        """S1; with the hidden-only confidence head (no w_m) also S5, in the
        same call."""
        if self.w_m is None:
            bd.dspark_lm_head_confidence(self.h.view(self.B, self.gamma, self.H), self.w_lm, self.U,
                                         self.w_c, self.b_c, self.conf, self.survival, stream=stream)
        else:
            bd.dspark_lm_head(self.h, self.w_lm, self.U.view(-1, self.V), stream=stream)

    def propose(self, stream=None):
        bd.dspark_markov_propose(self.U, self.anchor, self.A, self.Bm, self.tokens,
                                 temperature=self.temperature, seeds=self.seeds, offset=self.offset,
                                 topk=self.topk, tok_logit=self.tok_logit, lse=self.lse,
                                 topk_idx=self.topk_idx, topk_prob=self.topk_prob,
                                 logits_out=self.logits, ws=self.ws_markov, status=self.status[0:1],
                                 stream=stream)

    def confidence(self, stream=None):
        bd.dspark_confidence_survival(self.h.view(self.B, self.gamma, self.H), self.w_c, self.b_c,
                                      self.conf, self.survival, w_m=self.w_m, A=self.A,
                                      anchor=self.anchor, tokens=self.tokens, stream=stream)

    def overlap_tau(self, stream=None):
        if self.overlap == "dense":
            bd.dspark_overlap_tau(self.teacher, self.alpha, self.tau, draft=self.logits,
                                  accept_rate_at=self.accept_rate, tau_mean=self.tau_mean,
                                  ws=self.ws_overlap, status=self.status[1:2], stream=stream)
        elif self.overlap == "topk":
            bd.dspark_overlap_tau(self.teacher, self.alpha, self.tau, cand_idx=self.topk_idx,
                                  cand_prob=self.topk_prob, accept_rate_at=self.accept_rate,
                                  tau_mean=self.tau_mean, ws=self.ws_overlap, status=self.status[1:2],
                                  stream=stream)

    def run(self, stream=None, lm_done=None):
        """One pass; lm_done (optional event) is recorded right after the
        LM-head kernel (after the fused LM-head + confidence launch at small
        batch)."""
        main = stream if stream is not None else torch.cuda.current_stream()
        M = self.B * self.gamma
        if self.w_m is None and M <= 16 and self.h.dtype == torch.bfloat16:
            self.lm_head(main)               # one launch: S1 and the hidden-only S5
            if lm_done is not None:
                lm_done.record(main)
        else:                                # the same two launches dspark_lm_head_confidence makes
            bd.dspark_lm_head(self.h, self.w_lm, self.U.view(-1, self.V), stream=main)
            if lm_done is not None:
                lm_done.record(main)
            if self.w_m is None:
                self.confidence(main)
        self.propose(main)
        if self.w_m is not None:             # the Markov term needs the drafted tokens
            self.confidence(main)
        if self.overlap:
            self.overlap_tau(main)

    def check(self):
        """Wait for the last pass and raise DsparkError(ETIMEOUT) if one of its
        bounded waits ran out (its outputs are then invalid)."""
        bd.check_device_status(self.status, "DraftPath")
