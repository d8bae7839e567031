"""ctypes binding of libdspark.so: the C-ABI entry points under the same names.

Argument marshalling only: tensors become device pointers and sizes, the
stream is torch's current HIP stream, and a non-OK status raises DsparkError.
Every computation runs in the library's HIP kernels; there is no fallback, and
loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# DSPARK_LIB selects another build of the library (the host-sanitized one)
LIB_PATH = os.environ.get("DSPARK_LIB") or os.path.join(PKG, "libdspark.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dspark.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP, ETIMEOUT = range(6)
F32, BF16 = 0, 1

_vp, _i64, _i32, _f32, _u64, _sz = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_uint64, C.c_size_t

_SIGNATURES = {
    "dspark_last_error": (C.c_char_p, []),
    "dspark_version": (C.c_char_p, []),
    "dspark_lm_head": (C.c_int, [_vp, _vp, C.c_int, _i64, _i64, _i64, _vp, _vp]),
    "dspark_lm_head_confidence": (C.c_int, [_vp, _vp, C.c_int, _i64, _i64, _i64, _i64, _vp, _vp, C.c_float,
                                            _vp, _vp, _vp]),
    "dspark_markov_propose_workspace": (C.c_int, [_i64, _i64, _i64, _i32, C.POINTER(_sz)]),
    "dspark_markov_propose_plan": (C.c_int, [_i64, _i64, _i64, C.c_int, C.POINTER(_i32)]),
    "dspark_markov_propose": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, C.c_int, _i64,
                                        _f32, _vp, _u64, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _sz, _vp, _vp]),
    "dspark_markov_propose_noalloc": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, C.c_int, _i64,
                                                _f32, _vp, _u64, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _vp, _vp]),
    "dspark_confidence_survival": (C.c_int, [_vp, C.c_int, _i64, _i64, _i64, _vp, _f32, _vp, _vp,
                                             _i64, _vp, _vp, _vp, _vp, _vp]),
    "dspark_overlap_tau_workspace": (C.c_int, [_i64, _i64, _i64, C.POINTER(_sz)]),
    "dspark_overlap_tau": (C.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _vp, _vp,
                                     _vp, _vp, _vp, _sz, _vp, _vp]),
    "dspark_prefix_schedule": (C.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "dspark_apply_block_logits": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, C.c_int, _i64, _vp, _vp]),
    "dspark_compute_loss_workspace": (C.c_int, [_i64, _i64, _i64, C.POINTER(_sz)]),
    "dspark_compute_loss": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _f32, _f32, _f32,
                                      _i32, _vp, _vp, _vp, _sz, _vp, _vp]),
    "dspark_verify_workspace": (C.c_int, [_i64, _i64, _i64, C.POINTER(_sz)]),
    "dspark_markov_propose_head_workspace": (C.c_int, [_i32, _i64, _i64, _i64, _i64, C.c_int, _i32,
                                                       C.POINTER(_sz)]),
    "dspark_markov_propose_workspace_bmt": (C.c_int, [_i32, _i64, _i64, _i64, _i64, C.c_int, _i32,
                                                      C.POINTER(_sz)]),
    "dspark_markov_propose_head": (C.c_int, [_i32, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                             C.c_int, _i64, _f32, _vp, _u64, _i32, _vp, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _sz, _vp, _vp]),
    "dspark_verify": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _u64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
}


class DsparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_LIB: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """The loaded library (raises if it was never built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m semi_autoregressive_draft_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _LIB = L
    return _LIB


def header_symbols() -> list:
    """Entry points declared in include/dspark.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(dspark_[a-z_0-9]+)\s*\(", text)))


def last_error() -> str:
    return lib().dspark_last_error().decode()


def version() -> str:
    return lib().dspark_version().decode()


def _check(status: int) -> None:
    if status != OK:
        raise DsparkError(status, last_error())


def check_device_status(status, what: str = "dspark") -> None:
    """Raise DsparkError(ETIMEOUT) if a device status word (an int32 tensor
    that a call's ``status`` argument pointed at) reports a bounded wait that
    ran out.  Reading a device tensor synchronises with its stream, so the
    call's kernels have finished when the word is read."""
    vals = status.detach().reshape(-1).cpu().tolist()
    for v in vals:
        if v == ETIMEOUT:
            raise DsparkError(ETIMEOUT, f"{what}: a bounded wait inside the launch ran out (other work kept "
                                        "its workgroups from starting); the outputs are invalid")
        if v != OK:
            raise DsparkError(int(v), f"{what}: unexpected device status {v}")


# ---------------------------------------------------------------------------
# tensor marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("dspark: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"dspark: unsupported dtype {t.dtype}")


def dspark_lm_head(h, w_lm, U, stream=None) -> None:
    """U[M, V] = h[M, H] . w_lm[V, H]^T (float32 out)."""
    M, H = h.shape
    V = w_lm.shape[0]
    _check(lib().dspark_lm_head(_ptr(h), _ptr(w_lm), _dtype(h), M, H, V, _ptr(U), _stream(stream)))


def dspark_lm_head_confidence(h, w_lm, U, w_c, b_c: float, conf, survival, stream=None) -> None:
    """U [B, gamma, V] and the hidden-only confidence conf/survival [B, gamma]
    from h [B, gamma, H] in one call."""
    B, gamma, H = h.shape
    V = w_lm.shape[0]
    _check(lib().dspark_lm_head_confidence(_ptr(h), _ptr(w_lm), _dtype(h), B, gamma, H, V, _ptr(U),
                                           _ptr(w_c), float(b_c), _ptr(conf), _ptr(survival),
                                           _stream(stream)))


def dspark_markov_propose_workspace(B: int, gamma: int, V: int, topk: int = 0) -> int:
    n = _sz(0)
    _check(lib().dspark_markov_propose_workspace(B, gamma, V, topk, C.byref(n)))
    return n.value


def dspark_markov_propose_plan(B: int, V: int, r: int, wdtype: int = BF16) -> int:
    """Workgroups of the resident chain for these sizes (0: one step kernel per position)."""
    n = _i32(0)
    _check(lib().dspark_markov_propose_plan(B, V, r, wdtype, C.byref(n)))
    return n.value


def dspark_markov_propose(U, anchor, A, Bm, tokens, *, temperature: float = 0.0, seeds=None,
                          offset: int = 0, topk: int = 0, tok_logit=None, lse=None, topk_idx=None,
                          topk_prob=None, logits_out=None, ws=None, status=None, stream=None) -> None:
    """Sequential Markov proposal over U [B, gamma, V]; writes tokens [B, gamma]
    (status: optional int32 device word, see check_device_status)."""
    import torch
    B, gamma, V = U.shape
    r = A.shape[1]
    if ws is None:
        ws = torch.zeros(dspark_markov_propose_workspace(B, gamma, V, topk), dtype=torch.uint8,
                         device=U.device)
    _check(lib().dspark_markov_propose(
        _ptr(U), B, gamma, V, _ptr(anchor), _ptr(A), _ptr(Bm), _dtype(A), r, float(temperature),
        _ptr(seeds), int(offset), int(topk), _ptr(tokens), _ptr(tok_logit), _ptr(lse),
        _ptr(topk_idx), _ptr(topk_prob), _ptr(logits_out), _ptr(ws), ws.numel(), _ptr(status),
        _stream(stream)))


def dspark_markov_propose_noalloc(U, anchor, A, Bm, tokens, *, temperature: float = 0.0, seeds=None,
                                  offset: int = 0, topk: int = 0, tok_logit=None, lse=None, topk_idx=None,
                                  topk_prob=None, logits_out=None, status=None, stream=None) -> None:
    """dspark_markov_propose with the library's static scratch as its workspace
    (allocates nothing, here or in the library)."""
    B, gamma, V = U.shape
    r = A.shape[1]
    _check(lib().dspark_markov_propose_noalloc(
        _ptr(U), B, gamma, V, _ptr(anchor), _ptr(A), _ptr(Bm), _dtype(A), r, float(temperature),
        _ptr(seeds), int(offset), int(topk), _ptr(tokens), _ptr(tok_logit), _ptr(lse),
        _ptr(topk_idx), _ptr(topk_prob), _ptr(logits_out), _ptr(status), _stream(stream)))


def dspark_confidence_survival(h, w_c, b_c: float, conf, survival, *, w_m=None, A=None,
                               anchor=None, tokens=None, stream=None) -> None:
    """conf/survival [B, gamma] from h [B, gamma, H]."""
    B, gamma, H = h.shape
    r = A.shape[1] if (w_m is not None and A is not None) else 0
    _check(lib().dspark_confidence_survival(
        _ptr(h), _dtype(h), B, gamma, H, _ptr(w_c), float(b_c), _ptr(w_m), _ptr(A), r,
        _ptr(anchor), _ptr(tokens), _ptr(conf), _ptr(survival), _stream(stream)))


def dspark_overlap_tau_workspace(N: int, gamma: int, V: int) -> int:
    n = _sz(0)
    _check(lib().dspark_overlap_tau_workspace(N, gamma, V, C.byref(n)))
    return n.value


def dspark_overlap_tau(teacher, alpha, tau, *, draft=None, cand_idx=None, cand_prob=None,
                       valid=None, accept_rate_at=None, tau_mean=None, ws=None, status=None,
                       stream=None) -> None:
    """alpha [N, gamma], tau [N] (+ aggregates) from teacher [N, gamma, V]."""
    import torch
    N, gamma, V = teacher.shape
    k = 0 if cand_idx is None else cand_idx.shape[-1]
    if ws is None:
        ws = torch.zeros(dspark_overlap_tau_workspace(N, gamma, V), dtype=torch.uint8,
                         device=teacher.device)
    _check(lib().dspark_overlap_tau(
        _ptr(teacher), _ptr(draft), _ptr(cand_idx), _ptr(cand_prob), k, _ptr(valid), N, gamma, V,
        _ptr(alpha), _ptr(tau), _ptr(accept_rate_at), _ptr(tau_mean), _ptr(ws), ws.numel(),
        _ptr(status), _stream(stream)))


def dspark_prefix_schedule(survival, sps, lengths, stats, stream=None) -> None:
    """lengths [R] int32 and stats [3] float64 {Theta, tau, B} from survival
    [R, gamma] float32 and the SPS table sps [n] float64."""
    R, gamma = survival.shape
    _check(lib().dspark_prefix_schedule(_ptr(survival), R, gamma, _ptr(sps), sps.shape[0],
                                        _ptr(lengths), _ptr(stats), _stream(stream)))


def dspark_apply_block_logits(U, prev_tokens, A, Bm, logits_out, stream=None) -> None:
    """logits_out [B, gamma, V] = U + A[prev_tokens] . Bm (teacher-forced)."""
    B, gamma, V = U.shape
    _check(lib().dspark_apply_block_logits(_ptr(U), B, gamma, V, _ptr(prev_tokens), _ptr(A), _ptr(Bm),
                                           _dtype(A), A.shape[1], _ptr(logits_out), _stream(stream)))


def dspark_compute_loss_workspace(B: int, gamma: int, V: int) -> int:
    n = _sz(0)
    _check(lib().dspark_compute_loss_workspace(B, gamma, V, C.byref(n)))
    return n.value


def dspark_compute_loss(draft, teacher, target, losses, *, conf_logit=None, valid=None, per_pos=None,
                        lambda_ce: float = 0.1, lambda_l1: float = 0.9, lambda_conf: float = 1.0,
                        decay_gamma: float = 4.0, conf_decay: bool = False, ws=None, status=None,
                        stream=None) -> None:
    """losses [4] float64 (total, CE, L1, conf) and optional per_pos [B, gamma, 4]."""
    import torch
    B, gamma, V = draft.shape
    if ws is None:
        ws = torch.zeros(dspark_compute_loss_workspace(B, gamma, V), dtype=torch.uint8, device=draft.device)
    _check(lib().dspark_compute_loss(
        _ptr(draft), _ptr(teacher), _ptr(target), _ptr(conf_logit), _ptr(valid), B, gamma, V,
        float(lambda_ce), float(lambda_l1), float(lambda_conf), float(decay_gamma), int(bool(conf_decay)),
        _ptr(per_pos), _ptr(losses), _ptr(ws), ws.numel(), _ptr(status), _stream(stream)))


def dspark_verify_workspace(B: int, gamma: int, V: int) -> int:
    n = _sz(0)
    _check(lib().dspark_verify_workspace(B, gamma, V, C.byref(n)))
    return n.value


def dspark_verify(target_logits, draft_logits, draft_tokens, seeds, accepted, next_token, *, lengths=None,
                  offset: int = 0, accept_prob=None, ws=None, stream=None) -> None:
    """accepted [B] and next_token [B] from target_logits [B, gamma+1, V],
    draft_logits [B, gamma, V] and draft_tokens [B, gamma]."""
    import torch
    B, gamma, V = draft_logits.shape
    if ws is None:
        ws = torch.empty(dspark_verify_workspace(B, gamma, V), dtype=torch.uint8, device=draft_logits.device)
    _check(lib().dspark_verify(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(lengths), _ptr(seeds), int(offset),
        B, gamma, V, _ptr(accepted), _ptr(next_token), _ptr(accept_prob), _ptr(ws), ws.numel(),
        _stream(stream)))


HEAD_LINEAR, HEAD_SILU, HEAD_GATED, HEAD_RNN = 0, 1, 2, 3


def dspark_markov_propose_head_workspace(head: int, B: int, gamma: int, V: int, r: int, wdtype: int = BF16,
                                         topk: int = 0) -> int:
    n = _sz(0)
    _check(lib().dspark_markov_propose_head_workspace(head, B, gamma, V, r, wdtype, topk, C.byref(n)))
    return n.value


def dspark_markov_propose_workspace_bmt(head: int, B: int, gamma: int, V: int, r: int, wdtype: int = BF16,
                                        topk: int = 0) -> int:
    """Workspace bytes that also hold the transposed Bm of the top-k recompute."""
    n = _sz(0)
    _check(lib().dspark_markov_propose_workspace_bmt(head, B, gamma, V, r, wdtype, topk, C.byref(n)))
    return n.value


def dspark_markov_propose_head(head: int, U, anchor, A, Bm, tokens, *, h=None, W_g=None, temperature: float = 0.0,
                               seeds=None, offset: int = 0, topk: int = 0, tok_logit=None, lse=None,
                               topk_idx=None, topk_prob=None, logits_out=None, ws=None, status=None,
                               stream=None) -> None:
    """dspark_markov_propose with a sequential-head variant (HEAD_SILU, HEAD_GATED, HEAD_RNN;
    W_g is the gated head's [r, H + r] or the RNN head's stacked [3r, 2r + H])."""
    import torch
    B, gamma, V = U.shape
    r = A.shape[1]
    H = h.shape[-1] if h is not None else 0
    if ws is None:
        ws = torch.zeros(dspark_markov_propose_head_workspace(head, B, gamma, V, r, _dtype(A), topk),
                         dtype=torch.uint8, device=U.device)
    _check(lib().dspark_markov_propose_head(
        head, _ptr(h), H, _ptr(W_g), _ptr(U), B, gamma, V, _ptr(anchor), _ptr(A), _ptr(Bm), _dtype(A), r,
        float(temperature), _ptr(seeds), int(offset), int(topk), _ptr(tokens), _ptr(tok_logit), _ptr(lse),
        _ptr(topk_idx), _ptr(topk_prob), _ptr(logits_out), _ptr(ws), ws.numel(), _ptr(status),
        _stream(stream)))
