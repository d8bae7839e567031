"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, answers the workspace queries, and rejects invalid
arguments with the documented status before any device work is enqueued.

Every call below fails validation on the host (a required pointer is NULL, a
size is invalid, or the workspace is too small), so no kernel is launched; the
fake non-NULL pointers are never dereferenced."""
import ctypes as C
import os

import pytest

from semi_autoregressive_draft_amd import binding as bd

FAKE = 0x1000        # 16-byte aligned, never dereferenced
MISALIGNED = 0x1004


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bd.LIB_PATH):
        from semi_autoregressive_draft_amd import build
        build.build()
    return bd.lib()


def test_exports_every_declared_symbol(L):
    names = bd.header_symbols()
    assert set(names) >= {"dspark_lm_head", "dspark_markov_propose", "dspark_confidence_survival",
                          "dspark_overlap_tau", "dspark_last_error", "dspark_version",
                          "dspark_markov_propose_workspace", "dspark_overlap_tau_workspace"}
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(bd._SIGNATURES)


def test_version(L):
    assert bd.version().startswith("dspark-mi355x") and "gfx950" in bd.version()


def _ws(fn, *args):
    n = C.c_size_t(0)
    st = fn(*args, C.byref(n))
    return st, n.value


def test_workspace_queries(L):
    st, n = _ws(L.dspark_markov_propose_workspace, 1, 7, 151936, 0)
    assert st == bd.OK and n >= 5 * 1187 * 4
    st, n16 = _ws(L.dspark_markov_propose_workspace, 1, 7, 151936, 16)
    assert st == bd.OK and n16 >= n + 4748 * 4
    st, n256 = _ws(L.dspark_markov_propose_workspace, 256, 7, 151936, 16)
    # five per-tile partial arrays (64-column tiles) for every (request, position)
    assert st == bd.OK and n256 >= 5 * 256 * 7 * 2374 * 4
    assert _ws(L.dspark_markov_propose_workspace, 0, 7, 100, 0)[0] == bd.EINVAL
    assert _ws(L.dspark_markov_propose_workspace, 1, 7, 100, -1)[0] == bd.EINVAL
    st, n = _ws(L.dspark_overlap_tau_workspace, 4096, 7, 151936)
    assert st == bd.OK and n >= 16 * 16 * 8
    assert _ws(L.dspark_overlap_tau_workspace, 10, 17, 100)[0] == bd.EUNSUPPORTED
    assert L.dspark_markov_propose_workspace(1, 7, 100, 0, None) == bd.EINVAL
    # the larger workspace adds the transposed Bm (bf16 with top-k only)
    f = L.dspark_markov_propose_workspace_bmt
    st, base = _ws(L.dspark_markov_propose_head_workspace, bd.HEAD_LINEAR, 256, 7, 151936, 256, bd.BF16, 16)
    st2, n = _ws(f, bd.HEAD_LINEAR, 256, 7, 151936, 256, bd.BF16, 16)
    assert st == st2 == bd.OK and n == base + 256 * 151936 * 2
    st, base = _ws(L.dspark_markov_propose_head_workspace, bd.HEAD_LINEAR, 64, 7, 4096, 32, bd.F32, 16)
    assert _ws(f, bd.HEAD_LINEAR, 64, 7, 4096, 32, bd.F32, 16) == (bd.OK, base)
    st, base = _ws(L.dspark_markov_propose_head_workspace, bd.HEAD_LINEAR, 64, 7, 4096, 32, bd.BF16, 0)
    assert _ws(f, bd.HEAD_LINEAR, 64, 7, 4096, 32, bd.BF16, 0) == (bd.OK, base)
    assert _ws(f, bd.HEAD_LINEAR, 0, 7, 4096, 32, bd.BF16, 16)[0] == bd.EINVAL
    assert _ws(f, 9, 4, 7, 4096, 32, bd.BF16, 16)[0] == bd.EINVAL
    assert _ws(f, bd.HEAD_LINEAR, 4, 7, 4096, 32, 5, 16)[0] == bd.EUNSUPPORTED
    assert f(bd.HEAD_LINEAR, 4, 7, 4096, 32, bd.BF16, 16, None) == bd.EINVAL


def test_lm_head_validation(L):
    f = L.dspark_lm_head
    assert f(None, FAKE, bd.BF16, 7, 2560, 151936, FAKE, None) == bd.EINVAL
    assert "non-NULL" in bd.last_error()
    assert f(FAKE, FAKE, bd.BF16, 0, 2560, 151936, FAKE, None) == bd.EINVAL
    assert f(FAKE, FAKE, bd.BF16, 7, 2560, 2 ** 31, FAKE, None) == bd.EINVAL
    assert f(FAKE, FAKE, bd.BF16, 7, 2564, 151936, FAKE, None) == bd.EUNSUPPORTED
    assert f(FAKE, FAKE, bd.BF16, 7, 2560, 151932, FAKE, None) == bd.EUNSUPPORTED
    assert f(MISALIGNED, FAKE, bd.BF16, 7, 2560, 151936, FAKE, None) == bd.EUNSUPPORTED
    assert f(FAKE, FAKE, 7, 7, 2560, 151936, FAKE, None) == bd.EUNSUPPORTED


def test_lm_head_confidence_validation(L):
    f = L.dspark_lm_head_confidence
    ok = (FAKE, FAKE, bd.BF16, 1, 7, 2560, 151936, FAKE, FAKE, 0.5, FAKE, FAKE, None)
    def call(**kw):
        names = ["h", "w", "dt", "B", "gamma", "H", "V", "U", "w_c", "b_c", "conf", "surv", "s"]
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])
    assert call(w_c=None) == bd.EINVAL and "non-NULL" in bd.last_error()
    assert call(conf=None) == bd.EINVAL
    assert call(B=0) == bd.EINVAL
    assert call(gamma=17) == bd.EUNSUPPORTED
    assert call(h=None) == bd.EINVAL                  # the LM head's own checks
    assert call(H=2564) == bd.EUNSUPPORTED
    assert call(dt=7) == bd.EUNSUPPORTED


def _propose(L, **kw):
    a = dict(U=FAKE, B=1, gamma=7, V=151936, anchor=FAKE, A=FAKE, Bm=FAKE, wdt=bd.BF16, r=256,
             T=0.0, seeds=None, offset=0, topk=0, tokens=FAKE, tok_logit=None, lse=None,
             topk_idx=None, topk_prob=None, logits_out=None, ws=None, ws_bytes=0, status=None,
             stream=None)
    a.update(kw)
    return L.dspark_markov_propose(a["U"], a["B"], a["gamma"], a["V"], a["anchor"], a["A"], a["Bm"],
                                   a["wdt"], a["r"], a["T"], a["seeds"], a["offset"], a["topk"],
                                   a["tokens"], a["tok_logit"], a["lse"], a["topk_idx"],
                                   a["topk_prob"], a["logits_out"], a["ws"], a["ws_bytes"],
                                   a["status"], a["stream"])


def test_markov_validation(L):
    assert _propose(L, U=None) == bd.EINVAL
    assert _propose(L, tokens=None) == bd.EINVAL
    assert _propose(L, B=0) == bd.EINVAL
    assert _propose(L, r=0) == bd.EINVAL
    assert _propose(L, T=-1.0) == bd.EINVAL
    assert _propose(L, T=float("nan")) == bd.EINVAL
    assert _propose(L, T=1.0) == bd.EINVAL                       # sampling without seeds
    assert _propose(L, topk=16) == bd.EINVAL                     # no topk outputs
    assert _propose(L, topk_idx=FAKE, topk_prob=FAKE) == bd.EINVAL   # outputs with topk == 0
    assert _propose(L, topk=200000, topk_idx=FAKE, topk_prob=FAKE) == bd.EINVAL  # topk > V
    assert _propose(L, gamma=17) == bd.EUNSUPPORTED
    assert _propose(L, topk=33, topk_idx=FAKE, topk_prob=FAKE) == bd.EUNSUPPORTED
    assert _propose(L, r=48) == bd.EUNSUPPORTED                  # bf16 rank not a multiple of 32
    assert _propose(L, r=2048) == bd.EUNSUPPORTED
    assert _propose(L, V=151932) == bd.EUNSUPPORTED              # bf16 rows not 16-byte multiples
    assert _propose(L, A=MISALIGNED) == bd.EUNSUPPORTED
    assert _propose(L, wdt=5) == bd.EUNSUPPORTED
    assert _propose(L) == bd.EWORKSPACE                          # no workspace
    st, need = _ws(L.dspark_markov_propose_workspace, 1, 7, 151936, 0)
    assert _propose(L, ws=FAKE, ws_bytes=need - 1) == bd.EWORKSPACE
    assert "workspace" in bd.last_error()
    # float32 tables accept any rank and V
    assert _propose(L, wdt=bd.F32, r=48, V=151932) == bd.EWORKSPACE
    # the optional device status word: NULL or a 4-byte aligned int32
    assert _propose(L, status=FAKE) == bd.EWORKSPACE
    assert _propose(L, status=FAKE + 2) == bd.EINVAL
    assert "status" in bd.last_error()


def test_confidence_validation(L):
    f = L.dspark_confidence_survival
    assert f(None, bd.BF16, 1, 7, 2560, FAKE, 0.0, None, None, 0, None, None, FAKE, FAKE, None) == bd.EINVAL
    assert f(FAKE, bd.BF16, 1, 7, 2560, FAKE, 0.0, FAKE, None, 256, FAKE, FAKE, FAKE, FAKE, None) == bd.EINVAL
    assert f(FAKE, bd.BF16, 1, 7, 2560, FAKE, 0.0, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == bd.EINVAL
    assert f(FAKE, bd.BF16, 1, 17, 2560, FAKE, 0.0, None, None, 0, None, None, FAKE, FAKE, None) == bd.EUNSUPPORTED
    assert f(FAKE, 3, 1, 7, 2560, FAKE, 0.0, None, None, 0, None, None, FAKE, FAKE, None) == bd.EUNSUPPORTED


def test_overlap_validation(L):
    f = L.dspark_overlap_tau
    args = lambda **k: [k.get(n, d) for n, d in (
        ("teacher", FAKE), ("draft", FAKE), ("idx", None), ("prob", None), ("k", 0), ("valid", None),
        ("N", 4), ("gamma", 7), ("V", 151936), ("alpha", FAKE), ("tau", FAKE), ("acc", None),
        ("mean", None), ("ws", None), ("wsb", 0), ("status", None), ("s", None))]
    assert f(*args(teacher=None)) == bd.EINVAL
    assert f(*args(k=16)) == bd.EINVAL                       # dense with k
    assert f(*args(draft=None)) == bd.EINVAL                 # sparse without candidates
    assert f(*args(draft=None, idx=FAKE, prob=FAKE, k=0)) == bd.EINVAL
    assert f(*args(draft=None, idx=FAKE, prob=FAKE, k=65)) == bd.EUNSUPPORTED
    assert f(*args(gamma=17)) == bd.EUNSUPPORTED
    assert f(*args(V=151934)) == bd.EUNSUPPORTED
    assert f(*args(draft=MISALIGNED)) == bd.EUNSUPPORTED
    assert f(*args()) == bd.EWORKSPACE
    assert f(*args(draft=None, idx=FAKE, prob=FAKE, k=16)) == bd.EWORKSPACE
    assert f(*args(status=FAKE)) == bd.EWORKSPACE
    assert f(*args(status=FAKE + 1)) == bd.EINVAL


def test_prefix_schedule_validation(L):
    f = L.dspark_prefix_schedule
    args = lambda **k: [k.get(n, d) for n, d in (
        ("surv", FAKE), ("R", 256), ("gamma", 7), ("sps", FAKE), ("n", 2048), ("len", FAKE),
        ("stats", FAKE), ("s", None))]
    assert f(*args(surv=None)) == bd.EINVAL
    assert f(*args(stats=None)) == bd.EINVAL
    assert f(*args(R=0)) == bd.EINVAL
    assert f(*args(gamma=0)) == bd.EINVAL
    assert f(*args(n=255)) == bd.EINVAL                      # the table must reach B = R
    assert f(*args(gamma=17)) == bd.EUNSUPPORTED
    assert f(*args(R=2341, n=20000)) == bd.EUNSUPPORTED      # R * gamma > 16384
    assert "16384" in bd.last_error()


def test_block_logits_and_loss_validation(L):
    f = L.dspark_apply_block_logits
    args = lambda **k: [k.get(n, d) for n, d in (
        ("U", FAKE), ("B", 4), ("gamma", 7), ("V", 151936), ("prev", FAKE), ("A", FAKE), ("Bm", FAKE),
        ("dt", bd.BF16), ("r", 256), ("out", FAKE), ("s", None))]
    assert f(*args(U=None)) == bd.EINVAL
    assert f(*args(out=None)) == bd.EINVAL
    assert f(*args(r=0)) == bd.EINVAL
    assert f(*args(r=1025)) == bd.EUNSUPPORTED
    assert f(*args(dt=7)) == bd.EUNSUPPORTED
    st, n = _ws(L.dspark_compute_loss_workspace, 4, 7, 151936)
    assert st == bd.OK and n > 4 * 7 * 16
    assert _ws(L.dspark_compute_loss_workspace, 4, 17, 151936)[0] == bd.EUNSUPPORTED
    g = L.dspark_compute_loss
    largs = lambda **k: [k.get(n, d) for n, d in (
        ("draft", FAKE), ("teacher", FAKE), ("target", FAKE), ("conf", None), ("valid", None), ("B", 4),
        ("gamma", 7), ("V", 151936), ("lce", 0.1), ("ll1", 0.9), ("lcf", 1.0), ("decay", 4.0), ("cd", 0),
        ("per", None), ("losses", FAKE), ("ws", None), ("wsb", 0), ("status", None), ("s", None))]
    assert g(*largs(target=None)) == bd.EINVAL
    assert g(*largs(losses=None)) == bd.EINVAL
    assert g(*largs(decay=0.0)) == bd.EINVAL
    assert g(*largs(decay=float("nan"))) == bd.EINVAL
    assert g(*largs(gamma=17)) == bd.EUNSUPPORTED
    assert g(*largs(V=151934)) == bd.EUNSUPPORTED
    assert g(*largs(draft=MISALIGNED)) == bd.EUNSUPPORTED
    assert g(*largs()) == bd.EWORKSPACE
    assert g(*largs(status=FAKE + 3)) == bd.EINVAL


def test_verify_validation(L):
    st, n = _ws(L.dspark_verify_workspace, 256, 7, 151936)
    assert st == bd.OK and n > 256 * 15 * 8
    assert _ws(L.dspark_verify_workspace, 256, 17, 151936)[0] == bd.EUNSUPPORTED
    f = L.dspark_verify
    args = lambda **k: [k.get(n, d) for n, d in (
        ("t", FAKE), ("d", FAKE), ("tok", FAKE), ("len", None), ("seeds", FAKE), ("off", 0), ("B", 4),
        ("gamma", 7), ("V", 151936), ("acc", FAKE), ("nxt", FAKE), ("ap", None), ("ws", None), ("wsb", 0),
        ("s", None))]
    assert f(*args(seeds=None)) == bd.EINVAL
    assert f(*args(nxt=None)) == bd.EINVAL
    assert f(*args(gamma=0)) == bd.EINVAL
    assert f(*args(gamma=17)) == bd.EUNSUPPORTED
    assert f(*args(V=151934)) == bd.EUNSUPPORTED
    assert f(*args(t=MISALIGNED)) == bd.EUNSUPPORTED
    assert f(*args()) == bd.EWORKSPACE



def test_head_variant_validation(L):
    st, n = _ws(L.dspark_markov_propose_head_workspace, 1, 4, 7, 151936, 256, bd.BF16, 16)
    st0, n0 = _ws(L.dspark_markov_propose_workspace, 4, 7, 151936, 16)
    assert st == bd.OK and st0 == bd.OK and n >= n0 + 4 * 7 * 256 * 2
    assert _ws(L.dspark_markov_propose_head_workspace, 0, 4, 7, 151936, 256, bd.BF16, 16)[1] == n0
    st3, n3 = _ws(L.dspark_markov_propose_head_workspace, 3, 4, 7, 151936, 256, bd.BF16, 16)
    assert st3 == bd.OK and n3 >= n0 + 2 * 4 * 7 * 256 * 2                  # RNN: m_j and state tables
    assert _ws(L.dspark_markov_propose_head_workspace, 4, 4, 7, 151936, 256, bd.BF16, 16)[0] == bd.EINVAL
    f = L.dspark_markov_propose_head
    args = lambda **k: [k.get(n, d) for n, d in (
        ("head", 2), ("h", FAKE), ("H", 2560), ("Wg", FAKE), ("U", FAKE), ("B", 4), ("gamma", 7),
        ("V", 151936), ("anchor", FAKE), ("A", FAKE), ("Bm", FAKE), ("dt", bd.BF16), ("r", 256),
        ("T", 0.0), ("seeds", None), ("off", 0), ("topk", 0), ("tok", FAKE), ("tl", None), ("lse", None),
        ("ti", None), ("tp", None), ("lo", None), ("ws", None), ("wsb", 0), ("status", None), ("s", None))]
    assert f(*args(head=5)) == bd.EINVAL
    assert f(*args(h=None)) == bd.EINVAL
    assert f(*args(Wg=None)) == bd.EINVAL
    assert f(*args(H=16385)) == bd.EUNSUPPORTED
    assert f(*args()) == bd.EWORKSPACE
    assert f(*args(head=1, h=None, Wg=None, H=0)) == bd.EWORKSPACE     # SiLU needs no h
    assert f(*args(head=3, h=None)) == bd.EINVAL                       # the RNN head reads h and W
    assert f(*args(head=3, Wg=None)) == bd.EINVAL
    assert f(*args(head=3, H=16385)) == bd.EUNSUPPORTED
    assert f(*args(head=3)) == bd.EWORKSPACE
    assert f(*args(head=3, status=FAKE + 2)) == bd.EINVAL


def test_device_status_word_host_check():
    """The host side of the device status word: DSPARK_OK passes, the
    time-out value raises ETIMEOUT, anything else raises with its value (the
    words here are host tensors standing in for ones read back from the GPU)."""
    import torch
    bd.check_device_status(torch.zeros(2, dtype=torch.int32))
    with pytest.raises(bd.DsparkError) as e:
        bd.check_device_status(torch.tensor([0, bd.ETIMEOUT], dtype=torch.int32), "overlap")
    assert e.value.status == bd.ETIMEOUT and "overlap" in str(e.value)
    with pytest.raises(bd.DsparkError) as e:
        bd.check_device_status(torch.tensor([7], dtype=torch.int32))
    assert e.value.status == 7
    # the header's value of the time-out status is the binding's
    with open(bd.HEADER) as f:
        assert "DSPARK_ETIMEOUT = 5" in f.read()
    assert bd.ETIMEOUT == 5


def test_noalloc_validation(L):
    """The no-allocation propose call checks its arguments like
    dspark_markov_propose and rejects sizes beyond its static scratch before
    any device work."""
    f = L.dspark_markov_propose_noalloc
    args = lambda **k: [k.get(n, d) for n, d in (
        ("U", FAKE), ("B", 4), ("gamma", 7), ("V", 151936), ("anchor", FAKE), ("A", FAKE), ("Bm", FAKE),
        ("dt", bd.BF16), ("r", 256), ("T", 0.0), ("seeds", None), ("off", 0), ("topk", 0), ("tok", FAKE),
        ("tl", None), ("lse", None), ("ti", None), ("tp", None), ("lo", None), ("status", None), ("s", None))]
    assert f(*args(U=None)) == bd.EINVAL
    assert f(*args(T=1.0)) == bd.EINVAL                       # sampling without seeds
    assert f(*args(status=FAKE + 2)) == bd.EINVAL
    assert f(*args(gamma=17)) == bd.EUNSUPPORTED
    assert f(*args(A=MISALIGNED)) == bd.EUNSUPPORTED
    # B = 256 with top-16 needs 211 MiB of workspace; the scratch holds 64 MiB
    assert f(*args(B=256, topk=16, ti=FAKE, tp=FAKE)) == bd.EWORKSPACE
    assert "static scratch" in bd.last_error() and str(64 << 20) in bd.last_error()
