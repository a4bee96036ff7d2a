"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments synchronously (validation runs before any
HIP call, so none of these touches a device)."""

import ctypes
import os
import re

import pytest

from token_verification_row_amd import dlmverify as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlmverify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libdlmverify.so is not built (run __graft_entry__.build())")
    return B.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert names == sorted(["dv_verify_workspace_bytes", "dv_verify_rows", "dv_verify_rows_noalloc", "dv_decide", "dv_seed_score",
                           "dv_select_topk", "dv_seed_select", "dv_decide_seed_select", "dv_seed_select_decide", "dv_tree_accept", "dv_influence_drift_workspace_bytes",
                           "dv_influence_drift", "dv_dual_view_attention", "dv_debug_hash", "dv_debug_noise", "dv_debug_read_probe", "dv_status_str",
                           "dv_last_error", "dv_version"])
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dv_version() == 1


def test_status_strings(lib):
    for code, name in enumerate(["DV_OK", "DV_ERR_NULL", "DV_ERR_SHAPE", "DV_ERR_DTYPE", "DV_ERR_ALIGN",
                                 "DV_ERR_ARG", "DV_ERR_WORKSPACE", "DV_ERR_UNSUPPORTED", "DV_ERR_HIP"]):
        assert lib.dv_status_str(code).decode() == name


FAKE = 1 << 20  # a non-null, 16-byte aligned address that is never dereferenced


def _logits(rows=4, vocab=64, ld=64, dtype=B.DV_BF16, va=FAKE, vb=FAKE, flags=0):
    return B.dv_logits(verifier=va, drafter=vb, dtype=dtype, flags=flags, rows=rows, vocab=vocab, ld=ld)


def _noise(T=0.0, period=0, pos=None):
    return B.dv_noise(temperature=T, reserved=0, seed=0, pos=pos, pos_period=period)


def _verify(lib, lg, nz, tuning=None, out=True, ws=None, ws_bytes=0):
    st = B.dv_row_stats(kl=FAKE)
    return lib.dv_verify_rows(ctypes.byref(lg), ctypes.byref(nz), None if tuning is None else ctypes.byref(tuning),
                              ctypes.byref(st) if out else None, ws, ws_bytes, None)


def test_verify_validation(lib):
    assert lib.dv_verify_rows(None, ctypes.byref(_noise()), None, ctypes.byref(B.dv_row_stats()), None, 0,
                              None) == B.DV_ERR_NULL
    assert _verify(lib, _logits(), _noise(), out=False) == B.DV_ERR_NULL
    assert _verify(lib, _logits(dtype=7), _noise()) == B.DV_ERR_DTYPE
    assert _verify(lib, _logits(flags=2), _noise()) == B.DV_ERR_ARG             # unknown flag
    assert _verify(lib, _logits(rows=0, va=0, vb=0, flags=B.DV_LOGITS_NEG_INF), _noise()) == B.DV_OK
    assert _verify(lib, _logits(rows=-1), _noise()) == B.DV_ERR_SHAPE
    assert _verify(lib, _logits(vocab=0), _noise()) == B.DV_ERR_SHAPE
    assert _verify(lib, _logits(vocab=65, ld=64), _noise()) == B.DV_ERR_SHAPE
    assert _verify(lib, _logits(rows=1 << 31), _noise()) == B.DV_ERR_SHAPE
    assert _verify(lib, _logits(ld=68), _noise()) == B.DV_ERR_ALIGN          # 136 bytes per row
    assert _verify(lib, _logits(va=FAKE + 8), _noise()) == B.DV_ERR_ALIGN
    assert _verify(lib, _logits(vb=0), _noise()) == B.DV_ERR_NULL
    assert _verify(lib, _logits(), _noise(T=-1.0)) == B.DV_ERR_ARG
    assert _verify(lib, _logits(), _noise(T=float("nan"))) == B.DV_ERR_ARG
    assert _verify(lib, _logits(), _noise(T=float("inf"))) == B.DV_ERR_ARG
    assert _verify(lib, _logits(), _noise(period=-3)) == B.DV_ERR_SHAPE
    bad = B.dv_tuning(split=17, shared_noise=-1)
    assert _verify(lib, _logits(), _noise(), tuning=bad) == B.DV_ERR_ARG
    bad = B.dv_tuning(split=-1, shared_noise=-1)
    assert _verify(lib, _logits(), _noise(), tuning=bad) == B.DV_ERR_ARG
    bad = B.dv_tuning(split=0, shared_noise=2)
    assert _verify(lib, _logits(), _noise(), tuning=bad) == B.DV_ERR_ARG
    bad = B.dv_tuning(split=0, shared_noise=-1)
    bad.reserved[1] = 5
    assert _verify(lib, _logits(), _noise(), tuning=bad) == B.DV_ERR_ARG
    bad = B.dv_tuning(split=0, shared_noise=1)   # greedy cannot share noise
    assert _verify(lib, _logits(), _noise(), tuning=bad) == B.DV_ERR_ARG
    assert "shared noise" in lib.dv_last_error().decode()
    # the noise table needs a workspace
    t = B.dv_tuning(split=4, shared_noise=1)
    lg, nz = _logits(rows=8, vocab=4096, ld=4096), _noise(T=1.0, period=4)
    assert _verify(lib, lg, nz, tuning=t) == B.DV_ERR_WORKSPACE
    assert _verify(lib, lg, nz, tuning=t, ws=FAKE, ws_bytes=100) == B.DV_ERR_WORKSPACE
    assert _verify(lib, lg, nz, tuning=t, ws=FAKE + 16, ws_bytes=1 << 20) == B.DV_ERR_ALIGN


def test_verify_empty_rows_is_a_noop(lib):
    assert _verify(lib, _logits(rows=0, va=0, vb=0), _noise()) == B.DV_OK


def test_workspace_query(lib):
    out = ctypes.c_size_t(123)
    lg, nz = _logits(rows=4, vocab=4096, ld=4096), _noise()
    for split in (1, 4, 16):    # slices of a row are combined on chip: no workspace
        t = B.dv_tuning(split=split, shared_noise=0)
        assert lib.dv_verify_workspace_bytes(ctypes.byref(lg), ctypes.byref(nz), ctypes.byref(t),
                                             ctypes.byref(out)) == B.DV_OK
        assert out.value == 0
    assert lib.dv_verify_workspace_bytes(ctypes.byref(lg), ctypes.byref(nz), None, None) == B.DV_ERR_NULL
    # rows sharing positions: a table of the largest noise value per (position, 16-byte chunk)
    lg = _logits(rows=2048, vocab=151936, ld=151936)
    nz = _noise(T=1.0, period=32)
    table = 32 * (151936 // 8) * 4
    for t in (None, B.dv_tuning(split=4, shared_noise=1), B.dv_tuning(split=0, shared_noise=-1)):
        assert lib.dv_verify_workspace_bytes(ctypes.byref(lg), ctypes.byref(nz), None if t is None else ctypes.byref(t),
                                             ctypes.byref(out)) == B.DV_OK
        assert out.value == table
    t = B.dv_tuning(split=0, shared_noise=0)
    assert lib.dv_verify_workspace_bytes(ctypes.byref(lg), ctypes.byref(nz), ctypes.byref(t),
                                         ctypes.byref(out)) == B.DV_OK
    assert out.value == 0
    lg = _logits(rows=2048, vocab=1001, ld=1008)                 # 126 chunks, the last one partly filled
    assert lib.dv_verify_workspace_bytes(ctypes.byref(lg), ctypes.byref(nz), None, ctypes.byref(out)) == B.DV_OK
    assert out.value == ((32 * 126 * 4 + 255) // 256) * 256
    lg = _logits(rows=63, vocab=151936, ld=151936)               # fewer than two rows per position: no table
    assert lib.dv_verify_workspace_bytes(ctypes.byref(lg), ctypes.byref(nz), None, ctypes.byref(out)) == B.DV_OK
    assert out.value == 0


def _decide(lib, rule=B.DV_RULE_KL, rows=8, group_len=0, tau=0.1, thr=0.9, stats=None, subject=None, cur=None,
            decision=FAKE, out_tok=FAKE, prefix=None, best=None):
    a = B.dv_decide_args(rule=rule, tau_kl=tau, conf_thr=thr, mask_token=0, rows=rows, group_len=group_len)
    st = stats if stats is not None else B.dv_row_stats(kl=FAKE, conf=FAKE, tok_v=FAKE, tok_d=FAKE)
    return lib.dv_decide(ctypes.byref(a), ctypes.byref(st), subject, cur, decision, out_tok, prefix, best, None)


def test_decide_validation(lib):
    assert lib.dv_decide(None, None, None, None, None, None, None, None, None) == B.DV_ERR_NULL
    assert _decide(lib, rule=9) == B.DV_ERR_ARG
    assert _decide(lib, rows=-1) == B.DV_ERR_SHAPE
    assert _decide(lib, tau=float("nan")) == B.DV_ERR_ARG
    assert _decide(lib, rule=B.DV_RULE_COUPLED_ACCEPT, group_len=0) == B.DV_ERR_SHAPE
    assert _decide(lib, rule=B.DV_RULE_COUPLED_ACCEPT, group_len=3) == B.DV_ERR_SHAPE   # 3 does not divide 8
    assert _decide(lib, group_len=4, best=FAKE) == B.DV_ERR_NULL                      # best needs prefix
    assert _decide(lib, stats=B.dv_row_stats(conf=FAKE, tok_d=FAKE)) == B.DV_ERR_NULL  # KL needs kl
    assert _decide(lib, rule=B.DV_RULE_COVER, stats=B.dv_row_stats(conf=FAKE, tok_d=FAKE)) == B.DV_ERR_NULL
    assert _decide(lib, stats=B.dv_row_stats(kl=FAKE)) == B.DV_ERR_NULL                # no current token
    assert _decide(lib, rows=0) == B.DV_OK
    assert _decide(lib, rule=B.DV_RULE_KL_STOCHASTIC, tau=0.0) == B.DV_ERR_ARG             # needs tau > 0
    assert _decide(lib, rule=B.DV_RULE_KL_STOCHASTIC, stats=B.dv_row_stats(conf=FAKE, tok_d=FAKE)) == B.DV_ERR_NULL
    a = B.dv_decide_args(rule=B.DV_RULE_KL, tau_kl=0.1, conf_thr=0.9, rows=8, pos_period=-1)
    st = B.dv_row_stats(kl=FAKE, conf=FAKE, tok_v=FAKE, tok_d=FAKE)
    assert lib.dv_decide(ctypes.byref(a), ctypes.byref(st), None, None, FAKE, FAKE, None, None, None) == B.DV_ERR_SHAPE


def test_seed_score_select_hash_validation(lib):
    assert lib.dv_seed_score(-1, None, None, None, None, None, None) == B.DV_ERR_SHAPE
    assert lib.dv_seed_score(4, FAKE, None, FAKE, None, FAKE, None) == B.DV_ERR_NULL
    assert lib.dv_seed_score(0, None, None, None, None, None, None) == B.DV_OK
    sel = lib.dv_select_topk
    assert sel(1, 0, FAKE, None, 1, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_SHAPE
    assert sel(1, 10, FAKE, None, 0, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_ARG
    assert sel(1, 10, FAKE, None, 11, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_ARG
    assert sel(1, 10, FAKE, None, 3, 1, 1, float("inf"), None, None, None, None, None) == B.DV_ERR_ARG
    assert sel(1, 16385, FAKE, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_UNSUPPORTED
    assert sel(1, 10, None, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_NULL
    assert sel(0, 10, None, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_OK
    ss = lib.dv_seed_select
    assert ss(-1, 10, FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_SHAPE
    assert ss(1, 0, FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_SHAPE
    assert ss(1, 16385, FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_UNSUPPORTED
    assert ss(1, 10, FAKE, FAKE, FAKE, None, FAKE, None, 11, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_ARG
    assert ss(1, 10, FAKE, FAKE, FAKE, None, FAKE, None, 3, 1, 1, float("nan"), None, None, None, None, None) == B.DV_ERR_ARG
    assert ss(1, 10, FAKE, None, FAKE, None, FAKE, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_NULL
    assert ss(1, 10, FAKE, FAKE, FAKE, None, None, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_NULL
    assert ss(1 << 30, 16, FAKE, FAKE, FAKE, None, FAKE, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_ERR_SHAPE
    assert ss(0, 10, None, None, None, None, None, None, 3, 1, 0, 0.0, None, None, None, None, None) == B.DV_OK
    assert lib.dv_debug_hash(0, None, 0, -1, 4, FAKE, None) == B.DV_ERR_SHAPE
    assert lib.dv_debug_hash(0, None, -1, 1, 4, FAKE, None) == B.DV_ERR_SHAPE
    assert lib.dv_debug_hash(0, None, 0, 2, 4, None, None) == B.DV_ERR_NULL
    assert lib.dv_debug_hash(0, None, 0, 0, 4, None, None) == B.DV_OK


def test_decide_seed_select_validation(lib):
    """dv_decide_seed_select checks both calls' arguments, then that the two share no memory that either
    writes, before anything is launched (distinct fake device addresses, never dereferenced)."""
    f = lib.dv_decide_seed_select
    buf = lambda i: (1 << 32) + i * (1 << 24)  # disjoint 16 MiB ranges
    st = B.dv_row_stats(kl=buf(0), conf=buf(1), tok_v=buf(2), tok_d=buf(3))

    def call(rule=B.DV_RULE_KL, rows=64, group_len=0, subject=None, decision=buf(4), out_tok=buf(5), prefix=None,
             best=None, nseq=1, L=64, u=buf(6), d_in=buf(7), d_out=buf(8), score=buf(9), k=4, thr=0.0, use_thr=0,
             idx=buf(10), val=buf(11), cnt=buf(12), mask=buf(13)):
        a = B.dv_decide_args(rule=rule, tau_kl=0.1, conf_thr=0.9, mask_token=-1, rows=rows, group_len=group_len)
        return f(ctypes.byref(a), ctypes.byref(st), subject, None, decision, out_tok, prefix, best, nseq, L, u, d_in,
                 d_out, None, score, None, k, 1, use_thr, thr, idx, val, cnt, mask, None)

    # each call's own checks, the decision's first
    assert call(rule=99) == B.DV_ERR_ARG
    assert call(rows=64, group_len=7, best=buf(14), prefix=buf(15)) == B.DV_ERR_SHAPE
    assert call(k=0) == B.DV_ERR_ARG
    assert call(L=16385) == B.DV_ERR_UNSUPPORTED
    assert call(score=None) == B.DV_ERR_NULL
    assert call(use_thr=1, thr=float("inf")) == B.DV_ERR_ARG
    # shared memory: the selection's mask as the decisions' subject, outputs on each other, a decision
    # output on a selection input, a selection output on a decision input
    assert call(subject=buf(13)) == B.DV_ERR_ARG
    assert call(decision=buf(13) + 8) == B.DV_ERR_ARG
    assert call(out_tok=buf(6) + 4) == B.DV_ERR_ARG
    assert call(score=buf(0) + 64) == B.DV_ERR_ARG
    assert call(idx=buf(2)) == B.DV_ERR_ARG
    # nothing to do in either: nothing launched (empty ranges overlap nothing)
    assert call(rows=0, nseq=0) == B.DV_OK
    assert call(rows=0, nseq=0, subject=buf(13)) == B.DV_OK


def test_seed_select_decide_validation(lib):
    """dv_seed_select_decide checks the selection, its mask, the decisions, their shape and rule, and that
    neither part writes what the other touches, before anything is launched."""
    f = lib.dv_seed_select_decide
    buf = lambda i: (1 << 32) + i * (1 << 24)
    st = B.dv_row_stats(kl=buf(0), conf=buf(1), tok_v=buf(2), tok_d=buf(3))

    def call(rule=B.DV_RULE_COVER, rows=128, nseq=2, L=64, k=4, score=buf(9), mask=buf(13), decision=buf(4),
             out_tok=buf(5), cur=None, idx=buf(10), group_len=0):
        a = B.dv_decide_args(rule=rule, tau_kl=0.1, conf_thr=0.9, mask_token=-1, rows=rows, group_len=group_len)
        return f(nseq, L, buf(6), buf(7), buf(8), None, score, None, k, 1, 0, 0.0, idx, buf(11), buf(12), mask,
                 ctypes.byref(a), ctypes.byref(st), cur, decision, out_tok, None)

    assert call(k=0) == B.DV_ERR_ARG                              # the selection's checks first
    assert call(mask=None) == B.DV_ERR_NULL                      # the mask is the decisions' subject
    assert call(rule=99) == B.DV_ERR_ARG                         # then the decisions'
    assert call(rows=100) == B.DV_ERR_SHAPE                      # rows = nseq * seq_len
    assert call(rule=B.DV_RULE_COUPLED_ACCEPT) == B.DV_ERR_SHAPE  # (dv_decide's own check: no groups)
    assert call(rule=B.DV_RULE_COUPLED_ACCEPT, group_len=64) == B.DV_ERR_ARG  # a rule of single rows
    assert call(decision=buf(13) + 3) == B.DV_ERR_ARG            # a decision output on the mask
    assert call(out_tok=buf(8)) == B.DV_ERR_ARG                  # ... on a selection input
    assert call(score=buf(1) + 16) == B.DV_ERR_ARG               # a selection output on conf
    assert call(idx=buf(3)) == B.DV_ERR_ARG                      # ... on the current tokens (tok_d)
    assert call(nseq=0, rows=0) == B.DV_OK                       # nothing to do: nothing launched


def test_debug_noise_validation(lib):
    assert lib.dv_debug_noise(0, None, 0, -1, 4, 0, 8, FAKE, None) == B.DV_ERR_SHAPE
    assert lib.dv_debug_noise(0, None, -1, 1, 4, 0, 8, FAKE, None) == B.DV_ERR_SHAPE
    assert lib.dv_debug_noise(0, None, 0, 1, 4, 5, 8, FAKE, None) == B.DV_ERR_ARG       # unknown mode
    assert lib.dv_debug_noise(0, None, 0, 1, 4, -1, 8, FAKE, None) == B.DV_ERR_ARG
    assert lib.dv_debug_noise(0, None, 0, 1, 4, 0, 2, FAKE, None) == B.DV_ERR_ARG       # chunk_elems
    assert lib.dv_debug_noise(0, FAKE, 0, 1, 64, 4, 8, FAKE, None) == B.DV_ERR_ARG     # table: positions are rows
    assert lib.dv_debug_noise(0, None, 3, 1, 64, 4, 8, FAKE, None) == B.DV_ERR_ARG
    assert lib.dv_debug_noise(0, None, 0, 2, 64, 1, 8, None, None) == B.DV_ERR_NULL
    # group words of a vocabulary shorter than one group: an empty result, nothing launched
    assert lib.dv_debug_noise(0, None, 0, 2, 7, 1, 8, None, None) == B.DV_OK
    assert lib.dv_debug_noise(0, None, 0, 0, 64, 2, 4, None, None) == B.DV_OK


def test_read_probe_validation(lib):
    lg = _logits(rows=4, vocab=64, ld=64)
    assert lib.dv_debug_read_probe(ctypes.byref(lg), None, None, None) == B.DV_ERR_NULL
    bad = _logits(rows=4, vocab=64, ld=60)
    assert lib.dv_debug_read_probe(ctypes.byref(bad), None, FAKE, None) == B.DV_ERR_SHAPE
    t = B.dv_tuning(split=0, shared_noise=1)
    assert lib.dv_debug_read_probe(ctypes.byref(lg), ctypes.byref(t), FAKE, None) == B.DV_ERR_ARG
    t = B.dv_tuning(split=17, shared_noise=0)
    assert lib.dv_debug_read_probe(ctypes.byref(lg), ctypes.byref(t), FAKE, None) == B.DV_ERR_ARG
    empty = _logits(rows=0)
    assert lib.dv_debug_read_probe(ctypes.byref(empty), None, None, None) == B.DV_OK


def test_noalloc_validation(lib):
    """dv_verify_rows_noalloc rejects bad arguments, and a noise table larger than its fixed scratch, before any
    HIP call."""
    st = B.dv_row_stats(kl=FAKE)
    call = lambda lg, nz, t=None: lib.dv_verify_rows_noalloc(ctypes.byref(lg), ctypes.byref(nz),
                                                             None if t is None else ctypes.byref(t), ctypes.byref(st),
                                                             None)
    assert call(_logits(ld=60), _noise()) == B.DV_ERR_SHAPE
    assert call(_logits(), _noise(T=-1.0)) == B.DV_ERR_ARG
    assert call(_logits(), _noise(T=1e-45)) == B.DV_ERR_ARG            # log2(e) / T overflows
    assert lib.dv_verify_rows_noalloc(ctypes.byref(_logits()), ctypes.byref(_noise()), None, None, None) == B.DV_ERR_NULL
    # 128 positions x 19008 chunks x 4 bytes = 9.7 MB of table > 8 MiB of scratch
    big = _logits(rows=256, vocab=152064, ld=152064)
    assert call(big, _noise(T=1.0, period=128)) == B.DV_ERR_UNSUPPORTED
    assert "scratch" in lib.dv_last_error().decode()
    assert call(big, _noise(T=1.0, period=128), B.dv_tuning(split=0, shared_noise=1)) == B.DV_ERR_UNSUPPORTED
    # 8 MiB holds 64 positions of that vocabulary; empty batches launch nothing
    assert call(_logits(rows=0, vocab=152064, ld=152064), _noise(T=1.0, period=64)) == B.DV_OK
    assert B.DV_NOALLOC_SCRATCH_BYTES == 8 << 20


def test_binding_rejects_short_pos(monkeypatch):
    """A pos tensor with fewer entries than rows is refused before any launch (the kernels would read past it)."""
    import torch

    monkeypatch.setattr(B, "_need_cuda", lambda t, name: None)   # a CPU tensor stands in for a device one
    pos = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="3 positions for 4 rows"):
        B._check_pos(pos, 4)
    B._check_pos(pos, 3)
    with pytest.raises(TypeError):
        B._check_pos(torch.zeros(4, dtype=torch.int64), 4)


def test_binding_refuses_cpu_tensors():
    import torch
    a = torch.zeros((2, 8), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        B.dv_verify_rows(a, a)
    with pytest.raises(TypeError):
        B.dv_seed_score(torch.zeros(3), torch.zeros(3), torch.zeros(3))


def _tree(lib, ntrees=1, nodes=4, block_len=8, inputs=FAKE, args=True):
    a = B.dv_tree_args(ntrees=ntrees, nodes=nodes, block_len=block_len)
    return lib.dv_tree_accept(ctypes.byref(a) if args else None, inputs, inputs, inputs, inputs, inputs, inputs,
                              None, None, None, None, None, None, None, None, None)


def test_tree_validation(lib):
    assert _tree(lib, args=False) == B.DV_ERR_NULL
    assert _tree(lib, ntrees=-1) == B.DV_ERR_SHAPE
    assert _tree(lib, nodes=0) == B.DV_ERR_SHAPE
    assert _tree(lib, nodes=1025) == B.DV_ERR_SHAPE
    assert _tree(lib, block_len=0) == B.DV_ERR_SHAPE
    assert _tree(lib, block_len=1025) == B.DV_ERR_SHAPE
    assert _tree(lib, inputs=None) == B.DV_ERR_NULL
    assert _tree(lib, ntrees=0, inputs=None) == B.DV_OK        # nothing to do: no launch


def _att(nseq=1, heads=2, length=512, ld=None, dtype=B.DV_BF16, probs=FAKE):
    return B.dv_attention(probs=probs, dtype=dtype, reserved=0, nseq=nseq, heads=heads, len=length,
                          ld=length if ld is None else ld)


def test_influence_validation_and_workspace(lib):
    out = ctypes.c_size_t(0)
    a = _att(nseq=1, heads=784, length=512)
    assert lib.dv_influence_drift_workspace_bytes(ctypes.byref(a), ctypes.byref(out)) == B.DV_OK
    # one 64-byte partial (8 column sums, 8 row sums) per (map, row tile, group of 8 positions)
    # 784 maps: one row tile each, 64 groups
    assert out.value == 784 * 1 * 64 * 64
    a = _att(nseq=1, heads=32, length=512)                      # 32 maps: 8 tiles of 64 rows
    assert lib.dv_influence_drift_workspace_bytes(ctypes.byref(a), ctypes.byref(out)) == B.DV_OK
    assert out.value == 32 * 8 * 64 * 64
    a = _att(nseq=1, heads=1, length=100, ld=104)
    assert lib.dv_influence_drift_workspace_bytes(ctypes.byref(a), ctypes.byref(out)) == B.DV_OK
    assert out.value == 1 * 2 * 13 * 64                                    # 2 tiles of 56 rows, 13 groups
    def call(att, qm=FAKE, nc=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.dv_influence_drift(ctypes.byref(att) if att is not None else None, qm, nc, None, None, ws, ws_bytes,
                                      None)
    assert call(None) == B.DV_ERR_NULL
    assert call(_att(dtype=9)) == B.DV_ERR_DTYPE
    assert call(_att(heads=0)) == B.DV_ERR_SHAPE
    assert call(_att(nseq=70000)) == B.DV_ERR_SHAPE
    assert call(_att(length=4097)) == B.DV_ERR_SHAPE
    assert call(_att(length=64, ld=32)) == B.DV_ERR_SHAPE
    assert call(_att(length=60, ld=60)) == B.DV_ERR_ALIGN                  # 120-byte rows
    assert call(_att(probs=FAKE + 4)) == B.DV_ERR_ALIGN
    assert call(_att(), qm=None) == B.DV_ERR_NULL
    assert call(_att(), ws=None) == B.DV_ERR_WORKSPACE
    assert call(_att(), ws_bytes=16) == B.DV_ERR_WORKSPACE
    assert call(_att(), ws=FAKE + 16) == B.DV_ERR_ALIGN
    assert call(_att(nseq=0, probs=None), qm=None, nc=None, ws=None) == B.DV_OK   # nothing to do


def test_dual_view_validation(lib):
    def call(args, ptr=FAKE, seed=FAKE):
        return lib.dv_dual_view_attention(ctypes.byref(args) if args is not None else None, ptr, ptr, ptr, ptr, ptr,
                                          seed, ptr, None)
    A = lambda **kw: B.dv_dual_view_args(**{**dict(nseq=1, heads=4, kv_heads=2, len=64, head_dim=128, scale=0.1,
                                                   reserved=0), **kw})
    assert call(None) == B.DV_ERR_NULL
    assert call(A(heads=4, kv_heads=3)) == B.DV_ERR_SHAPE
    assert call(A(len=48)) == B.DV_ERR_SHAPE
    assert call(A(len=0)) == B.DV_ERR_SHAPE
    assert call(A(head_dim=96)) == B.DV_ERR_SHAPE
    assert call(A(nseq=-1)) == B.DV_ERR_SHAPE
    assert call(A(scale=float("nan"))) == B.DV_ERR_ARG
    assert call(A(), ptr=None) == B.DV_ERR_NULL
    assert call(A(), seed=None) == B.DV_ERR_NULL
    assert call(A(), ptr=FAKE + 8) == B.DV_ERR_ALIGN
    assert call(A(nseq=0), ptr=None, seed=None) == B.DV_OK
