"""GPU parity of dv_decide, dv_seed_score, dv_select_topk, dv_seed_select and dv_decide_seed_select, alone (fed the
same fp32 inputs as the oracle: exact) and chained after dv_verify_rows on the
workloads (against the oracle's own statistics: exact outside the near-tie
bands)."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from oracle import decide as odecide
from oracle import rowstats
from oracle import select as oselect
from parity_util import BAND, ATOL, RTOL, decisions_in_band, oracle_rows, to_numpy

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch.device("cuda:0")


def _t(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def _oracle_decide(rule, st, tau, theta, mask, subject=None, cur=None, group_len=0):
    st64 = {k: (np.asarray(v, np.float64) if k in ("kl", "conf") else np.asarray(v)) for k, v in st.items()
            if v is not None}
    return odecide.decide(rule, st64, tau_kl=np.float32(tau), conf_thr=np.float32(theta), mask_token=mask,
                          subject=subject, cur_tok=cur, group_len=group_len)


@pytest.mark.parametrize("rows,group_len", [(1, 0), (7, 0), (64, 1), (1000, 0), (960, 4), (960, 32), (960, 96),
                                            (2048, 32), (3000, 1000), (16384, 16), (8192, 4), (20000, 8)])
def test_decide_exact(rows, group_len):
    print(f"case: decide rows={rows} group_len={group_len}", flush=True)
    dev = _dev()
    rng = np.random.default_rng(rows + group_len)
    st = dict(kl=rng.uniform(0, 0.2, rows).astype(np.float32), conf=rng.uniform(0, 1, rows).astype(np.float32),
              tok_v=rng.integers(0, 3, rows).astype(np.int32), tok_d=rng.integers(0, 3, rows).astype(np.int32))
    st["kl"][::17] = np.float32(0.1)          # exactly at the thresholds
    st["conf"][::13] = np.float32(0.9)
    subject = (rng.random(rows) < 0.8).astype(np.uint8)
    cur = rng.integers(0, 3, rows).astype(np.int32)
    gst = {k: _t(v, dev) for k, v in st.items()}
    rules = ["TRUST", "KL", "CONF", "KL_OR_CONF", "COVER"] + (["COUPLED_ACCEPT"] if group_len else [])
    for rule in rules:
        for use_subject in (False, True):
            for use_cur in (False, True):
                subj = subject if use_subject else None
                c = cur if use_cur else None
                d, o, pre, best = dv.dv_decide(rule, gst, tau_kl=0.1, conf_thr=0.9, mask_token=-9,
                                               subject=None if subj is None else _t(subj, dev),
                                               cur_tok=None if c is None else _t(c, dev), group_len=group_len,
                                               want_prefix=group_len > 0,
                                               want_best=group_len > 0 and not (use_subject and use_cur))
                rd, ro = _oracle_decide(dv.RULES[rule], st, 0.1, 0.9, -9, subj, c, group_len)
                np.testing.assert_array_equal(d.cpu().numpy(), rd, err_msg=f"{rule} decisions")
                np.testing.assert_array_equal(o.cpu().numpy(), ro, err_msg=f"{rule} out_tok")
                if group_len:
                    rp = odecide.accepted_prefix(rd, group_len, subj)
                    np.testing.assert_array_equal(pre.cpu().numpy(), rp, err_msg=f"{rule} prefix")
                    if best is not None:
                        assert int(best.cpu()[0]) == odecide.best_group(rp)


@pytest.mark.parametrize("rows,group_len", [(7, 0), (1000, 0), (960, 32), (2048, 32), (20000, 8)])
def test_decide_kl_stochastic_exact(rows, group_len):
    """KL remasking with its probabilistic clause: the hash-keyed draw and the float32 decision u * tau < kl,
    bit for bit against the oracle, with rows placed exactly on and just above u * tau."""
    print(f"case: decide KL_STOCHASTIC rows={rows} group_len={group_len}", flush=True)
    dev = _dev()
    rng = np.random.default_rng(7 * rows + group_len)
    tau = np.float32(0.1)
    pos_arr = rng.integers(-5, 1 << 20, rows).astype(np.int32)
    for seed, pos, period in ((0, None, 0), (2 ** 40 + 7, pos_arr, 0), (3, None, 32)):
        rpos = pos if pos is not None else ((np.arange(rows) % period) if period else np.arange(rows))
        u = odecide.remask_uniforms(seed, rpos)
        kl = rng.uniform(0, 0.15, rows).astype(np.float32)
        on = (u * tau).astype(np.float32)
        kl[::11] = on[::11]                                   # on the boundary: KEEP (strict)
        kl[5::11] = np.nextafter(on[5::11], np.float32(1))    # just above: REMASK
        kl[3::29] = 0.0
        st = dict(kl=kl, tok_v=rng.integers(0, 3, rows).astype(np.int32), tok_d=rng.integers(0, 3, rows).astype(np.int32))
        gst = {k: _t(v, dev) for k, v in st.items()}
        subject = (rng.random(rows) < 0.8).astype(np.uint8)
        for subj in (None, subject):
            d, o, pre, _ = dv.dv_decide("KL_STOCHASTIC", gst, tau_kl=float(tau), mask_token=-9,
                                        subject=None if subj is None else _t(subj, dev), group_len=group_len,
                                        want_prefix=group_len > 0, seed=seed,
                                        pos=None if pos is None else _t(pos, dev), pos_period=period)
            rd, ro = odecide.decide(odecide.KL_STOCHASTIC, st, tau_kl=tau, mask_token=-9, subject=subj,
                                    group_len=group_len, seed=seed, pos=rpos)
            np.testing.assert_array_equal(d.cpu().numpy(), rd, err_msg=f"seed {seed} decisions")
            np.testing.assert_array_equal(o.cpu().numpy(), ro, err_msg=f"seed {seed} out_tok")
            if group_len:
                np.testing.assert_array_equal(pre.cpu().numpy(), odecide.accepted_prefix(rd, group_len, subj))
        on_boundary = np.zeros(rows, bool)
        on_boundary[::11] = True
        assert (rd[on_boundary & (subject != 0)] == odecide.KEEP).all()   # u * tau < kl is strict


def test_decide_empty_best_group():
    print("case: decide empty", flush=True)
    dev = _dev()
    st = {"tok_v": torch.zeros(0, dtype=torch.int32, device=dev), "tok_d": torch.zeros(0, dtype=torch.int32, device=dev)}
    d, o, pre, best = dv.dv_decide("COUPLED_ACCEPT", st, rows=0, group_len=4, want_prefix=True, want_best=True)
    assert int(best.cpu()[0]) == -1 and d.numel() == 0


def test_seed_score():
    print("case: seed score", flush=True)
    dev = _dev()
    rng = np.random.default_rng(0)
    n = 100003
    u = rng.uniform(0, 12, n).astype(np.float32)
    d_in = rng.uniform(0, 1, n).astype(np.float32)
    d_out = rng.uniform(0, 1, n).astype(np.float32)
    el = (rng.random(n) < 0.5).astype(np.uint8)
    for e in (None, el):
        got = dv.dv_seed_score(_t(u, dev), _t(d_in, dev), _t(d_out, dev), None if e is None else _t(e, dev))
        ref = oselect.seed_score(u, d_in, d_out, e)
        g = got.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref)
        np.testing.assert_array_equal(np.isfinite(g), fin)
        assert np.all(g[~fin] == -np.inf)
        np.testing.assert_allclose(g[fin], ref[fin], rtol=1e-6, atol=0)


@pytest.mark.parametrize("L", [1, 2, 3, 17, 64, 1000, 1024, 2048, 2049, 5000, 16384])
def test_select_topk_exact(L):
    print(f"case: select L={L}", flush=True)
    dev = _dev()
    rng = np.random.default_rng(L)
    nseq = 5 if L <= 5000 else 2
    score = (rng.standard_normal((nseq, L)) * 3).round(1).astype(np.float32)   # many ties
    score[0, : min(L, 5)] = -np.inf
    score[-1, :: 7] = 0.0
    score[-1, 1::7] = -0.0
    el = (rng.random((nseq, L)) < 0.7).astype(np.uint8)
    el[1] = 0                                                                 # a sequence with nothing eligible
    for k in sorted({1, min(L, 3), min(L, 32), min(L, 64), L}):
        for largest in (True, False):
            for use_thr, thr in ((False, 0.0), (True, 0.5), (True, -100.0)):
                for e in (None, el):
                    idx, val, cnt, mask = dv.dv_select_topk(_t(score, dev), k, eligible=None if e is None else _t(e, dev),
                                                            largest=largest, use_thr=use_thr, thr=thr, want_mask=True)
                    ri, rv, rc = oselect.select_topk(score, k, eligible=e, largest=largest, use_thr=use_thr,
                                                     thr=np.float32(thr))
                    ctx = f"L={L} k={k} largest={largest} thr={use_thr, thr} elig={e is not None}"
                    np.testing.assert_array_equal(cnt.cpu().numpy(), rc, err_msg=ctx)
                    np.testing.assert_array_equal(idx.cpu().numpy(), ri, err_msg=ctx)
                    gv = val.cpu().numpy().astype(np.float64)
                    np.testing.assert_array_equal(np.isnan(gv), np.isnan(rv), err_msg=ctx)
                    ok = ~np.isnan(rv)
                    np.testing.assert_array_equal(gv[ok], rv[ok], err_msg=ctx)
                    m = np.zeros((nseq, L), np.uint8)
                    for s in range(nseq):
                        m[s, ri[s, :rc[s]]] = 1
                    np.testing.assert_array_equal(mask.cpu().numpy(), m, err_msg=ctx)


@pytest.mark.parametrize("L", [1, 5, 32, 64, 100, 1024, 2048, 2049, 4096])
def test_seed_select_matches_two_calls(L):
    """dv_seed_select gives, output for output and bit for bit, dv_seed_score followed by dv_select_topk
    (one launch up to 2048 positions, two beyond), and the oracle's selection of those scores."""
    print(f"case: seed select L={L}", flush=True)
    dev = _dev()
    rng = np.random.default_rng(1000 + L)
    nseq = 4
    u = rng.uniform(0, 4, (nseq, L)).round(1).astype(np.float32)       # many equal scores
    d_in = rng.uniform(0, 1, (nseq, L)).round(1).astype(np.float32)
    d_out = rng.uniform(0, 1, (nseq, L)).round(1).astype(np.float32)
    u[0, : min(L, 3)] = 0.0
    seed_el = (rng.random((nseq, L)) < 0.8).astype(np.uint8)
    sel_el = (rng.random((nseq, L)) < 0.7).astype(np.uint8)
    sel_el[1] = 0
    gu, gi, go = _t(u, dev), _t(d_in, dev), _t(d_out, dev)
    bits = lambda x: x.contiguous().view(torch.int32).cpu().numpy()
    for k in sorted({1, min(L, 4), min(L, 64), L}):
        for largest in (True, False):
            for use_thr, thr in ((False, 0.0), (True, 1.0)):
                for se in (None, seed_el):
                    for xe in (None, sel_el):
                        ctx = f"L={L} k={k} largest={largest} thr={use_thr} seed_el={se is not None} sel_el={xe is not None}"
                        gse = None if se is None else _t(se, dev)
                        gxe = None if xe is None else _t(xe, dev)
                        score, idx, val, cnt, mask = dv.dv_seed_select(gu, gi, go, k, seed_eligible=gse,
                                                                       select_eligible=gxe, largest=largest,
                                                                       use_thr=use_thr, thr=thr, want_mask=True)
                        rs = dv.dv_seed_score(gu.view(-1), gi.view(-1), go.view(-1), None if gse is None else gse.view(-1))
                        ri, rv, rc, rm = dv.dv_select_topk(rs.view(nseq, L), k, eligible=gxe, largest=largest,
                                                           use_thr=use_thr, thr=thr, want_mask=True)
                        np.testing.assert_array_equal(bits(score.view(-1)), bits(rs), err_msg=ctx)
                        np.testing.assert_array_equal(idx.cpu().numpy(), ri.cpu().numpy(), err_msg=ctx)
                        np.testing.assert_array_equal(bits(val), bits(rv), err_msg=ctx)
                        np.testing.assert_array_equal(cnt.cpu().numpy(), rc.cpu().numpy(), err_msg=ctx)
                        np.testing.assert_array_equal(mask.cpu().numpy(), rm.cpu().numpy(), err_msg=ctx)
                        if k == min(L, 4) and se is not None:
                            # the selection of those scores, by the oracle
                            oi, _, oc = oselect.select_topk(score.cpu().numpy(), k, eligible=xe, largest=largest,
                                                            use_thr=use_thr, thr=np.float32(thr))
                            np.testing.assert_array_equal(cnt.cpu().numpy(), oc, err_msg=ctx)
                            np.testing.assert_array_equal(idx.cpu().numpy(), oi, err_msg=ctx)
    ref = oselect.seed_score(u.ravel(), d_in.ravel(), d_out.ravel(), seed_el.ravel())
    got = dv.dv_seed_select(gu, gi, go, 1, seed_eligible=_t(seed_el, dev))[0].cpu().numpy().ravel().astype(np.float64)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(np.isfinite(got), fin)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-6, atol=0)


# ---------------------------------------------------------------- chains ----

def _upload_bf16(x, dev):
    return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)


@pytest.mark.parametrize("rule,rows,group_len,prefix,best,nseq,L", [
    ("COUPLED_ACCEPT", 2048, 32, True, True, 64, 32),     # one launch: one-workgroup decisions
    ("KL_OR_CONF", 512, 0, False, False, 1, 512),          # one launch: one wave per 64 rows
    ("COVER", 960, 96, True, True, 3, 320),
    ("KL", 64, 1, True, False, 2, 2048),
    ("COUPLED_ACCEPT", 16384, 16, True, True, 8, 2048),    # the largest one-workgroup batch
    ("CONF", 16400, 16, True, False, 4, 64),               # one launch: one wave per group
    ("COUPLED_ACCEPT", 20000, 8, True, True, 4, 64),       # the decisions' own two launches, then the selection
    ("KL", 1000, 0, False, False, 2, 4096),                 # the selection's own two launches
    ("KL_OR_CONF", 300, 0, False, False, 0, 16),            # no selection
])
def test_decide_seed_select_matches_two_calls(rule, rows, group_len, prefix, best, nseq, L):
    """dv_decide_seed_select gives, output for output and bit for bit, dv_decide followed by
    dv_seed_select, whichever launch it takes."""
    print(f"case: decide+seed select {rule} rows={rows} group_len={group_len} nseq={nseq} L={L}", flush=True)
    dev = _dev()
    rng = np.random.default_rng(rows + 7 * L + group_len)
    st = dict(kl=rng.uniform(0, 0.2, rows).astype(np.float32), conf=rng.uniform(0, 1, rows).astype(np.float32),
              tok_v=rng.integers(0, 3, rows).astype(np.int32), tok_d=rng.integers(0, 3, rows).astype(np.int32))
    gst = {k: _t(v, dev) for k, v in st.items()}
    subject = _t((rng.random(rows) < 0.8).astype(np.uint8), dev) if rule == "COVER" else None
    cur = _t(rng.integers(0, 3, rows).astype(np.int32), dev) if rule == "COVER" else None
    u = _t(rng.uniform(0, 4, (nseq, L)).round(1).astype(np.float32), dev)
    d_in = _t(rng.uniform(0, 1, (nseq, L)).astype(np.float32), dev)
    d_out = _t(rng.uniform(0, 1, (nseq, L)).astype(np.float32), dev)
    seed_el = _t((rng.random((nseq, L)) < 0.8).astype(np.uint8), dev)
    k = min(L, 8)
    dkw = dict(rule=rule, stats=gst, tau_kl=0.1, conf_thr=0.9, mask_token=-9, subject=subject, cur_tok=cur,
               group_len=group_len, want_prefix=prefix, want_best=best)
    skw = dict(u=u, d_in=d_in, d_out=d_out, k=k, seed_eligible=seed_el, select_eligible=seed_el, want_mask=True)
    bits = lambda x: None if x is None else (x.contiguous().view(torch.int32) if x.dtype == torch.float32 else x).cpu().numpy()
    for rep in range(2):
        (d, o, pre, bg), (score, idx, val, cnt, mask) = dv.dv_decide_seed_select(dkw, skw)
        rd, ro, rpre, rbg = dv.dv_decide(dkw["rule"], gst, **{x: v for x, v in dkw.items() if x not in ("rule", "stats")})
        rscore, ridx, rval, rcnt, rmask = dv.dv_seed_select(u, d_in, d_out, k, seed_eligible=seed_el,
                                                            select_eligible=seed_el, want_mask=True)
        for name, x, y in (("decision", d, rd), ("out_tok", o, ro), ("prefix", pre, rpre), ("best", bg, rbg),
                           ("score", score, rscore), ("idx", idx, ridx), ("val", val, rval), ("cnt", cnt, rcnt),
                           ("mask", mask, rmask)):
            if y is None:
                assert x is None, name
                continue
            np.testing.assert_array_equal(bits(x), bits(y), err_msg=f"{name} rep={rep}")
    # the prepared form: one call on fixed buffers, the same outputs
    if nseq > 0:
        bd = dict(decision=torch.empty(rows, dtype=torch.uint8, device=dev),
                  out_tok=torch.empty(rows, dtype=torch.int32, device=dev),
                  prefix=torch.empty(max(1, rows // (group_len or rows)), dtype=torch.int32, device=dev),
                  best=torch.empty(1, dtype=torch.int32, device=dev))
        bs = dict(score=torch.empty((nseq, L), dtype=torch.float32, device=dev),
                  idx=torch.empty((nseq, k), dtype=torch.int32, device=dev),
                  val=torch.empty((nseq, k), dtype=torch.float32, device=dev),
                  cnt=torch.empty(nseq, dtype=torch.int32, device=dev),
                  mask=torch.empty((nseq, L), dtype=torch.uint8, device=dev))
        pd = dv.prepare_decide(rule, gst, bd["decision"], bd["out_tok"], rows=rows, tau_kl=0.1, conf_thr=0.9,
                               mask_token=-9, subject=subject, group_len=group_len,
                               prefix=bd["prefix"] if prefix else None, best=bd["best"] if best else None)
        ps = dv.prepare_seed_select(u, d_in, d_out, seed_el, bs["score"], k, bs["idx"], bs["val"], bs["cnt"],
                                    select_eligible=seed_el, mask=bs["mask"])
        if cur is None:
            dv.prepare_decide_seed_select(pd, ps)()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(bits(bd["decision"]), bits(rd))
            np.testing.assert_array_equal(bits(bd["out_tok"]), bits(ro))
            if best:
                np.testing.assert_array_equal(bits(bd["best"]), bits(rbg))
            np.testing.assert_array_equal(bits(bs["idx"]), bits(ridx))
            np.testing.assert_array_equal(bits(bs["mask"]), bits(rmask))
        # a selection's mask may not be the decisions' subject in the same call
        pd2 = dv.prepare_decide(rule, gst, bd["decision"], bd["out_tok"], rows=rows, tau_kl=0.1, conf_thr=0.9,
                                mask_token=-9, subject=bs["mask"].view(-1)[:rows] if nseq * L >= rows else None,
                                group_len=group_len, prefix=bd["prefix"] if prefix else None,
                                best=bd["best"] if best else None)
        if nseq * L >= rows:
            with pytest.raises(dv.DVError):
                dv.prepare_decide_seed_select(pd2, ps)()


@pytest.mark.parametrize("rule,nseq,L", [("COVER", 1, 512), ("COVER", 3, 2048), ("KL_OR_CONF", 64, 32),
                                          ("CONF_DRAFT", 2, 100), ("KL_STOCHASTIC", 2, 64), ("TRUST", 1, 1),
                                          ("COVER", 2, 4096)])
def test_seed_select_decide_matches_two_calls(rule, nseq, L):
    """dv_seed_select_decide gives, output for output and bit for bit, dv_seed_select followed by dv_decide with
    the selection's mask as the subject (one launch up to 2048 positions, the two calls' launches beyond)."""
    print(f"case: seed select + decide {rule} nseq={nseq} L={L}", flush=True)
    dev = _dev()
    rows = nseq * L
    rng = np.random.default_rng(31 * L + nseq)
    st = dict(kl=rng.uniform(0, 0.2, rows).astype(np.float32), conf=rng.uniform(0, 1, rows).astype(np.float32),
              tok_v=rng.integers(0, 3, rows).astype(np.int32), tok_d=rng.integers(0, 3, rows).astype(np.int32),
              p_tok_d=rng.uniform(0, 1, rows).astype(np.float32))
    st["conf"][::13] = np.float32(0.9)
    gst = {k: _t(v, dev) for k, v in st.items()}
    u = _t(rng.uniform(0, 4, (nseq, L)).round(1).astype(np.float32), dev)
    d_in = _t(rng.uniform(0, 1, (nseq, L)).astype(np.float32), dev)
    d_out = _t(rng.uniform(0, 1, (nseq, L)).astype(np.float32), dev)
    committed = _t((rng.random((nseq, L)) < 0.7).astype(np.uint8), dev)
    k = max(1, min(L, L // 10))
    bits = lambda x: (x.contiguous().view(torch.int32) if x.dtype == torch.float32 else x).cpu().numpy()
    for use_cur in (False, True):
        cur = _t(rng.integers(0, 3, rows).astype(np.int32), dev) if use_cur else None
        skw = dict(u=u, d_in=d_in, d_out=d_out, k=k, seed_eligible=committed, select_eligible=committed)
        dkw = dict(rule=rule, stats=gst, tau_kl=0.1, conf_thr=0.9, mask_token=-9, cur_tok=cur, seed=11,
                   pos_period=L)
        (score, idx, val, cnt, mask), (d, o) = dv.dv_seed_select_decide(skw, dkw)
        rscore, ridx, rval, rcnt, rmask = dv.dv_seed_select(u, d_in, d_out, k, seed_eligible=committed,
                                                            select_eligible=committed, want_mask=True)
        rd, ro, _, _ = dv.dv_decide(rule, gst, tau_kl=0.1, conf_thr=0.9, mask_token=-9, cur_tok=cur, seed=11,
                                    pos_period=L, subject=rmask.view(-1))
        for name, x, y in (("score", score, rscore), ("idx", idx, ridx), ("val", val, rval), ("cnt", cnt, rcnt),
                           ("mask", mask, rmask), ("decision", d, rd), ("out_tok", o, ro)):
            np.testing.assert_array_equal(bits(x), bits(y), err_msg=f"{name} cur={use_cur}")
        # the rows not selected are left undecided with their current token
        m = mask.view(-1).cpu().numpy().astype(bool)
        assert (d.cpu().numpy()[~m] == dv.DV_NONE).all()
    # the prepared form on fixed buffers
    bs = dict(score=torch.empty((nseq, L), dtype=torch.float32, device=dev),
              idx=torch.empty((nseq, k), dtype=torch.int32, device=dev),
              val=torch.empty((nseq, k), dtype=torch.float32, device=dev),
              cnt=torch.empty(nseq, dtype=torch.int32, device=dev),
              mask=torch.empty((nseq, L), dtype=torch.uint8, device=dev),
              decision=torch.empty(rows, dtype=torch.uint8, device=dev),
              out_tok=torch.empty(rows, dtype=torch.int32, device=dev))
    ps = dv.prepare_seed_select(u, d_in, d_out, committed, bs["score"], k, bs["idx"], bs["val"], bs["cnt"],
                                select_eligible=committed, mask=bs["mask"])
    pd = dv.prepare_decide(rule, gst, bs["decision"], bs["out_tok"], rows=rows, tau_kl=0.1, conf_thr=0.9,
                           mask_token=-9)
    dv.prepare_seed_select_decide(ps, pd)()
    # the prepared decision has no current-token array and seed 0, positions r
    pd_ref, po_ref, _, _ = dv.dv_decide(rule, gst, tau_kl=0.1, conf_thr=0.9, mask_token=-9, subject=rmask.view(-1))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(bs["mask"]), bits(rmask))
    np.testing.assert_array_equal(bits(bs["decision"]), bits(pd_ref))
    np.testing.assert_array_equal(bits(bs["out_tok"]), bits(po_ref))


def test_workload_tiny_rules_chain():
    w = W.workload(1)
    print(f"case: workload 1 chain ({w.name})", flush=True)
    dev = _dev()
    a_np, b_np = W.make_logits_numpy(w)
    got = dv.dv_verify_rows(_t(a_np, dev), _t(b_np, dev), temperature=w.temperature, seed=w.seed)
    ref = oracle_rows(a_np, b_np, "fp32", 0.0, w.seed, W.positions(w))
    subject = W.subject_rows(w)
    g = to_numpy(got)
    for rule in ("TRUST", "KL", "CONF", "KL_OR_CONF", "COVER"):
        d, o, _, _ = dv.dv_decide(rule, got, tau_kl=w.tau_kl, conf_thr=w.conf_thr, mask_token=-1,
                                  subject=_t(subject, dev))
        rd, ro = odecide.decide(dv.RULES[rule], ref, tau_kl=w.tau_kl, conf_thr=w.conf_thr, mask_token=-1,
                                subject=subject)
        band = decisions_in_band(dv.RULES[rule], ref["kl"], ref["conf"], w.tau_kl, w.conf_thr)
        bad = (d.cpu().numpy() != rd) & ~band
        assert not bad.any(), (rule, np.nonzero(bad))
        # on the GPU's own statistics the rules agree exactly
        gd, go = _oracle_decide(dv.RULES[rule], g, w.tau_kl, w.conf_thr, -1, subject)
        np.testing.assert_array_equal(d.cpu().numpy(), gd, err_msg=rule)
        np.testing.assert_array_equal(o.cpu().numpy(), go, err_msg=rule)


def test_workload_remask_chain_full_size():
    w = W.workload(2)
    print(f"case: workload 2 chain ({w.name})", flush=True)
    dev = _dev()
    a_np, b_np = W.make_logits_numpy(w)
    got = dv.dv_verify_rows(_upload_bf16(a_np, dev), _upload_bf16(b_np, dev), temperature=0.0, seed=w.seed)
    g = to_numpy(got)
    rows = np.arange(0, w.rows, 9)
    ref = oracle_rows(a_np[rows], b_np[rows], "bf16", 0.0, w.seed, W.positions(w)[rows])
    counts = {}
    for rule in w.rules:
        d, o, _, _ = dv.dv_decide(rule, got, tau_kl=w.tau_kl, conf_thr=w.conf_thr, mask_token=-1)
        dn = d.cpu().numpy()
        gd, go = _oracle_decide(dv.RULES[rule], g, w.tau_kl, w.conf_thr, -1)
        np.testing.assert_array_equal(dn, gd, err_msg=rule)
        rd, _ = odecide.decide(dv.RULES[rule], ref, tau_kl=w.tau_kl, conf_thr=w.conf_thr, mask_token=-1)
        band = decisions_in_band(dv.RULES[rule], ref["kl"], ref["conf"], w.tau_kl, w.conf_thr)
        assert not ((dn[rows] != rd) & ~band).any(), rule
        counts[rule] = {int(c): int((dn == c).sum()) for c in np.unique(dn)}
    print("decision counts", counts, flush=True)


def _oracle_stats_blocks(a_np, b_np, dtype, block=32):
    out = {}
    for s in range(0, a_np.shape[0], block):
        st = rowstats.row_stats(rowstats.as_float64(a_np[s:s + block], dtype), rowstats.as_float64(b_np[s:s + block], dtype))
        for k, v in st.items():
            out.setdefault(k, []).append(v)
    return {k: np.concatenate(v) for k, v in out.items()}


def test_workload_cover_chain_full_size():
    w = W.workload(3)
    print(f"case: workload 3 chain ({w.name})", flush=True)
    dev = _dev()
    a_np, b_np = W.make_logits_numpy(w)
    got = dv.dv_verify_rows(_upload_bf16(a_np, dev), _upload_bf16(b_np, dev), temperature=0.0, seed=w.seed)
    committed = W.committed_rows(w)
    d_in, d_out = W.diffusion_inputs(w)
    score = dv.dv_seed_score(got["entropy"], _t(d_in, dev), _t(d_out, dev), _t(committed, dev))
    idx, val, cnt, mask = dv.dv_select_topk(score.view(w.B, w.L), w.topk, eligible=_t(committed, dev).view(w.B, w.L),
                                            want_mask=True)
    d, o, _, _ = dv.dv_decide("COVER", got, conf_thr=w.conf_thr, mask_token=-1, subject=mask.view(-1))
    g = to_numpy(got)
    # exact on the GPU's own intermediate values
    gs = score.cpu().numpy()
    ri, rv, rc = oselect.select_topk(gs.reshape(w.B, w.L), w.topk, eligible=committed.reshape(w.B, w.L))
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    m = np.zeros(w.rows, np.uint8)
    m[ri[0, :rc[0]]] = 1
    np.testing.assert_array_equal(mask.cpu().numpy().ravel(), m)
    gd, go = _oracle_decide(dv.RULES["COVER"], g, 0.0, w.conf_thr, -1, m)
    np.testing.assert_array_equal(d.cpu().numpy(), gd)
    np.testing.assert_array_equal(o.cpu().numpy(), go)
    # the same step in one launch (the benchmark's): the same selection and decisions
    (_, fidx, _, _, fmask), (fd, fo) = dv.dv_seed_select_decide(
        dict(u=got["entropy"].view(w.B, w.L), d_in=_t(d_in, dev).view(w.B, w.L), d_out=_t(d_out, dev).view(w.B, w.L),
             k=w.topk, seed_eligible=_t(committed, dev).view(w.B, w.L),
             select_eligible=_t(committed, dev).view(w.B, w.L)),
        dict(rule="COVER", stats=got, conf_thr=w.conf_thr, mask_token=-1))
    np.testing.assert_array_equal(fidx.cpu().numpy(), ri)
    np.testing.assert_array_equal(fmask.cpu().numpy().ravel(), m)
    np.testing.assert_array_equal(fd.cpu().numpy(), gd)
    np.testing.assert_array_equal(fo.cpu().numpy(), go)
    # against the oracle's own chain: seed score within tolerance, selection exact unless a near-tie
    ost = _oracle_stats_blocks(a_np, b_np, "bf16")
    np.testing.assert_allclose(g["entropy"], ost["entropy"], rtol=RTOL, atol=ATOL)
    osc = oselect.seed_score(ost["entropy"], d_in, d_out, committed)
    fin = np.isfinite(osc)
    np.testing.assert_allclose(gs[fin], osc[fin], rtol=RTOL, atol=ATOL)
    oi, ov, oc = oselect.select_topk(osc.reshape(w.B, w.L), w.topk, eligible=committed.reshape(w.B, w.L))
    srt = np.sort(osc[fin])[::-1]
    kth_gap = srt[w.topk - 1] - srt[w.topk]
    if kth_gap > BAND:
        assert set(oi[0].tolist()) == set(idx.cpu().numpy()[0].tolist())
    counts = {int(c): int((d.cpu().numpy() == c).sum()) for c in range(4)}
    print("k-th score gap", kth_gap, "decision counts", counts, flush=True)


def test_workload_spot_tree_chain_full_size():
    w = W.workload(4)
    print(f"case: workload 4 chain ({w.name})", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    got = dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period)
    d, o, pre, best = dv.dv_decide("COUPLED_ACCEPT", got, mask_token=-1, group_len=w.group_len, want_prefix=True,
                                   want_best=True)
    g = to_numpy(got)
    gd, go = _oracle_decide(dv.RULES["COUPLED_ACCEPT"], g, 0.0, 0.0, -1, group_len=w.group_len)
    np.testing.assert_array_equal(d.cpu().numpy(), gd)
    np.testing.assert_array_equal(o.cpu().numpy(), go)
    rp = odecide.accepted_prefix(gd, w.group_len)
    np.testing.assert_array_equal(pre.cpu().numpy(), rp)
    assert int(best.cpu()[0]) == odecide.best_group(rp)
    # the benchmark's one-launch form (decisions beside the seed selection): the same decisions and prefixes
    d_in, d_out = torch.rand(w.rows, device=dev), torch.rand(w.rows, device=dev)
    (fd, fo, fpre, fbest), _ = dv.dv_decide_seed_select(
        dict(rule="COUPLED_ACCEPT", stats=got, mask_token=-1, group_len=w.group_len, want_prefix=True,
             want_best=True),
        dict(u=got["entropy"].view(w.B, w.L), d_in=d_in.view(w.B, w.L), d_out=d_out.view(w.B, w.L), k=8))
    np.testing.assert_array_equal(fd.cpu().numpy(), gd)
    np.testing.assert_array_equal(fo.cpu().numpy(), go)
    np.testing.assert_array_equal(fpre.cpu().numpy(), rp)
    assert int(fbest.cpu()[0]) == odecide.best_group(rp)
    # oracle tokens for three whole candidates give the same prefixes (unless a token is a near-tie)
    for c in (0, 17, 63):
        rows = np.arange(c * w.group_len, (c + 1) * w.group_len)
        an = a[c * w.group_len:(c + 1) * w.group_len].view(torch.int16).cpu().numpy().view(np.uint16)
        bn = b[c * w.group_len:(c + 1) * w.group_len].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle_rows(an, bn, "bf16", w.temperature, w.seed, W.positions(w)[rows])
        od, _ = odecide.decide(odecide.COUPLED_ACCEPT, ref, mask_token=-1, group_len=w.group_len)
        op = odecide.accepted_prefix(od, w.group_len)[0]
        near = (ref["margin_v"] <= BAND) | (ref["margin_d"] <= BAND)
        if not near[: min(op, rp[c]) + 1].any():
            assert op == rp[c], (c, op, rp[c])
    print("mean accepted prefix", float(rp.mean()), "best", int(best.cpu()[0]),
          "accept rate", float((g["tok_v"] == g["tok_d"]).mean()), flush=True)


def test_workload_throughput_topk_chain():
    w = W.workload(5)
    print(f"case: workload 5 chain ({w.name})", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    got = dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed)
    idx, val, cnt, _ = dv.dv_select_topk(got["kl"].view(w.B, w.L), w.topk)
    kl = got["kl"].cpu().numpy().reshape(w.B, w.L)
    ri, rv, rc = oselect.select_topk(kl, w.topk)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    del a, b, got
    torch.cuda.empty_cache()


def test_band_set_decisions():
    """Rows calibrated so that confidence and KL straddle the thresholds."""
    print("case: band set", flush=True)
    dev = _dev()
    rng = np.random.default_rng(2024)
    rows, V = 512, 8192
    a = rng.standard_normal((rows, V)).astype(np.float32)
    spike = rng.uniform(7.0, 13.0, rows).astype(np.float32)        # conf spans roughly [0.5, 1)
    tok = rng.integers(0, V, rows)
    a[np.arange(rows), tok] += spike
    b = a + rng.standard_normal((rows, V)).astype(np.float32) * rng.uniform(0.0, 0.6, (rows, 1)).astype(np.float32)
    a16, b16 = W.round_bf16_bits(a), W.round_bf16_bits(b)
    ref = oracle_rows(a16, b16, "bf16", 0.0, 0, np.arange(rows))
    tau = float(np.median(ref["kl"]))
    theta = float(np.median(ref["conf"]))
    got = dv.dv_verify_rows(_upload_bf16(a16, dev), _upload_bf16(b16, dev))
    inband = {}
    for rule in ("KL", "CONF", "KL_OR_CONF", "COVER"):
        d, _, _, _ = dv.dv_decide(rule, got, tau_kl=tau, conf_thr=theta, mask_token=-1)
        rd, _ = odecide.decide(dv.RULES[rule], ref, tau_kl=np.float32(tau), conf_thr=np.float32(theta), mask_token=-1)
        band = decisions_in_band(dv.RULES[rule], ref["kl"], ref["conf"], np.float32(tau), np.float32(theta))
        bad = (d.cpu().numpy() != rd) & ~band
        assert not bad.any(), (rule, np.nonzero(bad))
        inband[rule] = int(band.sum())
        counts = np.bincount(d.cpu().numpy(), minlength=4)
        if rule != "COVER":
            assert counts[dv.DV_REMASK] > 50 and counts[dv.DV_KEEP] > 50, (rule, counts)
    print("in-band rows", inband, flush=True)


def test_conf_draft_rule():
    """CONF_DRAFT: REMASK iff the verifier's probability of the drafted token is below theta."""
    print("case: CONF_DRAFT", flush=True)
    dev = _dev()
    rng = np.random.default_rng(12)
    rows = 999
    p_tok = rng.uniform(0, 1, rows).astype(np.float32)
    p_tok[::7] = np.float32(0.6)                      # exactly at the threshold: KEEP
    tok_d = rng.integers(0, 50, rows).astype(np.int32)
    subject = (rng.random(rows) < 0.7).astype(np.uint8)
    gst = {"p_tok_d": _t(p_tok, dev), "tok_d": _t(tok_d, dev)}
    for subj in (None, subject):
        d, o, _, _ = dv.dv_decide("CONF_DRAFT", gst, conf_thr=0.6, mask_token=-5,
                                  subject=None if subj is None else _t(subj, dev))
        rd, ro = odecide.decide(odecide.CONF_DRAFT, {"p_tok": p_tok.astype(np.float64), "tok_d": tok_d},
                                conf_thr=np.float32(0.6), mask_token=-5, subject=subj)
        np.testing.assert_array_equal(d.cpu().numpy(), rd)
        np.testing.assert_array_equal(o.cpu().numpy(), ro)
