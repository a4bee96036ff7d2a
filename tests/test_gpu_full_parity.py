"""Whole-population parity at the workloads' full sizes, in the launch configuration bench.py times.

Every row of workloads 2-5 is compared with the CPU oracle (run on the host in worker processes, on the exact
bytes the GPU read), and so is every decision, accepted prefix and selection of each workload's chain, against
the oracle's own chain:
  [DualDiffusion] §2 "Verification algorithms" items 2-3 (workload 2: KL and confidence remasking);
  [COVER] "Method: COVER" parts 2-3 (workload 3: entropy seed score, top-32 seeds, KEEP/REPLACE/REMASK);
  [SPOT] §1 "Coupled-Noise Verification" and §3 (workload 4: every candidate's acceptance depends on all of
  its rows, so every row is checked);
  workload 5: per-row statistics and shared-noise tokens, then the top-64 positions of each sequence by KL.
Integers are exact except the in-band cases (oracle margins or threshold distances within 1e-5), which are
counted and reported (printed as PARITY lines, and appended to the file DV_PARITY_REPORT names, if set)."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from oracle import decide as odecide
from oracle import select as oselect
from parity_util import BAND, OraclePool, compare_stats, decisions_in_band, report, to_numpy, token_band

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch.device("cuda:0")


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def pool():
    with OraclePool() as p:
        yield p


def _topk_parity(gpu_idx, ora_idx, ora_score, k):
    """Per-sequence top-k of the GPU chain against the oracle chain. Sets agree unless the oracle's k-th and
    (k+1)-th scores are within BAND; at each rank the indices agree unless their oracle scores are within BAND
    of each other. Returns the number of in-band sequences / ranks."""
    inband_set = inband_rank = 0
    for s in range(gpu_idx.shape[0]):
        sc = ora_score[s]
        srt = np.sort(sc[np.isfinite(sc)])[::-1]
        kth_gap = srt[k - 1] - srt[k] if len(srt) > k else np.inf
        g, o = gpu_idx[s], ora_idx[s]
        if set(g.tolist()) != set(o.tolist()):
            assert kth_gap <= BAND, f"sequence {s}: selected sets differ with k-th gap {kth_gap}"
            inband_set += 1
            continue
        for j in np.nonzero(g != o)[0]:
            assert abs(sc[g[j]] - sc[o[j]]) <= BAND, f"sequence {s} rank {j}: {g[j]} vs {o[j]}"
            inband_rank += 1
    return inband_set, inband_rank


@pytest.mark.parametrize("num", [2, 3])
def test_full_parity_single_sequence(num, pool):
    """All 512 rows of workload 2 (KL / confidence remasking) and workload 3 (COVER revision)."""
    w = W.workload(num)
    print(f"case: workload {num} ({w.name}), every row and its chain", flush=True)
    dev = _dev()
    a_np, b_np = W.make_logits_numpy(w)
    a = torch.from_numpy(a_np.view(np.int16)).to(dev).view(torch.bfloat16)
    b = torch.from_numpy(b_np.view(np.int16)).to(dev).view(torch.bfloat16)
    got = dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed)
    g = to_numpy(got)
    ref = pool.rows(a_np, b_np, "bf16", w.temperature, w.seed, W.positions(w))
    rep = compare_stats(g, ref, w.temperature, w.name)
    if num == 2:
        for rule in w.rules:
            d, _, _, _ = dv.dv_decide(rule, got, tau_kl=w.tau_kl, conf_thr=w.conf_thr, mask_token=-1)
            rd, _ = odecide.decide(dv.RULES[rule], ref, tau_kl=np.float32(w.tau_kl), conf_thr=np.float32(w.conf_thr),
                                   mask_token=-1)
            band = decisions_in_band(dv.RULES[rule], ref["kl"], ref["conf"], w.tau_kl, w.conf_thr)
            dn = d.cpu().numpy()
            assert not ((dn != rd) & ~band).any(), rule
            rep[f"{rule}_in_band"] = int(band.sum())
            rep[f"{rule}_remask"] = int((dn == dv.DV_REMASK).sum())
    else:
        committed = W.committed_rows(w)
        d_in, d_out = W.diffusion_inputs(w)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        score = dv.dv_seed_score(got["entropy"], t(d_in), t(d_out), t(committed))
        idx, _, _, mask = dv.dv_select_topk(score.view(w.B, w.L), w.topk, eligible=t(committed).view(w.B, w.L),
                                            want_mask=True)
        d, _, _, _ = dv.dv_decide("COVER", got, conf_thr=w.conf_thr, mask_token=-1, subject=mask.view(-1))
        osc = oselect.seed_score(ref["entropy"], d_in, d_out, committed)
        fin = np.isfinite(osc)
        gs = score.cpu().numpy()
        assert np.array_equal(np.isfinite(gs), fin)
        assert (np.abs(gs[fin] - osc[fin]) <= 1e-5 + 1e-4 * np.abs(osc[fin])).all()
        oi, _, _ = oselect.select_topk(osc.reshape(w.B, w.L), w.topk, eligible=committed.reshape(w.B, w.L))
        gi = idx.cpu().numpy()
        in_set, in_rank = _topk_parity(gi, oi, osc.reshape(w.B, w.L), w.topk)
        rep.update(topk_in_band_sets=in_set, topk_in_band_ranks=in_rank)
        # COVER outcomes on the oracle's own seeds and statistics
        if in_set == 0:
            subj = np.zeros(w.rows, np.uint8)
            subj[oi[0]] = 1
            rd, _ = odecide.decide(odecide.COVER, ref, conf_thr=np.float32(w.conf_thr), mask_token=-1, subject=subj)
            band = decisions_in_band(dv.RULES["COVER"], None, ref["conf"], 0.0, w.conf_thr)
            dn = d.cpu().numpy()
            assert not ((dn != rd) & ~band).any()
            rep["cover_in_band"] = int((band & (subj != 0)).sum())
            rep["cover_counts"] = {int(c): int((dn == c).sum()) for c in range(4)}
    report(f"workload {num} ({w.name}): all {w.rows} rows", rep)


def test_full_parity_spot_tree(pool):
    """All 2048 rows of workload 4 (64 candidates x 32 positions, T = 1, noise shared per position) and every
    candidate's accepted prefix and the best candidate, against the oracle's own coupled acceptance."""
    w = W.workload(4)
    print(f"case: workload 4 ({w.name}), every row and every candidate", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    got = dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period)
    _, _, pre, best = dv.dv_decide("COUPLED_ACCEPT", got, mask_token=-1, group_len=w.group_len, want_prefix=True,
                                   want_best=True)
    g = to_numpy(got)
    gp = pre.cpu().numpy()
    ref = pool.rows(_bits(a), _bits(b), "bf16", w.temperature, w.seed, W.positions(w))
    rep = compare_stats(g, ref, w.temperature, w.name)
    od, _ = odecide.decide(odecide.COUPLED_ACCEPT, ref, mask_token=-1, group_len=w.group_len)
    op = odecide.accepted_prefix(od, w.group_len)
    band = token_band(ref["absmax"], w.temperature)
    near = ((ref["margin_v"] <= band) | (ref["margin_d"] <= band)).reshape(-1, w.group_len)
    inband = 0
    for c in range(len(op)):
        if near[c, : min(op[c], gp[c]) + 1].any():
            inband += 1
            continue
        assert op[c] == gp[c], (c, op[c], gp[c])
    if inband == 0:
        assert int(best.cpu()[0]) == odecide.best_group(op)
    rep.update(candidates=len(op), prefix_in_band=inband, mean_prefix=float(op.mean()),
               best=int(best.cpu()[0]), oracle_best=int(odecide.best_group(op)))
    report(f"workload 4 ({w.name}): all {w.rows} rows, {len(op)} candidates", rep)
    del a, b
    torch.cuda.empty_cache()


def test_full_parity_throughput(pool):
    """All 32 768 rows of workload 5 (32 sequences x 1024, T = 1, noise per row), verified in one launch as the
    benchmark does, and every sequence's top-64 by KL against the oracle's own KL chain."""
    w = W.workload(5)
    print(f"case: workload 5 ({w.name}), every row and every sequence's top-{w.topk}", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    got = dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed)
    idx, _, _, _ = dv.dv_select_topk(got["kl"].view(w.B, w.L), w.topk)
    g = to_numpy(got)
    gi = idx.cpu().numpy()
    pos = W.positions(w)
    totals = {}
    ora_kl = np.zeros(w.rows)
    per = 2                                     # sequences per batch handed to the workers
    for s0 in range(0, w.B, per):
        r0, r1 = s0 * w.L, min(w.B, s0 + per) * w.L
        ref = pool.rows(_bits(a[r0:r1]), _bits(b[r0:r1]), "bf16", w.temperature, w.seed, pos[r0:r1])
        rep = compare_stats({k: v[r0:r1] for k, v in g.items()}, ref, w.temperature, f"{w.name} rows {r0}..{r1}")
        for k, v in rep.items():
            totals[k] = max(totals.get(k, 0), v) if k.startswith("max_") else totals.get(k, 0) + v
        ora_kl[r0:r1] = ref["kl"]
        print(f"  rows {r0}..{r1 - 1} agree", flush=True)
    oi, _, _ = oselect.select_topk(ora_kl.reshape(w.B, w.L), w.topk)
    in_set, in_rank = _topk_parity(gi, oi, ora_kl.reshape(w.B, w.L), w.topk)
    totals.update(topk_in_band_sets=in_set, topk_in_band_ranks=in_rank)
    report(f"workload 5 ({w.name}): all {w.rows} rows, top-{w.topk} of {w.B} sequences", totals)
    del a, b, got
    torch.cuda.empty_cache()
