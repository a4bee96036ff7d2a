"""Pins for oracle.decide and oracle.select: hand-written truth tables taken
from the pages' statements of the rules, closed forms of the seed score and a
brute-force check of the top-k order."""

import itertools

import numpy as np
import pytest

from oracle import decide as D
from oracle import select as S

K, R, M, N = D.KEEP, D.REPLACE, D.REMASK, D.NONE


def _stats(kl=None, conf=None, tok_v=None, tok_d=None):
    return dict(kl=None if kl is None else np.asarray(kl, float),
                conf=None if conf is None else np.asarray(conf, float),
                tok_v=None if tok_v is None else np.asarray(tok_v, np.int32),
                tok_d=None if tok_d is None else np.asarray(tok_d, np.int32))


def test_trust_keeps_everything():
    st = _stats(kl=[9.0, 0.0], conf=[0.0, 1.0], tok_v=[1, 2], tok_d=[3, 2])
    dec, out = D.decide(D.TRUST, st, tau_kl=0.1, conf_thr=0.9, mask_token=-7)
    assert list(dec) == [K, K] and list(out) == [3, 2]


# (kl, conf) -> expected decision under KL (tau=0.1), CONF (theta=0.9), KL_OR_CONF
TABLE = [
    (0.05, 0.95, K, K, K),
    (0.10, 0.95, K, K, K),     # kl == tau is not above tau
    (0.20, 0.95, M, K, M),
    (0.05, 0.90, K, K, K),     # conf == theta is not below theta
    (0.05, 0.50, K, M, M),
    (0.20, 0.50, M, M, M),
]


@pytest.mark.parametrize("kl,conf,e_kl,e_conf,e_or", TABLE)
def test_threshold_rules_truth_table(kl, conf, e_kl, e_conf, e_or):
    st = _stats(kl=[kl], conf=[conf], tok_v=[4], tok_d=[5])
    for rule, want in ((D.KL, e_kl), (D.CONF, e_conf), (D.KL_OR_CONF, e_or)):
        dec, out = D.decide(rule, st, tau_kl=0.1, conf_thr=0.9, mask_token=-7)
        assert dec[0] == want, rule
        assert out[0] == (-7 if want == M else 5)


# COVER: (tok_v == current, conf >= theta) -> KEEP / REPLACE / REMASK
COVER_TABLE = [
    (True, True, K), (True, False, K), (False, True, R), (False, False, M),
]


@pytest.mark.parametrize("match,confident,want", COVER_TABLE)
def test_cover_truth_table(match, confident, want):
    st = _stats(conf=[0.95 if confident else 0.3], tok_v=[11], tok_d=[11 if match else 12])
    dec, out = D.decide(D.COVER, st, conf_thr=0.9, mask_token=99)
    assert dec[0] == want
    assert out[0] == {K: 11 if match else 12, R: 11, M: 99}[want]
    # an explicit current token takes precedence over the drafter's token
    dec2, out2 = D.decide(D.COVER, st, conf_thr=0.9, mask_token=99, cur_tok=[11])
    assert dec2[0] == K and out2[0] == 11


def test_subject_mask_gives_none_and_current_token():
    st = _stats(kl=[1.0, 1.0, 0.0], conf=[0.0, 0.0, 1.0], tok_v=[1, 2, 3], tok_d=[4, 5, 6])
    dec, out = D.decide(D.KL_OR_CONF, st, tau_kl=0.1, conf_thr=0.9, mask_token=0,
                        subject=[0, 1, 1], cur_tok=[7, 8, 9])
    assert list(dec) == [N, M, K] and list(out) == [7, 0, 9]


def test_coupled_accept_prefix_replace_and_remask():
    # two candidates of 4 rows: the first agrees up to offset 2, the second fully
    tok_v = [5, 6, 7, 8, 1, 2, 3, 4]
    tok_d = [5, 6, 0, 8, 1, 2, 3, 4]
    st = _stats(tok_v=tok_v, tok_d=tok_d)
    dec, out = D.decide(D.COUPLED_ACCEPT, st, mask_token=-1, group_len=4)
    assert list(dec) == [K, K, R, M, K, K, K, K]
    assert list(out) == [5, 6, 7, -1, 1, 2, 3, 4]
    pre = D.accepted_prefix(dec, 4)
    assert list(pre) == [2, 4] and D.best_group(pre) == 1


def test_coupled_accept_identical_tokens_and_subject_skips():
    st = _stats(tok_v=list(range(12)), tok_d=list(range(12)))
    dec, _ = D.decide(D.COUPLED_ACCEPT, st, group_len=3)
    pre = D.accepted_prefix(dec, 3)
    assert list(pre) == [3, 3, 3, 3] and D.best_group(pre) == 0
    # a non-subject disagreeing row neither breaks the prefix nor is decided
    st = _stats(tok_v=[1, 9, 3, 4], tok_d=[1, 2, 3, 5])
    dec, _ = D.decide(D.COUPLED_ACCEPT, st, group_len=4, subject=[1, 0, 1, 1])
    assert list(dec) == [K, N, K, R]
    assert list(D.accepted_prefix(dec, 4, subject=[1, 0, 1, 1])) == [3]


def test_coupled_accept_brute_force():
    rng = np.random.default_rng(0)
    for G in (1, 2, 5):
        for _ in range(50):
            n = G * 4
            tv = rng.integers(0, 3, n)
            td = rng.integers(0, 3, n)
            subj = rng.integers(0, 2, n)
            dec, out = D.decide(D.COUPLED_ACCEPT, _stats(tok_v=tv, tok_d=td), group_len=G,
                                subject=subj, mask_token=-1)
            pre = D.accepted_prefix(dec, G, subject=subj)
            for c in range(4):
                rows = range(c * G, (c + 1) * G)
                bad = [j for j, r in enumerate(rows) if subj[r] and tv[r] != td[r]]
                assert pre[c] == (bad[0] if bad else G)
            assert D.best_group(pre) == min(c for c in range(4) if pre[c] == pre.max())


def test_best_group_ties_and_empty():
    assert D.best_group([3, 5, 5, 1]) == 1
    assert D.best_group([]) == -1


def test_rule_argument_errors():
    st = _stats(tok_v=[1, 2, 3], tok_d=[1, 2, 3])
    with pytest.raises(ValueError):
        D.decide(D.COUPLED_ACCEPT, st, group_len=2)
    with pytest.raises(ValueError):
        D.decide(42, st)


def test_seed_score_closed_forms():
    u = np.array([1.0, 2.0, 0.5, 3.0])
    s = S.seed_score(u, [0.3, 0.0, 1.0, 0.2], [0.3, 1.0, 0.0, 0.2])
    assert s[0] == pytest.approx(1.0) and s[1] == pytest.approx(1.0)
    assert s[2] == pytest.approx(1.0) and s[3] == pytest.approx(3.0)
    s = S.seed_score(u, [0, 0, 0, 0], [0, 0, 0, 0], eligible=[1, 0, 1, 0])
    assert s[0] == 1.0 and s[1] == -np.inf and s[2] == 0.5 and s[3] == -np.inf


def _order_ok(score, elig, idx, cnt, k, largest):
    """Selected entries beat every unselected eligible entry; lower index wins ties."""
    L = score.shape[0]
    sel = [int(i) for i in idx[:cnt]]
    key = (lambda i: (-score[i], i)) if largest else (lambda i: (score[i], i))
    assert sel == sorted(sel, key=key)
    rest = [i for i in range(L) if elig[i] and i not in sel]
    assert len(sel) == min(k, int(np.sum(elig)))
    for i in sel:
        for j in rest:
            assert key(i) < key(j)


def test_topk_brute_force_small():
    rng = np.random.default_rng(1)
    for L in (1, 2, 5, 9):
        for _ in range(40):
            score = rng.integers(0, 4, size=(3, L)).astype(float)   # many ties
            elig = rng.integers(0, 2, size=(3, L))
            for k in range(1, L + 1):
                for largest in (True, False):
                    idx, val, cnt = S.select_topk(score, k, eligible=elig, largest=largest)
                    for s in range(3):
                        _order_ok(score[s], elig[s], idx[s], cnt[s], k, largest)
                        assert np.all(idx[s, cnt[s]:] == -1) and np.all(np.isnan(val[s, cnt[s]:]))
                        np.testing.assert_array_equal(val[s, :cnt[s]], score[s, idx[s, :cnt[s]]])


def test_topk_matches_lexsort_and_threshold_prefix():
    rng = np.random.default_rng(2)
    score = rng.standard_normal((4, 1000)).round(2)
    for largest in (True, False):
        idx, val, cnt = S.select_topk(score, 37, largest=largest)
        for s in range(4):
            order = np.lexsort((np.arange(1000), -score[s] if largest else score[s]))[:37]
            np.testing.assert_array_equal(idx[s], order)
        thr = 1.0 if largest else -1.0
        idx2, val2, cnt2 = S.select_topk(score, 37, largest=largest, use_thr=True, thr=thr)
        for s in range(4):
            keep = (val[s] > thr) if largest else (val[s] < thr)
            assert cnt2[s] == keep.sum()
            np.testing.assert_array_equal(idx2[s, :cnt2[s]], idx[s, :cnt2[s]])


def test_topk_errors():
    with pytest.raises(ValueError):
        S.select_topk(np.zeros((1, 4)), 5)
    with pytest.raises(ValueError):
        S.select_topk(np.zeros((1, 4)), 0)


def test_exhaustive_small_rule_grid():
    # every combination of the inputs the rules read, for the threshold rules
    for kl, conf in itertools.product([0.0, 0.1, 0.2], [0.5, 0.9, 1.0]):
        st = _stats(kl=[kl], conf=[conf], tok_v=[0], tok_d=[0])
        d_or = D.decide(D.KL_OR_CONF, st, tau_kl=0.1, conf_thr=0.9)[0][0]
        d_kl = D.decide(D.KL, st, tau_kl=0.1, conf_thr=0.9)[0][0]
        d_cf = D.decide(D.CONF, st, tau_kl=0.1, conf_thr=0.9)[0][0]
        assert d_or == (M if M in (d_kl, d_cf) else K)


def test_conf_draft_truth_table():
    # REMASK exactly when the verifier's probability of the drafted token is below theta (strict)
    st = dict(p_tok=np.array([0.1, 0.9, 0.95, 0.899999]), tok_d=np.array([3, 4, 5, 6], np.int32),
              tok_v=np.array([3, 0, 0, 0], np.int32))
    dec, out = D.decide(D.CONF_DRAFT, st, conf_thr=0.9, mask_token=-2)
    assert list(dec) == [M, K, K, M] and list(out) == [-2, 4, 5, -2]
    dec, _ = D.decide(D.CONF_DRAFT, st, conf_thr=0.9, subject=[1, 0, 1, 0])
    assert list(dec) == [M, N, K, N]


# --------------------------------------------- stochastic KL remasking ----

def _kl_stats(kl):
    kl = np.asarray(kl, np.float64)
    return {"kl": kl, "tok_d": np.zeros(len(kl), np.int32)}


def test_kl_stochastic_contains_the_threshold_rule():
    # kl > tau always remasks (u < 1), kl = 0 never does (u > 0): the threshold clause of item 2
    n = 5000
    for seed in (0, 1, 2 ** 40 + 7):
        above = D.decide(D.KL_STOCHASTIC, _kl_stats(np.full(n, 0.1000001)), tau_kl=0.1, seed=seed)[0]
        assert (above == D.REMASK).all()
        zero = D.decide(D.KL_STOCHASTIC, _kl_stats(np.zeros(n)), tau_kl=0.1, seed=seed)[0]
        assert (zero == D.KEEP).all()


@pytest.mark.parametrize("frac", [0.05, 0.3, 0.7, 0.95])
def test_kl_stochastic_remask_frequency(frac):
    # below the threshold a row remasks with probability kl / tau: binomial bound at 5 sigma
    n, tau = 40000, 0.2
    dec = D.decide(D.KL_STOCHASTIC, _kl_stats(np.full(n, frac * tau)), tau_kl=tau, seed=11)[0]
    got = (dec == D.REMASK).mean()
    assert abs(got - frac) <= 5 * np.sqrt(frac * (1 - frac) / n)


def test_kl_stochastic_draws_are_uniform_and_keyed_by_position():
    from scipy import stats as sst
    pos = np.arange(50000, dtype=np.int32)
    u = D.remask_uniforms(5, pos).astype(np.float64)
    assert (u > 0).all() and (u < 1).all()
    assert sst.kstest(u, "uniform").pvalue > 1e-4
    # the draw belongs to (seed, position), not to the row: permuting rows with their positions permutes decisions
    rng = np.random.default_rng(0)
    kl = rng.random(4096) * 0.1
    p = rng.permutation(4096)
    d0 = D.decide(D.KL_STOCHASTIC, _kl_stats(kl), tau_kl=0.1, seed=9, pos=np.arange(4096))[0]
    d1 = D.decide(D.KL_STOCHASTIC, _kl_stats(kl[p]), tau_kl=0.1, seed=9, pos=p)[0]
    np.testing.assert_array_equal(d1, d0[p])
    # another seed draws anew; the draw is not the Gumbel noise of any token of the row
    assert (D.decide(D.KL_STOCHASTIC, _kl_stats(kl), tau_kl=0.1, seed=10)[0] != d0).mean() > 0.2
    from oracle import noise as N
    assert np.abs(np.corrcoef(u[:4096], N.uniforms(N.hash_words(5, pos[:4096], 1, start=0)[:, 0]))[0, 1]) < 0.05


def test_kl_stochastic_needs_positive_tau():
    with pytest.raises(ValueError):
        D.decide(D.KL_STOCHASTIC, _kl_stats([0.1]), tau_kl=0.0)
