"""Pins for oracle.rowstats: closed forms, library routines, invariants and a
50-digit brute force at V <= 8. None of the pages prints a worked example."""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import rowstats
from oracle import rowstats as R


def _decimal_stats(a, b):
    """Brute force with 50-digit decimals, straight from the definitions."""
    getcontext().prec = 50
    A = [Decimal(float(x)) for x in a]
    B = [Decimal(float(x)) for x in b]
    za = sum(x.exp() for x in A)
    zb = sum(x.exp() for x in B)
    pa = [x.exp() / za for x in A]
    pb = [x.exp() / zb for x in B]
    kl = sum(p * (p.ln() - q.ln()) for p, q in zip(pa, pb))
    h = -sum(p * p.ln() for p in pa)
    return dict(lse_v=float(za.ln()), lse_d=float(zb.ln()), kl=float(kl), entropy=float(h),
                conf=float(max(pa)))


@pytest.mark.parametrize("V", [1, 2, 3, 5, 8])
def test_brute_force_decimal(V):
    rng = np.random.default_rng(100 + V)
    for scale in (0.1, 1.0, 5.0, 30.0):
        a = rng.standard_normal((6, V)) * scale + rng.uniform(-50, 50)
        b = a + rng.standard_normal((6, V)) * scale * 0.7 + rng.uniform(-3, 3)
        st = rowstats.row_stats(a, b)
        for r in range(6):
            ref = _decimal_stats(a[r], b[r])
            for key in ("lse_v", "lse_d", "kl", "entropy", "conf"):
                assert st[key][r] == pytest.approx(ref[key], rel=1e-10, abs=1e-12), (key, scale, r)


def test_lse_matches_scipy():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 3001)) * 4 + 100
    np.testing.assert_allclose(rowstats.log_sum_exp(x), scipy.special.logsumexp(x, axis=1), rtol=1e-14)
    x = np.array([[1000.0, 999.0, -1000.0]])
    np.testing.assert_allclose(rowstats.log_sum_exp(x), scipy.special.logsumexp(x, axis=1), rtol=1e-15)


def test_kl_identical_and_shift_invariant():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((5, 777)) * 3
    st = rowstats.row_stats(a, a)
    assert np.all(st["kl"] == 0.0)
    st = rowstats.row_stats(a, a + 12.5)  # the same distribution
    np.testing.assert_allclose(st["kl"], 0.0, atol=1e-12)


def test_kl_direction_and_library():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((9, 500)) * 2
    b = a + rng.standard_normal((9, 500))
    st = rowstats.row_stats(a, b)
    pv = scipy.special.softmax(a, axis=1)
    pd = scipy.special.softmax(b, axis=1)
    ref = scipy.special.rel_entr(pv, pd).sum(axis=1)       # KL(p_v || p_d)
    rev = scipy.special.rel_entr(pd, pv).sum(axis=1)
    np.testing.assert_allclose(st["kl"], ref, rtol=1e-11)
    assert not np.allclose(st["kl"], rev, rtol=1e-3)
    np.testing.assert_allclose(st["kl"], scipy.stats.entropy(pv, pd, axis=1), rtol=1e-11)
    assert np.all(st["kl"] > 0)  # Gibbs' inequality, strict for distinct distributions


@pytest.mark.parametrize("p,q", [(0.3, 0.6), (0.99, 0.01), (0.5, 0.5), (1e-6, 0.2)])
def test_kl_two_point_closed_form(p, q):
    a = np.log(np.array([[p, 1 - p]]))
    b = np.log(np.array([[q, 1 - q]]))
    ref = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
    assert rowstats.row_stats(a, b)["kl"][0] == pytest.approx(ref, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("V", [1, 2, 17, 1024, 151936])
def test_uniform_row(V):
    a = np.full((1, V), -3.25)
    st = rowstats.row_stats(a, a)
    assert st["entropy"][0] == pytest.approx(math.log(V), rel=1e-12, abs=1e-14)
    assert st["conf"][0] == pytest.approx(1.0 / V, rel=1e-12)
    assert st["lse_v"][0] == pytest.approx(-3.25 + math.log(V), rel=1e-13)
    assert st["argmax_v"][0] == 0  # all tied: lowest index


@pytest.mark.parametrize("V,delta", [(2, 0.5), (10, 3.0), (1000, 7.0), (126464, 12.0), (64, 40.0)])
def test_spike_closed_forms(V, delta):
    a = np.zeros((1, V))
    a[0, V // 3] = delta
    st = rowstats.row_stats(a, a)
    z = 1 + (V - 1) * math.exp(-delta)
    h = math.log(z) + (V - 1) * delta * math.exp(-delta) / z
    assert st["entropy"][0] == pytest.approx(h, rel=1e-11, abs=1e-14)
    assert st["conf"][0] == pytest.approx(1 / z, rel=1e-12)
    assert st["argmax_v"][0] == V // 3
    if delta >= 40:
        assert st["conf"][0] == pytest.approx(1.0, abs=1e-15)


def test_entropy_and_conf_bounds_and_library():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((20, 300)) * rng.uniform(0.1, 8, size=(20, 1))
    st = rowstats.row_stats(a, a)
    assert np.all(st["entropy"] >= 0) and np.all(st["entropy"] <= math.log(300) + 1e-12)
    assert np.all(st["conf"] >= 1 / 300 - 1e-15) and np.all(st["conf"] <= 1)
    pv = scipy.special.softmax(a, axis=1)
    np.testing.assert_allclose(st["entropy"], scipy.stats.entropy(pv, axis=1), rtol=1e-11)
    np.testing.assert_allclose(st["conf"], pv.max(axis=1), rtol=1e-12)


def test_argmax_lowest_index_on_ties():
    a = np.array([[1.0, 3.0, 2.0, 3.0, 3.0],
                  [5.0, 5.0, 5.0, 5.0, 5.0],
                  [0.0, -1.0, 0.0, -2.0, 0.0]])
    b = a[:, ::-1].copy()
    st = rowstats.row_stats(a, b)
    assert list(st["argmax_v"]) == [1, 0, 0]
    assert list(st["argmax_d"]) == [0, 0, 0]


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    vals = rowstats.widen_bf16(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625                     # 0x4049 = 1.5703125 * 2
    assert vals[5] == pytest.approx(3.3895313892515355e38, rel=1e-15)
    assert vals[6] == 2.0 ** -133                  # smallest bf16 subnormal


def test_rejects_non_finite_and_empty_vocab():
    with pytest.raises(ValueError):
        rowstats.row_stats(np.array([[0.0, np.inf]]), np.zeros((1, 2)))
    with pytest.raises(ValueError):
        rowstats.row_stats(np.zeros((1, 0)), np.zeros((1, 0)))


def test_empty_rows():
    st = rowstats.row_stats(np.zeros((0, 5)), np.zeros((0, 5)))
    assert all(len(v) == 0 for v in st.values())


# --- variants: reverse KL, -inf logits, probability of a given token ----

def test_kl_reverse_direction_and_closed_form():
    rng = np.random.default_rng(3)
    a, b = rng.standard_normal((5, 9)), rng.standard_normal((5, 9)) * 2
    # the reverse divergence is the forward one with the models exchanged
    np.testing.assert_allclose(R.kl_reverse(a, b), R.row_stats(b, a)["kl"], rtol=1e-12)
    # two tokens: KL(q || p) = q ln(q/p) + (1-q) ln((1-q)/(1-p))
    p, q = 0.3, 0.8
    a2 = np.log([[p, 1 - p]]); b2 = np.log([[q, 1 - q]])
    want = q * np.log(q / p) + (1 - q) * np.log((1 - q) / (1 - p))
    np.testing.assert_allclose(R.kl_reverse(a2, b2), [want], rtol=1e-12)


def test_neg_inf_entries_are_absent_tokens():
    rng = np.random.default_rng(4)
    V = 12
    a, b = rng.standard_normal((3, V)) * 2, rng.standard_normal((3, V))
    drop = np.array([1, 5, 6, 11])
    ai, bi = a.copy(), b.copy()
    ai[:, drop] = -np.inf
    bi[:, drop] = -np.inf
    keep = np.setdiff1d(np.arange(V), drop)
    got = R.row_stats(ai, bi, neg_inf=True)
    ref = R.row_stats(a[:, keep], b[:, keep])
    for k in ("lse_v", "lse_d", "kl", "entropy", "conf"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(got["argmax_v"], keep[ref["argmax_v"]])
    np.testing.assert_allclose(R.kl_reverse(ai, bi, neg_inf=True), R.kl_reverse(a[:, keep], b[:, keep]), rtol=1e-12)
    with pytest.raises(ValueError):
        R.row_stats(ai, bi)                       # -inf only when asked for


def test_neg_inf_divergence_to_a_zero():
    a = np.array([[0.0, 1.0, -np.inf]])
    b = np.array([[0.0, -np.inf, 2.0]])
    # the verifier puts mass on token 1 where the drafter has none, and the other way round for token 2
    assert R.row_stats(a, b, neg_inf=True)["kl"][0] == np.inf
    assert R.kl_reverse(a, b, neg_inf=True)[0] == np.inf
    c = np.array([[0.0, 1.0, 2.0]])
    # mass of the drafter only where the verifier has some: KL(p_v || p_d) is finite, the reverse is not
    st = R.row_stats(a, c, neg_inf=True)
    assert np.isfinite(st["kl"][0]) and np.isfinite(st["entropy"][0])
    assert R.kl_reverse(a, c, neg_inf=True)[0] == np.inf
    with pytest.raises(ValueError):
        R.row_stats(np.full((1, 3), -np.inf), c, neg_inf=True)   # a row needs a finite logit


def test_prob_of_token():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((4, 30)) * 3
    st = R.row_stats(a, a)
    np.testing.assert_allclose(R.prob_of(a, st["argmax_v"]), st["conf"], rtol=1e-12)
    total = sum(R.prob_of(a, np.full(4, t)) for t in range(30))
    np.testing.assert_allclose(total, 1.0, rtol=1e-12)
