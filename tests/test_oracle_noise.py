"""Pins for oracle.noise: MurmurHash3 known answers for the finalizer, hash
and uniform properties, the Gumbel law (KS), Gumbel-max = softmax sampling
(chi-square), the T -> 0 limit and the shared-noise coupling."""

import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import noise

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rotl(x, r):
    return ((x << r) | (x >> (32 - r))) & 0xFFFFFFFF


def _murmur3_x86_32(data: bytes, seed: int) -> int:
    """MurmurHash3_x86_32 body and tail (Appleby), finishing with the oracle's mix32."""
    c1, c2 = 0xCC9E2D51, 0x1B873593
    h = seed & 0xFFFFFFFF
    nblocks = len(data) // 4
    for i in range(nblocks):
        k = int.from_bytes(data[4 * i:4 * i + 4], "little")
        k = (k * c1) & 0xFFFFFFFF
        k = _rotl(k, 15)
        k = (k * c2) & 0xFFFFFFFF
        h ^= k
        h = _rotl(h, 13)
        h = (h * 5 + 0xE6546B64) & 0xFFFFFFFF
    tail = data[4 * nblocks:]
    k = 0
    if len(tail) >= 3:
        k ^= tail[2] << 16
    if len(tail) >= 2:
        k ^= tail[1] << 8
    if len(tail) >= 1:
        k ^= tail[0]
        k = (k * c1) & 0xFFFFFFFF
        k = _rotl(k, 15)
        k = (k * c2) & 0xFFFFFFFF
        h ^= k
    h ^= len(data)
    return int(noise.mix32(h))


def _vectors():
    out = []
    with open(os.path.join(GOLDEN, "murmur3_x86_32.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, seed, want = line.split()
            data = b"" if key == "-" else bytes.fromhex(key)
            out.append((data, int(seed, 16), int(want, 16)))
    return out


def test_murmur3_known_answers():
    vecs = _vectors()
    assert len(vecs) == 12
    for data, seed, want in vecs:
        assert _murmur3_x86_32(data, seed) == want, (data, hex(seed))


def test_mix32_direct_values_and_zero():
    assert int(noise.mix32(0)) == 0
    assert int(noise.mix32(1)) == 0x514E28B7
    assert int(noise.mix32(0xFFFFFFFF)) == 0x81F16F39


def test_mix32_is_a_bijection_on_a_range():
    x = np.arange(1 << 24, dtype=np.uint32) + np.uint32(0x12345678)
    y = noise.mix32(x)
    assert np.unique(y).size == x.size


def test_hash_words_distinct_within_row_and_keyed_on_everything():
    h = noise.hash_words(7, np.array([3], np.int32), 1 << 20)[0]
    assert np.unique(h).size == h.size   # i -> i*step is injective mod 2^32, mix32 bijective
    base = noise.hash_words(7, np.array([3, 4], np.int32), 64)
    assert not np.array_equal(base[0], base[1])                       # position enters
    assert not np.array_equal(base, noise.hash_words(8, np.array([3, 4], np.int32), 64))
    assert not np.array_equal(base, noise.hash_words(7 + (1 << 32), np.array([3, 4], np.int32), 64))
    # a window that starts later is the same counter sequence
    tail = noise.hash_words(7, np.array([3, 4], np.int32), 32, start=32)
    np.testing.assert_array_equal(base[:, 32:], tail)
    # negative positions are their two's-complement words
    np.testing.assert_array_equal(noise.row_keys(5, np.array([-1], np.int32)),
                                  noise.row_keys(5, np.array([0xFFFFFFFF], np.int64)))


def test_hash_avalanche_on_position_and_seed():
    pos = np.arange(4096, dtype=np.int32)
    h0 = noise.hash_words(11, pos, 8)
    h1 = noise.hash_words(11, pos ^ 1, 8)
    flips = np.unpackbits((h0 ^ h1).view(np.uint8)).mean()
    assert abs(flips - 0.5) < 0.01
    h2 = noise.hash_words(11 ^ (1 << 40), pos, 8)
    flips = np.unpackbits((h0 ^ h2).view(np.uint8)).mean()
    assert abs(flips - 0.5) < 0.01


def test_uniforms_exact_cells_and_range():
    h = np.array([0, 1, 511, 512, 0xFFFFFFFF, 0x80000000], np.uint32)
    u = noise.uniforms(h)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[2] == 2.0 ** -24
    assert u[3] == 3 * 2.0 ** -24
    assert u[4] == 1 - 2.0 ** -24
    assert u[5] == 0.5 + 2.0 ** -24
    # every value is an odd multiple of 2^-24 and exact in float32
    rng = np.random.default_rng(0)
    hh = rng.integers(0, 1 << 32, size=100000, dtype=np.uint64).astype(np.uint32)
    uu = noise.uniforms(hh)
    assert np.all(uu.astype(np.float32).astype(np.float64) == uu)
    m = uu * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(np.round(m) % 2 == 1)
    g = noise.gumbel(np.array([2.0 ** -24, 1 - 2.0 ** -24]))
    assert g[0] == pytest.approx(-2.8115, abs=1e-4) and g[1] == pytest.approx(16.6355, abs=1e-4)


def test_uniform_chi_square_and_gumbel_ks():
    u = noise.uniforms(noise.hash_words(2024, np.arange(64, dtype=np.int32), 4096)).ravel()
    counts = np.bincount((u * 1024).astype(np.int64), minlength=1024)
    assert scipy.stats.chisquare(counts).pvalue > 1e-4
    g = noise.gumbel(u)
    assert scipy.stats.kstest(g, scipy.stats.gumbel_r.cdf).pvalue > 1e-4
    # serial pairs of neighbouring vocabulary indices look independent
    uu = u.reshape(64, 4096)
    pairs = (np.floor(uu[:, :-1] * 32) * 32 + np.floor(uu[:, 1:] * 32)).astype(np.int64).ravel()
    assert scipy.stats.chisquare(np.bincount(pairs, minlength=1024)).pvalue > 1e-4


@pytest.mark.parametrize("V,T", [(2, 1.0), (5, 1.0), (8, 0.7), (8, 2.0)])
def test_gumbel_max_samples_softmax(V, T):
    rng = np.random.default_rng(V)
    logits = rng.standard_normal(V) * 1.5
    n = 100000
    a = np.broadcast_to(logits, (n, V))
    tok = noise.gumbel_tokens(a, a, T, seed=99, pos=np.arange(n, dtype=np.int32))["tok_v"]
    counts = np.bincount(tok, minlength=V)
    p = scipy.special.softmax(logits / T)
    assert scipy.stats.chisquare(counts, p * n).pvalue > 1e-4
    # a plausible mistake (sampling softmax(x) instead of softmax(x / T)) is rejected
    if T != 1.0:
        assert scipy.stats.chisquare(counts, scipy.special.softmax(logits) * n).pvalue < 1e-6


def test_zero_temperature_is_argmax_and_small_temperature_limit():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((50, 300)) * 3
    b = a + rng.standard_normal((50, 300))
    pos = np.arange(50, dtype=np.int32)
    t0 = noise.gumbel_tokens(a, b, 0.0, 1, pos)
    np.testing.assert_array_equal(t0["tok_v"], np.argmax(a, axis=1))
    np.testing.assert_array_equal(t0["tok_d"], np.argmax(b, axis=1))
    # g lies in [-2.9293, 18.7150] (a group maximum reaches -ln(-ln(1 - 2^-24) / 8), the value
    # truncated below the smallest maximum -ln(-(1 + 1/8) ln 2^-24)), so a top-2 logit gap above
    # T * 21.6443 fixes the token
    lo = -math.log(-(1 + 1 / 8) * math.log(2.0 ** -24))
    hi = -math.log(-math.log(1 - 2.0 ** -24) / 8)
    assert lo == pytest.approx(-2.92932, abs=1e-5) and hi == pytest.approx(18.71497, abs=1e-5)
    g = noise.noise(1, pos, 300)
    assert g.min() >= lo and g.max() <= hi
    srt = np.sort(a, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    T = float(gap.min()) / (hi - lo + 1e-3)
    tt = noise.gumbel_tokens(a, b, T, 1, pos)
    np.testing.assert_array_equal(tt["tok_v"], np.argmax(a, axis=1))


def test_identical_logits_give_identical_tokens_and_coupling_beats_independent_noise():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((400, 2000)) * 2
    pos = np.arange(400, dtype=np.int32)
    t = noise.gumbel_tokens(a, a, 1.0, 3, pos)
    np.testing.assert_array_equal(t["tok_v"], t["tok_d"])
    b = a + rng.standard_normal(a.shape) * 0.3
    shared = noise.gumbel_tokens(a, b, 1.0, 3, pos)
    agree_shared = np.mean(shared["tok_v"] == shared["tok_d"])
    other = noise.gumbel_tokens(b, b, 1.0, 4, pos)        # drafter drawn with other noise
    agree_indep = np.mean(shared["tok_v"] == other["tok_d"])
    assert agree_shared > 0.5 and agree_indep < 0.05


def test_margin_is_top_two_gap():
    a = np.array([[0.0, 3.0, 1.0, 2.5]])
    t = noise.gumbel_tokens(a, a, 0.0, 0, np.zeros(1, np.int32))
    assert t["margin_v"][0] == pytest.approx(0.5)
    g = noise.gumbel(noise.uniforms(noise.hash_words(0, np.zeros(1, np.int32), 4)))[0]
    t = noise.gumbel_tokens(a, a, 2.0, 0, np.zeros(1, np.int32))
    s = np.sort(a[0] / 2.0 + g)
    assert t["margin_v"][0] == pytest.approx(s[-1] - s[-2], rel=1e-12)
    assert t["tok_v"][0] == int(np.argmax(a[0] / 2.0 + g))


def test_seed_words_use_both_halves():
    assert noise.seed_words(1) != noise.seed_words(1 + (1 << 32))
    assert noise.seed_words(0)[0] == int(noise.mix32(noise.SEED_SALT))
    assert math.isfinite(float(noise.gumbel(np.array([0.5]))[0]))


def _gumbel_ks(x, loc=0.0):
    return scipy.stats.kstest(np.ravel(x), scipy.stats.gumbel_r(loc=loc).cdf).pvalue


def test_grouped_noise_is_iid_gumbel_in_law():
    """DV_NOISE_V2 draws each full group of 8 largest first; the values must still be i.i.d.
    standard Gumbel: marginals, group maxima (Gumbel shifted by ln 8), the place of the maximum
    (uniform) and pairs inside a group (independent)."""
    R, V = 256, 4096
    g = noise.noise(77, np.arange(R, dtype=np.int32), V)
    assert _gumbel_ks(g) > 1e-4
    grp = g.reshape(R, V // 8, 8)
    assert _gumbel_ks(grp.max(axis=2), loc=math.log(8)) > 1e-4
    assert scipy.stats.chisquare(np.bincount(grp.argmax(axis=2).ravel(), minlength=8)).pvalue > 1e-4
    # every place j of a group has the standard law, not only the pooled values
    for j in (0, 3, 7):
        assert _gumbel_ks(grp[:, :, j]) > 1e-4
    # pairs of places: their CDF values fall uniformly on an 8 x 8 grid
    cdf = scipy.stats.gumbel_r.cdf
    for j, k in ((0, 1), (2, 7)):
        a = np.minimum((cdf(grp[:, :, j]) * 8).astype(np.int64), 7).ravel()
        b = np.minimum((cdf(grp[:, :, k]) * 8).astype(np.int64), 7).ravel()
        assert scipy.stats.chisquare(np.bincount(a * 8 + b, minlength=64)).pvalue > 1e-4


def test_grouped_noise_follows_its_definition():
    """The maximum sits where the group word says; the others are the truncated inverse CDF of
    their own words; a partial last group draws each value on its own."""
    pos = np.array([0, 5, -3], dtype=np.int32)
    V = 8 * 37 + 5
    g = noise.noise(9, pos, V)
    w = noise.group_words(9, pos, 37)
    u = noise.uniforms(noise.hash_words(9, pos, V))
    um = noise.uniforms(w)
    for r in range(len(pos)):
        for c in range(37):
            js = int(w[r, c]) & 7
            for j in range(8):
                i = 8 * c + j
                if j == js:
                    want = -math.log(-math.log(um[r, c]) / 8)
                else:
                    want = -math.log(-(math.log(u[r, i]) + math.log(um[r, c]) / 8))
                    assert g[r, i] < g[r, 8 * c + js]
                assert g[r, i] == pytest.approx(want, rel=1e-13, abs=1e-13)
    np.testing.assert_array_equal(g[:, 8 * 37:], noise.gumbel(u[:, 8 * 37:]))
    # the group key differs from the row key: group words are not element words
    assert not np.any(noise.group_words(9, pos, 37) == noise.hash_words(9, pos, 37))


def test_grouped_noise_tests_reject_plausible_mistakes():
    """The law tests above have the power to catch a wrong construction: a maximum without the
    ln 8 shift, or a truncation at the maximum's own uniform instead of its 1/8 power."""
    R, V = 256, 4096
    pos = np.arange(R, dtype=np.int32)
    w = noise.group_words(77, pos, V // 8)
    u = noise.uniforms(noise.hash_words(77, pos, V)).reshape(R, V // 8, 8)
    um = noise.uniforms(w)[:, :, None]
    js = (w & 7).astype(np.int64)[:, :, None]
    no_shift = -np.log(-(np.log(u) + np.log(um)))
    np.put_along_axis(no_shift, js, -np.log(-np.log(um)), axis=2)
    assert _gumbel_ks(no_shift) < 1e-6
    wrong_trunc = -np.log(-(np.log(u) + np.log(um)))
    np.put_along_axis(wrong_trunc, js, -np.log(-np.log(um) / 8), axis=2)
    assert _gumbel_ks(wrong_trunc) < 1e-6
