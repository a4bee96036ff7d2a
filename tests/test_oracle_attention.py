"""Pins for oracle.attention (COVER's d_in and d_out): closed forms for uniform
and one-hot attention, the row-stochastic totals, and invariance to the order
of heads."""

import numpy as np

from oracle import attention as A


def _softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_uniform_attention():
    B, H, L = 2, 3, 10
    probs = np.full((B, H, L, L), 1.0 / L)
    qm = np.zeros((B, L), np.uint8); qm[0, [1, 4, 7]] = 1; qm[1, :] = 1
    nc = np.zeros((B, L), np.uint8); nc[0, [2, 3]] = 1
    d_in, d_out = A.influence_drift(probs, qm, nc)
    # every column receives 1/L from each masked row; every row gives 1/L to each new column
    np.testing.assert_allclose(d_in[0], 3.0 / L); np.testing.assert_allclose(d_in[1], L / L)
    np.testing.assert_allclose(d_out[0], 2.0 / L); np.testing.assert_allclose(d_out[1], 0.0)


def test_one_hot_attention():
    rng = np.random.default_rng(0)
    B, H, L = 1, 4, 9
    target = rng.integers(0, L, (H, L))             # row i of head h looks only at column target[h, i]
    probs = np.zeros((B, H, L, L))
    for h in range(H):
        probs[0, h, np.arange(L), target[h]] = 1.0
    qm = (rng.random(L) < 0.5).astype(np.uint8)
    nc = (rng.random(L) < 0.5).astype(np.uint8)
    d_in, d_out = A.influence_drift(probs, qm[None], nc[None])
    want_in = np.zeros(L); want_out = np.zeros(L)
    for h in range(H):
        for i in range(L):
            if qm[i]:
                want_in[target[h, i]] += 1
            want_out[i] += nc[target[h, i]]
    np.testing.assert_array_equal(d_in[0], want_in / H)
    np.testing.assert_array_equal(d_out[0], want_out / H)


def test_totals_and_head_order():
    rng = np.random.default_rng(1)
    B, H, L = 2, 5, 16
    probs = _softmax(rng.standard_normal((B, H, L, L)) * 3)
    qm = (rng.random((B, L)) < 0.4).astype(np.uint8)
    nc = (rng.random((B, L)) < 0.3).astype(np.uint8)
    d_in, d_out = A.influence_drift(probs, qm, nc)
    # each masked row hands out exactly one unit per head
    np.testing.assert_allclose(d_in.sum(axis=1), qm.sum(axis=1), rtol=1e-12)
    assert (d_out >= 0).all() and (d_out <= 1 + 1e-12).all()
    # all columns new: every row gives everything away
    _, full = A.influence_drift(probs, qm, np.ones((B, L)))
    np.testing.assert_allclose(full, 1.0, rtol=1e-12)
    perm = rng.permutation(H)
    d_in2, d_out2 = A.influence_drift(probs[:, perm], qm, nc)
    np.testing.assert_allclose(d_in2, d_in, rtol=1e-12); np.testing.assert_allclose(d_out2, d_out, rtol=1e-12)
    # a sequence's result depends only on its own attention
    d_in3, _ = A.influence_drift(probs[1:], qm[1:], nc[1:])
    np.testing.assert_allclose(d_in3[0], d_in[1], rtol=1e-12)
