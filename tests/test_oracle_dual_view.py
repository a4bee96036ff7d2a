"""Pins for oracle.dual_view: without seeds it is PyTorch's own attention (CPU,
float64); the override and the diagonal correction are pinned by what they must
and must not depend on, by a two-position example worked by hand, and by
grouped-query heads reducing to repeated key/value heads."""

import numpy as np
import torch

from oracle import dual_view as DV


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _case(rng, B=2, H=4, Hkv=2, L=9, D=8):
    return (_rand(rng, B, H, L, D), _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D),
            _rand(rng, B, Hkv, L, D), _rand(rng, B, Hkv, L, D))


def test_no_seed_is_plain_attention():
    rng = np.random.default_rng(0)
    q, kc, vc, kp, vp = _case(rng, H=4, Hkv=4)
    o = DV.dual_view_attention(q, kc, vc, kp, vp, np.zeros((2, 9)), scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(kc),
                                                           torch.from_numpy(vc), scale=0.3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_grouped_heads_are_repeated_heads():
    rng = np.random.default_rng(1)
    q, kc, vc, kp, vp = _case(rng, H=6, Hkv=2)
    seed = (rng.random((2, 9)) < 0.4).astype(np.uint8)
    o = DV.dual_view_attention(q, kc, vc, kp, vp, seed, scale=0.5)
    rep = lambda x: np.repeat(x, 3, axis=1)
    o2 = DV.dual_view_attention(q, rep(kc), rep(vc), rep(kp), rep(vp), seed, scale=0.5)
    np.testing.assert_allclose(o, o2, rtol=1e-13)


def test_override_and_diagonal_dependencies():
    rng = np.random.default_rng(2)
    q, kc, vc, kp, vp = _case(rng)
    seed = np.zeros((2, 9), np.uint8); seed[:, [1, 4, 5]] = 1
    o = DV.dual_view_attention(q, kc, vc, kp, vp, seed, scale=0.4)
    # cache equal to the current values: the override changes nothing
    np.testing.assert_allclose(DV.dual_view_attention(q, kc, vc, kc, vc, seed, 0.4),
                               DV.dual_view_attention(q, kc, vc, kc, vc, np.zeros((2, 9)), 0.4), rtol=1e-13)
    # a seed's current K/V reach only its own query (the diagonal); everyone else reads its cache
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, 4] += 5.0; vc2[:, :, 4] -= 3.0
    o2 = DV.dual_view_attention(q, kc2, vc2, kp, vp, seed, 0.4)
    others = [i for i in range(9) if i != 4]
    np.testing.assert_allclose(o2[:, :, others], o[:, :, others], rtol=1e-13)
    assert np.abs(o2[:, :, 4] - o[:, :, 4]).max() > 1e-3
    # a seed's cache reaches every query but its own
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[:, :, 4] += 5.0; vp2[:, :, 4] -= 3.0
    o3 = DV.dual_view_attention(q, kc, vc, kp2, vp2, seed, 0.4)
    np.testing.assert_allclose(o3[:, :, 4], o[:, :, 4], rtol=1e-13)
    assert np.abs(o3[:, :, others] - o[:, :, others]).max(axis=(0, 1, 3)).min() > 1e-6
    # non-seed positions: the cache is never read
    kp3, vp3 = kp.copy(), vp.copy()
    kp3[:, :, [0, 2, 3, 6, 7, 8]] = 99.0
    np.testing.assert_allclose(DV.dual_view_attention(q, kc, vc, kp3, vp3, seed, 0.4), o, rtol=1e-13)


def test_two_positions_by_hand():
    # L = 2, D = 1, position 1 is a seed. Query 0 reads k_prev[1], v_prev[1]; query 1 reads its own current k, v.
    q = np.array([[[[1.0], [2.0]]]])
    kc = np.array([[[[0.5], [1.5]]]]); vc = np.array([[[[10.0], [20.0]]]])
    kp = np.array([[[[9.0], [-1.0]]]]); vp = np.array([[[[30.0], [40.0]]]])
    o = DV.dual_view_attention(q, kc, vc, kp, vp, np.array([[0, 1]]), scale=1.0)
    w0 = np.exp([1.0 * 0.5, 1.0 * -1.0]); w0 /= w0.sum()
    w1 = np.exp([2.0 * 0.5, 2.0 * 1.5]); w1 /= w1.sum()
    np.testing.assert_allclose(o[0, 0, 0, 0], w0 @ [10.0, 40.0], rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1, 0], w1 @ [10.0, 20.0], rtol=1e-14)
