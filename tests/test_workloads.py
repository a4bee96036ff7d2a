"""The seeded generators: shapes, determinism, bf16 rounding and the recipes'
stated proportions."""

import dataclasses

import numpy as np
import pytest
import torch

import workloads as W


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-40], np.float32)])
    ours = W.round_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert W.round_bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80


def test_generators_are_deterministic_and_shaped():
    w = dataclasses.replace(W.workload(4), B=3, L=4, V=264)
    a1, b1 = W.make_logits_numpy(w)
    a2, b2 = W.make_logits_numpy(w)
    assert a1.shape == (12, 264) and a1.dtype == np.uint16
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(b1, b2)
    a3, _ = W.make_logits_numpy(w, seqs=[1])
    np.testing.assert_array_equal(a3, a1[4:8])
    w1 = W.workload(1)
    a, b = W.make_logits_numpy(w1)
    assert a.dtype == np.float32 and a.shape == (64, 1024)


def test_peaked_and_spiked_recipes():
    rng = np.random.default_rng(1)
    a, b = W.peaked_logits(2000, 500, rng)
    assert abs(np.std(a) - 2.0) < 0.1
    assert abs(np.std(b - a) - 0.5) < 0.02
    assert np.all(a.max(axis=1) > 3)
    a, b = W.spiked_logits(4000, 300, np.random.default_rng(2))
    spiked = a.max(axis=1) > 6
    assert 0.87 < spiked.mean() < 0.93
    moved = spiked & (np.argmax(b, axis=1) != np.argmax(a, axis=1)) & (b.max(axis=1) > 6)
    assert 0.10 < moved.sum() / spiked.sum() < 0.20


def test_masks_and_inputs():
    w = W.workload(1)
    m = W.subject_rows(w)
    assert m.sum() == 16 and m.shape == (64,)
    w3 = W.workload(3)
    c = W.committed_rows(w3)
    assert c.sum() == 256
    d_in, d_out = W.diffusion_inputs(w3)
    assert d_in.dtype == np.float32 and d_in.shape == (512,) and 0 <= d_in.min() and d_in.max() < 1
    assert W.subject_rows(W.workload(2)) is None
    np.testing.assert_array_equal(W.positions(W.workload(4))[:64], np.tile(np.arange(32), 2))
    assert W.workload(4).input_bytes == 2 * 2048 * 151936 * 2


def test_workload_table_matches_stated_sizes():
    assert [W.workload(i).rows for i in range(1, 6)] == [64, 512, 512, 2048, 32768]
    assert [W.workload(i).V for i in range(1, 6)] == [1024, 126464, 152064, 151936, 126464]
    assert W.workload(5).input_bytes == pytest.approx(16.5759e9, rel=1e-4)
