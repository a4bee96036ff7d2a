"""GPU pins of the shared noise, word for word, through dv_debug_noise.

The pages require only that both models draw with the same Gumbel noise ([SPOT]
§1 "Key Terms & Definitions", coupled-noise verification); how it is drawn is
this library's own specification (DV_HASH_V1 words, DV_NOISE_V2 grouping), so
the kernels' words are compared bit for bit with the oracle's, the Gumbel
values within the hardware logarithm's rounding, and the pruning bounds
against every value they cover."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
from oracle import noise as onoise

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
LOG2_LN2 = np.log2(np.log(2.0))

SEEDS = (0, 1, 0xDEADBEEFCAFEF00D, 2 ** 64 - 1)
# (rows, vocab, pos_period, explicit positions)
CASES = ((3, 1000, 0, None), (5, 17, 2, None), (4, 333, 0, [7, -1, 2 ** 31 - 1, -2 ** 31]),
         (2, 151936, 0, [0, 31]), (3, 126464, 0, [0, 1023, 32767]), (6, 8, 0, None), (2, 7, 0, None))


def _dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch.device("cuda:0")


def _positions(rows, pos, period):
    if pos is not None:
        return np.asarray(pos, np.int32)
    r = np.arange(rows)
    return (r % period if period else r).astype(np.int32)


def _call(seed, rows, V, mode, pos, period, chunk_elems=8):
    dev = _dev()
    p = None if pos is None else torch.tensor(pos, dtype=torch.int32, device=dev)
    out = dv.dv_debug_noise(seed, rows, V, mode, chunk_elems=chunk_elems, pos=p, pos_period=period, device=dev)
    torch.cuda.synchronize()
    x = out.cpu().numpy()
    return x.view(np.uint32) if mode in ("index_words", "group_words") else x


@pytest.mark.parametrize("seed", SEEDS)
def test_index_and_group_words_bit_exact(seed):
    print(f"case: index and group words, seed {seed:#x}", flush=True)
    for rows, V, period, pos in CASES:
        ps = _positions(rows, pos, period)
        idx = _call(seed, rows, V, "index_words", pos, period)
        np.testing.assert_array_equal(idx, onoise.hash_words(seed, ps, V), err_msg=f"index words {rows}x{V}")
        grp = _call(seed, rows, V, "group_words", pos, period)
        assert grp.shape == (rows, V // 8)
        np.testing.assert_array_equal(grp, onoise.group_words(seed, ps, V // 8), err_msg=f"group words {rows}x{V}")


def test_group_words_full_size_workload_positions():
    """Every group word the verification pass uses at the SPOT tree workload (32 positions x 151 936) and at the
    first sequence of the throughput workload (1024 positions x 126 464)."""
    print("case: group words at the workloads' positions", flush=True)
    for rows, V in ((32, 151936), (1024, 126464)):
        grp = _call(0, rows, V, "group_words", None, 0)
        np.testing.assert_array_equal(grp, onoise.group_words(0, np.arange(rows, dtype=np.int32), V // 8))


@pytest.mark.parametrize("seed", (0, 0xDEADBEEFCAFEF00D))
def test_noise_values_match_the_definition(seed):
    """The kernels' Gumbel values in log2 units, G = g log2(e) + log2(ln 2), against the oracle's float64 g:
    within the hardware log2's rounding. A missing ln 8 shift (3 in log2 units) or a wrong truncation would
    be off by far more."""
    print(f"case: noise values, seed {seed:#x}", flush=True)
    for rows, V, period, pos in CASES:
        ps = _positions(rows, pos, period)
        G = _call(seed, rows, V, "noise_log2", pos, period).astype(np.float64)
        ref = onoise.noise(seed, ps, V) * LOG2E + LOG2_LN2
        err = np.abs(G - ref)
        tol = 1e-5 + 1e-6 * np.abs(ref)
        assert (err <= tol).all(), f"{rows}x{V}: max err {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"


@pytest.mark.parametrize("chunk_elems", (8, 4))
def test_pruning_bounds_cover_every_value(chunk_elems):
    """Both per-chunk bounds (in registers, and the table the shared-noise path builds) are at least every noise
    value of their chunk, agree with each other on whole chunks, and for a chunk inside a full group are the
    group's maximum itself plus the few-ulp slack."""
    print(f"case: pruning bounds, chunk of {chunk_elems}", flush=True)
    for rows, V in ((5, 1003), (4, 20000), (3, 151936), (2, 126464), (3, 9), (2, 4)):
        G = _call(7, rows, V, "noise_log2", None, 0, chunk_elems)
        bound = _call(7, rows, V, "chunk_bound", None, 0, chunk_elems)
        table = _call(7, rows, V, "table_bound", None, 0, chunk_elems)
        nch = -(-V // chunk_elems)
        pad = np.full((rows, nch * chunk_elems), -np.inf, np.float32)
        pad[:, :V] = G
        cmax = pad.reshape(rows, nch, chunk_elems).max(axis=2)
        whole = (np.arange(nch) + 1) * chunk_elems <= V
        assert (bound[:, whole] >= cmax[:, whole]).all(), f"register bound below a value, V={V}"
        assert np.isinf(bound[:, ~whole]).all()
        assert (table >= cmax).all(), f"table bound below a value, V={V}"
        np.testing.assert_array_equal(table[:, whole], bound[:, whole])
        in_group = (np.arange(nch) * chunk_elems // 8 + 1) * 8 <= V
        gmax = pad[:, :V // 8 * 8].reshape(rows, V // 8, 8).max(axis=2)
        gm = np.repeat(gmax, 8 // chunk_elems, axis=1)[:, :int(in_group.sum())]
        slack = np.abs(gm) * 2.0 ** -19 + 2.0 ** -19
        assert (bound[:, in_group] - gm <= slack).all(), f"full-group bound not tight, V={V}"
