"""GPU parity of dv_verify_rows (and the noise hash) against the CPU oracle.

Every case prints its name before it touches the GPU. Sizes: small shapes
that still span many 16-byte chunks, several waves and slices and a ragged
tail; and the five workloads at full size, checked on sampled rows."""

import dataclasses

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from oracle import noise as onoise
from parity_util import compare_stats, oracle_rows, to_numpy

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch.device("cuda:0")


def _upload(x: np.ndarray, dtype: str, dev, ld=None, pad_bits=None):
    """numpy logits (float32 values or bf16 bits) -> device tensor [rows, vocab] view with row pitch ld."""
    rows, V = x.shape
    per16 = 8 if dtype == "bf16" else 4          # the library wants 16-byte row pitches
    ld = -(-V // per16) * per16 if ld is None else ld
    if dtype == "bf16":
        buf = np.zeros((rows, ld), np.uint16)
        if pad_bits is not None:
            buf[:, V:] = pad_bits
        buf[:, :V] = x
        t = torch.from_numpy(buf.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        buf = np.zeros((rows, ld), np.float32)
        if pad_bits is not None:
            buf.view(np.uint32)[:, V:] = pad_bits
        buf[:, :V] = x
        t = torch.from_numpy(buf).to(dev)
    return t[:, :V]


def _peaked(rows, V, seed, dtype):
    rng = np.random.default_rng(seed)
    a, b = W.peaked_logits(rows, V, rng)
    if dtype == "bf16":
        return W.round_bf16_bits(a), W.round_bf16_bits(b)
    return a, b


def _run(a_np, b_np, dtype, T, seed=0, pos=None, period=0, tuning=None, ld=None, pad_bits=None):
    dev = _dev()
    a = _upload(a_np, dtype, dev, ld, pad_bits)
    b = _upload(b_np, dtype, dev, ld, pad_bits)
    pos_t = None if pos is None else torch.from_numpy(np.asarray(pos, np.int32)).to(dev)
    got = dv.dv_verify_rows(a, b, temperature=T, seed=seed, pos=pos_t, pos_period=period, tuning=tuning)
    torch.cuda.synchronize()
    return to_numpy(got)


def _positions(rows, pos=None, period=0):
    if pos is not None:
        return np.asarray(pos, np.int32)
    r = np.arange(rows)
    return (r % period if period else r).astype(np.int32)


def test_noise_hash_bit_exact():
    dev = _dev()
    print("case: noise hash words", flush=True)
    for seed in (0, 1, 0xDEADBEEFCAFEF00D, 2 ** 64 - 1):
        for rows, V, period, pos in ((3, 1000, 0, None), (5, 17, 2, None), (4, 333, 0, [7, -1, 2 ** 31 - 1, -2 ** 31])):
            p = None if pos is None else torch.tensor(pos, dtype=torch.int32, device=dev)
            got = dv.dv_debug_hash(seed, rows, V, pos=p, pos_period=period, device=dev).cpu().numpy().view(np.uint32)
            want = onoise.hash_words(seed, _positions(rows, pos, period), V)
            np.testing.assert_array_equal(got, want)


SHAPES = [
    # (dtype, rows, V)
    ("fp32", 1, 1), ("fp32", 3, 5), ("fp32", 7, 1023), ("fp32", 64, 1024), ("fp32", 9, 4099),
    ("bf16", 1, 1), ("bf16", 2, 7), ("bf16", 5, 8), ("bf16", 4, 9), ("bf16", 33, 1000),
    ("bf16", 6, 20001), ("bf16", 3, 70000), ("bf16", 130, 2056),
]


@pytest.mark.parametrize("dtype,rows,V", SHAPES)
@pytest.mark.parametrize("T", [0.0, 1.0, 0.7])
def test_small_shapes(dtype, rows, V, T):
    print(f"case: small shape {dtype} {rows}x{V} T={T}", flush=True)
    a, b = _peaked(rows, V, rows * 7919 + V, dtype)
    got = _run(a, b, dtype, T, seed=5)
    ref = oracle_rows(a, b, dtype, T, 5, _positions(rows))
    compare_stats(got, ref, T, f"{dtype} {rows}x{V} T={T}")


@pytest.mark.parametrize("dtype,V", [("bf16", (1 << 20) + 5), ("fp32", (1 << 20) + 3)])
def test_large_vocab_ragged(dtype, V):
    """A vocabulary of about 2^20 with a partly filled last chunk: chunk indices past 2^17, long slices,
    the noise table over many chunks (period 2 over 6 rows) and the per-row hash bound."""
    print(f"case: large vocab {dtype} V={V}", flush=True)
    a, b = _peaked(6, V, V, dtype)
    for T in (0.0, 1.0):
        for period, tuning in ((0, None), (2, {"shared_noise": 1}), (2, {"shared_noise": 0, "split": 16})):
            if T == 0.0 and period:
                continue
            got = _run(a, b, dtype, T, seed=21, period=period, tuning=tuning)
            ref = oracle_rows(a, b, dtype, T, 21, _positions(6, None, period))
            compare_stats(got, ref, T, f"large vocab {dtype} T={T} period={period} {tuning}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T", [0.1, 0.02])
def test_low_temperature_flat_rows(dtype, T):
    """Small temperatures on flat (unpeaked) rows, where x/T dominates the perturbed score and its float32
    rounding grows: tokens agree outside the score's rounding band, through the per-row hash bound and the
    shared-noise table."""
    print(f"case: low temperature {dtype} T={T}", flush=True)
    rows, V = 48, 20000
    rng = np.random.default_rng(int(T * 1000) + (dtype == "fp32"))
    a = rng.standard_normal((rows, V), dtype=np.float32)
    b = a + rng.standard_normal((rows, V), dtype=np.float32) * np.float32(0.5)
    if dtype == "bf16":
        a, b = W.round_bf16_bits(a), W.round_bf16_bits(b)
    for period, tuning in ((0, None), (8, {"shared_noise": 1}), (8, {"shared_noise": 0})):
        got = _run(a, b, dtype, T, seed=13, period=period, tuning=tuning)
        rep = compare_stats(got, oracle_rows(a, b, dtype, T, 13, _positions(rows, None, period)), T,
                            f"low T {dtype} T={T} period={period} {tuning}")
        print(rep, flush=True)


def test_explicit_positions_and_period():
    print("case: explicit positions / period", flush=True)
    a, b = _peaked(40, 3001, 11, "bf16")
    pos = np.random.default_rng(3).integers(-2 ** 31, 2 ** 31 - 1, size=40).astype(np.int32)
    got = _run(a, b, "bf16", 1.0, seed=77, pos=pos)
    compare_stats(got, oracle_rows(a, b, "bf16", 1.0, 77, pos), 1.0, "explicit pos")
    for tuning in (None, {"shared_noise": 0}, {"shared_noise": 1}):
        got = _run(a, b, "bf16", 1.0, seed=77, period=8, tuning=tuning)
        compare_stats(got, oracle_rows(a, b, "bf16", 1.0, 77, _positions(40, None, 8)), 1.0, f"period 8 {tuning}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_row_padding_is_ignored(dtype):
    print(f"case: padded rows {dtype}", flush=True)
    V = 1001
    ld = 1008 if dtype == "bf16" else 1004
    a, b = _peaked(6, V, 5, dtype)
    pad = 0x7FC0 if dtype == "bf16" else 0x7FC00000   # NaN bit patterns in the padding
    for T in (0.0, 1.0):
        got = _run(a, b, dtype, T, seed=3, ld=ld, pad_bits=pad)
        compare_stats(got, oracle_rows(a, b, dtype, T, 3, _positions(6)), T, f"padding {dtype} T={T}")


def test_geometry_invariance_and_determinism():
    print("case: geometry invariance", flush=True)
    rows, V = 96, 20000
    a, b = _peaked(rows, V, 21, "bf16")
    ref = oracle_rows(a, b, "bf16", 1.0, 9, _positions(rows, None, 8))
    base = None
    for tuning in ({"split": 1, "shared_noise": 0}, {"split": 2, "shared_noise": 0}, {"split": 5, "shared_noise": 0},
                   {"split": 16, "shared_noise": 0}, {"split": 1, "shared_noise": 1}, {"split": 3, "shared_noise": 1},
                   {"split": 8, "shared_noise": 1}, {"split": 4, "shared_noise": 1}, None):
        got = _run(a, b, "bf16", 1.0, seed=9, period=8, tuning=tuning)
        compare_stats(got, ref, 1.0, str(tuning))
        if base is None:
            base = got
        for k in ("argmax_v", "argmax_d", "tok_v", "tok_d"):
            np.testing.assert_array_equal(got[k], base[k], err_msg=f"{k} {tuning}")
    again = _run(a, b, "bf16", 1.0, seed=9, period=8)
    again2 = _run(a, b, "bf16", 1.0, seed=9, period=8)
    for k in again:
        np.testing.assert_array_equal(again[k], again2[k], err_msg=f"determinism {k}")


def test_special_rows():
    print("case: special rows", flush=True)
    V = 4000
    rows = []
    rows.append((np.full(V, 1.5, np.float32), np.full(V, 1.5, np.float32)))              # uniform, identical
    x = np.random.default_rng(1).standard_normal(V).astype(np.float32)
    rows.append((x, x.copy()))                                                           # identical
    y = np.zeros(V, np.float32); y[[5, 77, 3999]] = 9.0                                  # exact ties
    rows.append((y, y[::-1].copy()))
    z = np.full(V, -1e6, np.float32); z[123] = 1e6                                       # huge magnitudes
    rows.append((z, np.roll(z, 5)))
    w = np.linspace(-50, 50, V).astype(np.float32)                                       # wide range
    rows.append((w, -w))
    s = np.zeros(V, np.float32); s[17] = 200.0                                           # conf == 1
    rows.append((s, s + 0.25))
    a = np.stack([r[0] for r in rows]); b = np.stack([r[1] for r in rows])
    for dtype in ("fp32", "bf16"):
        aa, bb = (a, b) if dtype == "fp32" else (W.round_bf16_bits(a), W.round_bf16_bits(b))
        for T in (0.0, 1.0, 3.0):
            got = _run(aa, bb, dtype, T, seed=1)
            ref = oracle_rows(aa, bb, dtype, T, 1, _positions(len(rows)))
            compare_stats(got, ref, T, f"special {dtype} T={T}")
            assert got["kl"][0] == 0.0 and got["kl"][1] == 0.0       # same logits: KL exactly 0
            assert got["argmax_v"][2] == 5 and got["argmax_d"][2] == 0
            assert got["conf"][5] >= np.float32(1.0) - np.float32(2.0 ** -24) * 2
            np.testing.assert_array_equal(got["tok_v"][:2], got["tok_d"][:2])  # identical logits, shared noise


def test_empty_batch():
    print("case: empty batch", flush=True)
    dev = _dev()
    a = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    got = dv.dv_verify_rows(a, a, temperature=1.0)
    torch.cuda.synchronize()
    assert all(v.numel() == 0 for k, v in got.items() if not k.startswith("_") and v is not None)


# --------------------------------------------------------- full-size workloads ----

def _sample_rows(rows, n, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(rows, size=min(n, rows), replace=False).tolist())
    pick |= {0, rows - 1}
    return np.array(sorted(pick))


def _bf16_rows_to_numpy(t, rows):
    return t[torch.as_tensor(rows, device=t.device)].view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("num", [2, 3])
def test_workload_single_sequence_full_size(num):
    w = W.workload(num)
    print(f"case: workload {num} ({w.name}) full size", flush=True)
    dev = _dev()
    a_np, b_np = W.make_logits_numpy(w)
    a = torch.from_numpy(a_np.view(np.int16)).to(dev).view(torch.bfloat16)
    b = torch.from_numpy(b_np.view(np.int16)).to(dev).view(torch.bfloat16)
    got = to_numpy(dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed))
    torch.cuda.synchronize()
    rows = _sample_rows(w.rows, 40, num)
    ref = oracle_rows(a_np[rows], b_np[rows], "bf16", w.temperature, w.seed, W.positions(w)[rows])
    rep = compare_stats({k: v[rows] for k, v in got.items()}, ref, w.temperature, w.name)
    print(rep, flush=True)


def test_workload_spot_tree_full_size():
    w = W.workload(4)
    print(f"case: workload 4 ({w.name}) full size", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    got = to_numpy(dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period))
    torch.cuda.synchronize()
    # three whole candidates and scattered rows
    rows = np.unique(np.concatenate([np.arange(0, 32), np.arange(32 * 31, 32 * 32), np.arange(32 * 63, 32 * 64),
                                     _sample_rows(w.rows, 24, 4)]))
    ref = oracle_rows(_bf16_rows_to_numpy(a, rows), _bf16_rows_to_numpy(b, rows), "bf16", w.temperature, w.seed,
                      W.positions(w)[rows])
    rep = compare_stats({k: v[rows] for k, v in got.items()}, ref, w.temperature, w.name)
    print(rep, flush=True)
    # shared and per-row noise paths agree on every row
    alt = to_numpy(dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period,
                                     tuning={"shared_noise": 0}))
    for k in ("argmax_v", "argmax_d", "tok_v", "tok_d"):
        np.testing.assert_array_equal(alt[k], got[k], err_msg=k)


def test_workload_throughput_full_size():
    w = W.workload(5)
    print(f"case: workload 5 ({w.name}) full size", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    got = to_numpy(dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed))
    torch.cuda.synchronize()
    rows = _sample_rows(w.rows, 48, 5)
    ref = oracle_rows(_bf16_rows_to_numpy(a, rows), _bf16_rows_to_numpy(b, rows), "bf16", w.temperature, w.seed,
                      W.positions(w)[rows])
    rep = compare_stats({k: v[rows] for k, v in got.items()}, ref, w.temperature, w.name)
    print(rep, flush=True)
    del a, b
    torch.cuda.empty_cache()


# ------------------------------------------- extended pass: -inf, reverse KL ----

ALL_OUT = dv.STAT_FIELDS


def _run_ext(a_np, b_np, dtype, T, seed=0, period=0, neg_inf=False, tuning=None):
    dev = _dev()
    a = _upload(a_np, dtype, dev)
    b = _upload(b_np, dtype, dev)
    got = dv.dv_verify_rows(a, b, temperature=T, seed=seed, pos_period=period, outputs=ALL_OUT, neg_inf=neg_inf,
                            tuning=tuning)
    torch.cuda.synchronize()
    return to_numpy(got)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extended_outputs_and_core_unchanged(dtype):
    """kl_rev and p_tok_d against the oracle; the extended pass leaves every core output bit for bit the same."""
    print(f"case: extended outputs {dtype}", flush=True)
    for rows, V, T, period in ((9, 1003, 1.0, 0), (40, 20000, 1.0, 4), (33, 5000, 0.0, 0), (64, 4096, 0.7, 8)):
        a, b = _peaked(rows, V, rows + V, dtype)
        ext = _run_ext(a, b, dtype, T, seed=3, period=period)
        base = _run(a, b, dtype, T, seed=3, period=period)
        for k in dv.CORE_FIELDS:
            np.testing.assert_array_equal(ext[k], base[k], err_msg=f"{k} differs in the extended pass")
        ref = oracle_rows(a, b, dtype, T, 3, _positions(rows, None, period))
        compare_stats(ext, ref, T, f"extended {dtype} {rows}x{V} T={T}")
        for split in (1, 3, 16):
            got = _run_ext(a, b, dtype, T, seed=3, period=period, tuning={"split": split})
            compare_stats(got, ref, T, f"extended {dtype} split={split}")


LIM = np.float32(-2.0 ** 100)


def _below_as_neg_inf(x, dtype):
    """Values at or below -2^100 count as -inf (the documented meaning of the flag)."""
    if dtype == "fp32":
        return np.where(x <= LIM, np.float32(-np.inf), x).astype(np.float32)
    vals = (x.astype(np.uint32) << 16).view(np.float32)
    return np.where(vals <= LIM, np.uint16(0xFF80), x).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_neg_inf_logits(dtype):
    """-inf entries (masked vocabulary) in one or both models, against the oracle's -inf conventions."""
    print(f"case: -inf logits {dtype}", flush=True)
    rng = np.random.default_rng(31)
    rows, V = 24, 3001
    a = (rng.standard_normal((rows, V)) * 2).astype(np.float32)
    b = (a + rng.standard_normal((rows, V)) * 0.5).astype(np.float32)
    shared = rng.random((rows, V)) < 0.3
    a[shared] = -np.inf
    b[shared] = -np.inf
    # rows 0-3: extra -inf in the drafter only (KL(p_v || p_d) = +inf); rows 4-7: in the verifier only
    only_d = (rng.random((rows, V)) < 0.2) & ~shared
    b[:4][only_d[:4]] = -np.inf
    a[4:8][only_d[4:8]] = -np.inf
    a[8, :] = -np.inf; a[8, 17] = 3.0                              # one finite logit left
    a[9, :] = -np.inf; a[9, V - 1] = 1.5                           # only the last element, in the tail chunk
    b[9, :] = -np.inf; b[9, V - 1] = -2.0
    a[10, :] = -1e35                                               # below -2^100: the same as -inf but one
    a[10, 5] = 0.0
    a[11, :] = -np.inf                                             # -2^100 itself, and -inf, in a row
    a[11, ::3] = -2.0 ** 100
    a[11, 7] = -4.0
    if dtype == "bf16":
        aa, bb = W.round_bf16_bits(a), W.round_bf16_bits(b)
    else:
        aa, bb = a, b
    for T, period in ((0.0, 0), (1.0, 0), (1.0, 4)):
        got = _run_ext(aa, bb, dtype, T, seed=8, period=period, neg_inf=True)
        ref = oracle_rows(_below_as_neg_inf(aa, dtype), _below_as_neg_inf(bb, dtype), dtype, T, 8,
                          _positions(rows, None, period), neg_inf=True)
        compare_stats(got, ref, T, f"-inf {dtype} T={T} period={period}")
        assert np.isinf(got["kl"][:4]).all() and np.isfinite(got["kl"][4:8]).all()
        assert np.isinf(got["kl_rev"][4:8]).all() and np.isfinite(got["kl_rev"][:4]).all()
        assert got["argmax_v"][8] == 17 and got["argmax_v"][9] == V - 1 and got["tok_d"][9] == V - 1
        assert got["conf"][8] == 1.0


def test_extended_workload_spot_tree_full_size():
    """The extended pass as `bench.py --extended` launches it (all eleven outputs, -inf allowed) at workload 4's
    full size, with masked vocabulary entries (-inf) written into some rows of both models, on sampled rows."""
    w = W.workload(4)
    print(f"case: workload 4 ({w.name}) full size, extended pass with -inf entries", flush=True)
    dev = _dev()
    a, b = W.make_logits_torch(w, dev)
    rng = np.random.default_rng(41)
    masked = _sample_rows(w.rows, 16, 7)
    for r in masked:                                  # a block of masked entries and scattered ones
        cols_a = np.concatenate([np.arange(1000, 1000 + 4096), rng.choice(w.V, 64, replace=False)])
        cols_b = rng.choice(w.V, 128, replace=False)
        a[int(r), torch.as_tensor(cols_a, device=dev)] = float("-inf")
        b[int(r), torch.as_tensor(cols_b, device=dev)] = float("-inf")
    got = to_numpy(dv.dv_verify_rows(a, b, temperature=w.temperature, seed=w.seed, pos_period=w.pos_period,
                                     outputs=ALL_OUT, neg_inf=True))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([masked, np.arange(32 * 7, 32 * 8), _sample_rows(w.rows, 24, 8)]))
    ref = oracle_rows(_bf16_rows_to_numpy(a, rows), _bf16_rows_to_numpy(b, rows), "bf16", w.temperature, w.seed,
                      W.positions(w)[rows], neg_inf=True)
    rep = compare_stats({k: v[rows] for k, v in got.items()}, ref, w.temperature, w.name + " extended")
    print(rep, flush=True)
    del a, b
    torch.cuda.empty_cache()
