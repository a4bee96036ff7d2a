"""dv_verify_rows_noalloc (the entry point for callers that cannot allocate) against dv_verify_rows, the
entry point it is a variant of: the same kernels and launch shape, so every output must agree bit for bit.
Two calls in a row, the second smaller, so that the second reads the scratch the first left behind and must
overwrite what it uses; then a call without a table, and the size limit."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from parity_util import compare_stats, oracle_rows, to_numpy

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch.device("cuda:0")


def _logits(rows, V, seed, dev):
    rng = np.random.default_rng(seed)
    a, b = W.peaked_logits(rows, V, rng)
    a, b = W.round_bf16_bits(a), W.round_bf16_bits(b)
    t = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    return a, b, t(a), t(b)


def _outputs(rows, dev):
    return {f: torch.full((rows,), -7, dtype=torch.float32 if f in ("lse_v", "lse_d", "kl", "entropy", "conf")
                          else torch.int32, device=dev) for f in dv.CORE_FIELDS}


def _same(got, ref, ctx):
    for k in dv.CORE_FIELDS:
        g, r = got[k].cpu().numpy(), ref[k].cpu().numpy()
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{ctx}: {k} differs"


def test_noalloc_matches_verify_rows():
    dev = _dev()
    # (candidates x positions, vocab, T, tuning): a table of 32 x 18992 chunks (2.4 MB), then a smaller one
    # of 16 x 6250 chunks, then greedy (no table), then the per-row bound (no table)
    cases = [(8, 32, 151936, 1.0, None), (4, 16, 50000, 0.7, None), (2, 16, 50000, 0.0, None),
             (4, 16, 50000, 1.0, {"shared_noise": 0})]
    for n, period, V, T, tuning in cases:
        rows = n * period
        print(f"case: noalloc {rows} rows ({n} x {period}), V={V}, T={T}, tuning={tuning}", flush=True)
        a_np, b_np, a, b = _logits(rows, V, rows + V, dev)
        out = _outputs(rows, dev)
        got = dv.dv_verify_rows_noalloc(a, b, temperature=T, seed=11, pos_period=period, out=out, tuning=tuning)
        ref = dv.dv_verify_rows(a, b, temperature=T, seed=11, pos_period=period, tuning=tuning)
        torch.cuda.synchronize()
        _same(got, ref, f"{rows}x{V} T={T}")
        # and the oracle's bar on a few rows (positions repeat with the period)
        pick = np.array([0, 1, period - 1, rows - 1])
        pos = (np.arange(rows) % period).astype(np.int32)
        compare_stats(to_numpy(got, pick), oracle_rows(a_np[pick], b_np[pick], "bf16", T, 11, pos[pick]), T,
                      f"noalloc {rows}x{V}")


def test_noalloc_rejects_tables_beyond_its_scratch():
    dev = _dev()
    print("case: noalloc size limit", flush=True)
    a = torch.zeros((256, 152064), dtype=torch.bfloat16, device=dev)
    with pytest.raises(dv.DVError) as e:
        dv.dv_verify_rows_noalloc(a, a, temperature=1.0, pos_period=128)
    assert e.value.status == 7 and "scratch" in str(e.value)
    # without the table the same call runs
    got = dv.dv_verify_rows_noalloc(a[:4], a[:4], temperature=1.0, pos_period=128, tuning={"shared_noise": 0})
    torch.cuda.synchronize()
    assert (got["argmax_v"].cpu().numpy() == 0).all()
