"""Shared helpers of the GPU parity tests: run the oracle on the exact bytes the
GPU read and compare, with the tolerances and near-tie bands below.

Floats (lse_v, lse_d, kl, entropy, conf, scores): |gpu - oracle| <= ATOL + RTOL |oracle|.
Integers: bit-exact, except decisions that sit within BAND of a threshold and
Gumbel-max tokens whose oracle top-2 margin is within BAND; those are counted
and reported, not failed.
"""

from __future__ import annotations

import numpy as np

from oracle import noise as onoise
from oracle import rowstats

RTOL = 1e-4
ATOL = 1e-5
BAND = 1e-5
FLOAT_STATS = ("lse_v", "lse_d", "kl", "entropy", "conf", "kl_rev")


def oracle_rows(a, b, dtype: str, temperature: float, seed: int, pos, neg_inf: bool = False) -> dict:
    """Oracle statistics, tokens and token margins of rows stored as ``dtype``
    (with kl_rev and p_tok_d, the verifier's probability of the drafter's token)."""
    a64 = rowstats.as_float64(a, dtype)
    b64 = rowstats.as_float64(b, dtype)
    st = rowstats.row_stats(a64, b64, neg_inf=neg_inf)
    st.update(onoise.gumbel_tokens(a64, b64, temperature, seed, np.asarray(pos)))
    st["kl_rev"] = rowstats.kl_reverse(a64, b64, neg_inf=neg_inf)
    st["p_tok_d"] = rowstats.prob_of(a64, st["tok_d"]) if len(a64) else np.zeros(0)
    return st


def to_numpy(gpu: dict, rows=None) -> dict:
    out = {}
    for k, v in gpu.items():
        if k.startswith("_") or v is None:
            continue
        x = v.detach().cpu().numpy()
        out[k] = x if rows is None else x[rows]
    return out


def compare_stats(got: dict, ref: dict, temperature: float, ctx: str = "") -> dict:
    """Assert parity of one batch of rows; returns the report (max errors, in-band counts)."""
    rep = {"rows": int(len(ref["lse_v"]))}
    for k in FLOAT_STATS:
        if k not in got:
            continue
        g = got[k].astype(np.float64)
        r = np.asarray(ref[k], np.float64)
        same_inf = np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r))   # e.g. KL = +inf on both sides
        err = np.where(same_inf, 0.0, np.abs(g - r))
        bad = ~(err <= ATOL + RTOL * np.where(same_inf, 0.0, np.abs(r)))     # a NaN on either side fails
        rep[f"max_abs_err_{k}"] = float(err.max()) if err.size else 0.0
        assert not bad.any(), f"{ctx} {k}: rows {np.nonzero(bad)[0][:10]} gpu {g[bad][:5]} oracle {r[bad][:5]}"
    for k in ("argmax_v", "argmax_d"):
        if k in got:
            bad = got[k] != ref[k]
            assert not bad.any(), f"{ctx} {k}: rows {np.nonzero(bad)[0][:10]} gpu {got[k][bad][:5]} oracle {ref[k][bad][:5]}"
    if "p_tok_d" in got and "tok_d" in got:
        # the probability of the drafter's token, where both sides picked the same token
        same = got["tok_d"] == ref["tok_d"]
        g, r = got["p_tok_d"].astype(np.float64)[same], np.asarray(ref["p_tok_d"], np.float64)[same]
        bad = ~(np.abs(g - r) <= ATOL + RTOL * np.abs(r))
        assert not bad.any(), f"{ctx} p_tok_d: gpu {g[bad][:5]} oracle {r[bad][:5]}"
    for k, mk in (("tok_v", "margin_v"), ("tok_d", "margin_d")):
        if k not in got:
            continue
        diff = got[k] != ref[k]
        if temperature == 0.0:
            assert not diff.any(), f"{ctx} {k} (greedy): rows {np.nonzero(diff)[0][:10]}"
            continue
        inband = ref[mk] <= BAND
        bad = diff & ~inband
        rep[f"{k}_in_band"] = int(inband.sum())
        rep[f"{k}_in_band_mismatch"] = int((diff & inband).sum())
        assert not bad.any(), (f"{ctx} {k}: rows {np.nonzero(bad)[0][:10]} gpu {got[k][bad][:5]} "
                               f"oracle {ref[k][bad][:5]} margin {ref[mk][bad][:5]}")
    return rep


def decisions_in_band(rule: int, kl, conf, tau: float, theta: float) -> np.ndarray:
    """Rows whose decision depends on a statistic within BAND of its threshold."""
    n = len(kl) if kl is not None else len(conf)
    m = np.zeros(n, bool)
    if kl is not None and rule in (1, 3):
        m |= np.abs(np.asarray(kl, np.float64) - tau) <= BAND
    if conf is not None and rule in (2, 3, 4):
        m |= np.abs(np.asarray(conf, np.float64) - theta) <= BAND
    return m
