"""Shared helpers of the GPU parity tests: run the oracle on the exact bytes the
GPU read and compare, with the tolerances and near-tie bands below.

Floats (lse_v, lse_d, kl, entropy, conf, scores): |gpu - oracle| <= ATOL + RTOL |oracle|.
Integers: bit-exact, except decisions that sit within BAND of a threshold and
Gumbel-max tokens whose oracle top-2 margin is within their band; those are
counted and reported, not failed.

The band of a T > 0 token is BAND, or the rounding bound of the kernel's
float32 score when that is larger (token_band): the kernel forms
s = fma(x, log2(e)/T, G) in float32 with G from the hardware log2 (1 ulp), so
the difference of two scores is off by at most
2^-23 (|s_top| + |x_top| / T) + 4.6e-6 nats, with |s_top| <= max|x| / T + 16.64
(the largest Gumbel value the uniforms allow) and |x_top| <= max|x|. At the
workloads' T = 1 and |x| <= 15 this is about 1e-5; it grows as T shrinks.
"""

from __future__ import annotations

import json
import os

import numpy as np

from oracle import noise as onoise
from oracle import rowstats

RTOL = 1e-4
ATOL = 1e-5
BAND = 1e-5
FLOAT_STATS = ("lse_v", "lse_d", "kl", "entropy", "conf", "kl_rev")


def token_band(absmax, temperature: float) -> np.ndarray:
    """Per-row margin band of T > 0 tokens: BAND, or the float32 score's rounding bound when larger."""
    absmax = np.asarray(absmax, np.float64)
    if temperature <= 0.0:
        return np.full(absmax.shape, BAND)
    xs = absmax / temperature
    return np.maximum(BAND, 2.0 ** -23 * (2.0 * xs + 16.64) + 4.6e-6)


def _absmax(a64, b64) -> np.ndarray:
    """max |x| over the finite logits of both models, per row."""
    if a64.shape[0] == 0:
        return np.zeros(0)
    fa = np.where(np.isfinite(a64), np.abs(a64), 0.0).max(axis=1)
    fb = np.where(np.isfinite(b64), np.abs(b64), 0.0).max(axis=1)
    return np.maximum(fa, fb)


def oracle_rows(a, b, dtype: str, temperature: float, seed: int, pos, neg_inf: bool = False) -> dict:
    """Oracle statistics, tokens and token margins of rows stored as ``dtype``
    (with kl_rev and p_tok_d, the verifier's probability of the drafter's token)."""
    a64 = rowstats.as_float64(a, dtype)
    b64 = rowstats.as_float64(b, dtype)
    st = rowstats.row_stats(a64, b64, neg_inf=neg_inf)
    st.update(onoise.gumbel_tokens(a64, b64, temperature, seed, np.asarray(pos)))
    st["absmax"] = _absmax(a64, b64)
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
        with np.errstate(invalid="ignore"):                                  # inf - inf where both are inf
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
        band = token_band(ref["absmax"], temperature) if "absmax" in ref else BAND
        inband = ref[mk] <= band
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


# ---------------------------------------------------- whole-population parity ----

CORE_KEYS = ("lse_v", "lse_d", "kl", "entropy", "conf", "argmax_v", "argmax_d", "tok_v", "tok_d",
             "margin_v", "margin_d", "absmax")


def oracle_block(args) -> dict:
    """Oracle statistics and shared-noise tokens (with margins) of one block of rows (a worker-process task)."""
    a, b, dtype, temperature, seed, pos = args
    a64 = rowstats.as_float64(a, dtype)
    b64 = rowstats.as_float64(b, dtype)
    st = rowstats.row_stats(a64, b64)
    st.update(onoise.gumbel_tokens(a64, b64, temperature, seed, np.asarray(pos)))
    st["absmax"] = _absmax(a64, b64)
    return {k: st[k] for k in CORE_KEYS}


def oracle_workers() -> int:
    """Worker processes for the host-side oracle: the host's cores, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class OraclePool:
    """Runs oracle_block over blocks of rows in spawned worker processes (numpy only, no GPU state)."""

    def __init__(self, workers: int | None = None, block: int = 64):
        import multiprocessing as mp

        self.workers = workers or oracle_workers()
        self.block = block
        self._pool = mp.get_context("spawn").Pool(self.workers)

    def rows(self, a, b, dtype: str, temperature: float, seed: int, pos) -> dict:
        """Oracle results of every row of a, b (uint16 bf16 bits or float32 values), in row order."""
        n = a.shape[0]
        tasks = [(a[s:s + self.block], b[s:s + self.block], dtype, temperature, seed, np.asarray(pos)[s:s + self.block])
                 for s in range(0, n, self.block)]
        parts = self._pool.map(oracle_block, tasks)
        if not parts:
            return {k: np.zeros(0) for k in CORE_KEYS}
        return {k: np.concatenate([p[k] for p in parts]) for k in CORE_KEYS}

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def report(name: str, rep: dict):
    """Print one parity record, and append it to the JSON-lines file named by DV_PARITY_REPORT when set."""
    line = json.dumps({"case": name, **rep}, sort_keys=True)
    print("PARITY", line, flush=True)
    path = os.environ.get("DV_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
