"""COVER's seed score and the per-sequence top-k / threshold selection (oracle).

Test infrastructure: see the package docstring for who may import this.

[COVER] §2 "Stability-aware seed selection": each committed position gets the
score u * (1 + d_in) / (1 + d_out), where u is the uncertainty (entropy of
the current token assignment), d_in how much the still-masked positions rely
on the token, and d_out how strongly the token attends to newly written
positions; a small set of the highest-scoring positions becomes the seeds.
The page gives no formula for d_in / d_out, so they are inputs here, and no
rule for the size of the "small, adaptive" set, so the size is a fixed k.

[SPOT] §3 "Method" names a dynamic-threshold decoding mode (SPOT-Sets with the
threshold decoder, Table 2) whose schedule the review does not give; the
selection therefore takes an optional fixed threshold.

Readings:

* Ineligible positions score -inf.
* top-k over eligible positions of one sequence, largest (or smallest)
  scores first; equal scores go to the lower index; the result is sorted.
* with a threshold, only selected entries with score > thr (largest mode) or
  score < thr (smallest mode) are kept; they form a prefix of the sorted list.
* outputs past ``count`` are padded with index -1 and value NaN.
"""

from __future__ import annotations

import numpy as np

__all__ = ["seed_score", "select_topk"]


def seed_score(u, d_in, d_out, eligible=None) -> np.ndarray:
    """u * (1 + d_in) / (1 + d_out) per position; -inf where not eligible."""
    u = np.asarray(u, dtype=np.float64)
    d_in = np.asarray(d_in, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    s = u * (1.0 + d_in) / (1.0 + d_out)
    if eligible is not None:
        s = np.where(np.asarray(eligible) != 0, s, -np.inf)
    return s


def select_topk(score, k: int, *, eligible=None, largest: bool = True,
                use_thr: bool = False, thr: float = 0.0):
    """Per-sequence top-k of ``score`` [nseq, L].

    Returns (idx int32 [nseq, k], val float64 [nseq, k], count int32 [nseq]).
    """
    score = np.asarray(score, dtype=np.float64)
    if score.ndim != 2:
        raise ValueError("score must be [nseq, L]")
    nseq, L = score.shape
    if not 1 <= k <= L:
        raise ValueError("need 1 <= k <= L")
    elig = np.ones_like(score, bool) if eligible is None else (np.asarray(eligible) != 0)
    idx = np.full((nseq, k), -1, np.int32)
    val = np.full((nseq, k), np.nan)
    cnt = np.zeros(nseq, np.int32)
    for s in range(nseq):
        cand = [(float(score[s, i]), i) for i in range(L) if elig[s, i]]
        if largest:
            cand.sort(key=lambda t: (-t[0], t[1]))
        else:
            cand.sort(key=lambda t: (t[0], t[1]))
        chosen = cand[:k]
        if use_thr:
            chosen = [c for c in chosen if (c[0] > thr if largest else c[0] < thr)]
        for j, (v, i) in enumerate(chosen):
            idx[s, j] = i
            val[s, j] = v
        cnt[s] = len(chosen)
    return idx, val, cnt
