"""COVER's influence d_in and drift sensitivity d_out from attention probabilities (oracle).

Test infrastructure: see the package docstring for who may import this.

Source: [COVER] "Method: COVER", part 2 (Stability-Aware Seed Selection). The
seed score u·(1 + d_in)/(1 + d_out) weighs two quantities:
- a token's influence d_in: how much the positions that are still masked rely
  on it as context;
- its drift sensitivity d_out: how strongly the token itself attends to the
  positions written in the current draft.

The page gives no formula for either. Readings taken, with A[h, i, j] the
attention probability of query row i on key column j in head h (rows sum to
one):
    d_in[j]  = (1/H) * sum over h, and over masked queries i, of A[h, i, j]
    d_out[i] = (1/H) * sum over h, and over newly written columns k, of A[h, i, k]
That is: attention mass summed over the relevant rows (d_in) or columns
(d_out), then averaged over the heads given. How heads and layers are
combined is not stated, so all heads passed in are averaged with equal
weight. To average over layers too, pass the layers stacked as more heads.
"""

from __future__ import annotations

import numpy as np

__all__ = ["influence_drift"]


def influence_drift(probs, query_masked, new_cols):
    """d_in, d_out (float64 [B, L]) from probs [B, H, L, L] (any float dtype,
    widened exactly), query_masked [B, L] and new_cols [B, L] (nonzero = set)."""
    A = np.asarray(probs, dtype=np.float64)
    if A.ndim != 4 or A.shape[2] != A.shape[3]:
        raise ValueError("probs must be [B, H, L, L]")
    B, H, L, _ = A.shape
    qm = np.asarray(query_masked).reshape(B, L) != 0
    nc = np.asarray(new_cols).reshape(B, L) != 0
    d_in = np.zeros((B, L))
    d_out = np.zeros((B, L))
    for b in range(B):
        for h in range(H):
            d_in[b] += A[b, h][qm[b], :].sum(axis=0)
            d_out[b] += A[b, h][:, nc[b]].sum(axis=1)
    return d_in / H, d_out / H
