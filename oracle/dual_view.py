"""COVER's dual-view attention with KV-cache override and diagonal correction (oracle).

Test infrastructure: see the package docstring for who may import this.

Source: [COVER] "Method: COVER", part 1 (Dual-View Feed Forward through KV cache
override). The summary says:
- Queries, keys and values are computed from the current input, in which the
  seed positions (tokens being re-checked) are replaced by [MASK].
- For every query, the key/value column of a seed position is overridden with
  the K and V cached at the previous step, so that other positions keep
  reading the seed's stable, unmasked context.
- A seed query's own diagonal column is restored to the K and V computed
  from the masked input, and the weights are renormalized. The seed is
  therefore verified leave-one-out, without seeing its own cached token.

Reading (the summary gives no formulas):
    k_eff(i, j) = K_prev[j] if seed[j] and j != i, else K_cur[j] (likewise v_eff)
    s_ij = scale * <q_i, k_eff(i, j)>
    o_i  = sum_j softmax_j(s_ij) * v_eff(i, j)
The attention is bidirectional: there is no causal mask in a diffusion
language model. Query head h reads key/value head h // (H / H_kv), as in
grouped-query attention.
"""

from __future__ import annotations

import numpy as np

__all__ = ["dual_view_attention"]


def dual_view_attention(q, k_cur, v_cur, k_prev, v_prev, seed, scale):
    """o [B, H, L, D] (float64) from q [B, H, L, D], k_*, v_* [B, Hkv, L, D],
    seed [B, L] (nonzero = seed position) and the score scale."""
    q = np.asarray(q, np.float64)
    k_cur, v_cur = np.asarray(k_cur, np.float64), np.asarray(v_cur, np.float64)
    k_prev, v_prev = np.asarray(k_prev, np.float64), np.asarray(v_prev, np.float64)
    B, H, L, D = q.shape
    Hkv = k_cur.shape[1]
    if H % Hkv or k_cur.shape != (B, Hkv, L, D) or k_prev.shape != k_cur.shape:
        raise ValueError("shapes: q [B, H, L, D], k/v [B, Hkv, L, D] with Hkv dividing H")
    sd = np.asarray(seed).reshape(B, L) != 0
    out = np.empty((B, H, L, D))
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            for i in range(L):
                use_prev = sd[b].copy()
                use_prev[i] = False          # the diagonal always reads the current input
                K = np.where(use_prev[:, None], k_prev[b, g], k_cur[b, g])
                V = np.where(use_prev[:, None], v_prev[b, g], v_cur[b, g])
                s = scale * (K @ q[b, h, i])
                w = np.exp(s - s.max())
                out[b, h, i] = (w / w.sum()) @ V
    return out
