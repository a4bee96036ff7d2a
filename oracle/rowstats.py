"""Per-row statistics of verifier and drafter logits, by definition (float64).

Test infrastructure: see the package docstring for who may import this.

Every row r holds two length-V logit vectors: the verifier's ``a`` and the
drafter's ``b``. The distributions are the softmaxes of the raw logits
(temperature only enters the sampled tokens, see ``noise``).

[DualDiffusion] §2 "Verification algorithms": the KL remasking rule compares
the drafter's and the verifier's predictive distributions through their KL
divergence (item 2) and the confidence rule uses the verifier's maximum
probability (item 3). [COVER] §2 "Stability-aware seed selection": the
uncertainty u is the entropy of the current token assignment, taken here as
the entropy of the verifier's distribution at that position.

Readings (the pages leave these open):

* KL direction: KL(p_verifier || p_drafter) = sum_i p_v,i (log p_v,i - log p_d,i).
* Entropy uses the natural logarithm (nats).
* Confidence is the verifier's maximum probability, max_i p_v,i.
* Argmax ties go to the lowest index.
* Logits must be finite; the oracle asserts this. With ``neg_inf=True`` a
  logit may also be -inf: a vocabulary entry masked out of the
  distribution (probability 0). Then 0 log 0 = 0, and a divergence is +inf
  when the first distribution puts mass where the second has none. Every row
  keeps at least one finite logit in each model.

Further quantities (cheap variants of the same pass):

* kl_reverse: KL(p_drafter || p_verifier), the other direction.
* prob_of: p_v of a given token, e.g. the verifier's probability of the
  drafted token (the other reading of "confidence for the token" in
  [DualDiffusion] §2 item 3).
"""

from __future__ import annotations

import numpy as np

__all__ = ["widen_bf16", "as_float64", "log_sum_exp", "log_softmax", "row_stats", "kl_reverse", "prob_of"]


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bfloat16 is the upper half of an IEEE binary32, so placing the 16 bits
    in the high half of a 32-bit word gives the same number exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Logits stored as ``dtype`` ("fp32" values or "bf16" bit patterns) -> float64."""
    if dtype == "bf16":
        return widen_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def log_sum_exp(x: np.ndarray) -> np.ndarray:
    """log sum_i exp(x_i) per row, shifted by the row max (two passes)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))[..., 0]


def log_softmax(x: np.ndarray) -> np.ndarray:
    """log p_i = x_i - log sum_j exp(x_j)."""
    x = np.asarray(x, dtype=np.float64)
    return x - log_sum_exp(x)[..., None]


def _check_logits(a, b, neg_inf):
    if a.ndim != 2 or a.shape != b.shape:
        raise ValueError("a and b must both have shape [R, V]")
    if a.shape[1] == 0:
        raise ValueError("V must be positive")
    if not neg_inf:
        if not (np.isfinite(a).all() and np.isfinite(b).all()):
            raise ValueError("logits must be finite")
        return
    for x in (a, b):
        if np.isnan(x).any() or (x == np.inf).any():
            raise ValueError("logits must be finite or -inf")
        if x.shape[0] and not np.isfinite(x).any(axis=1).all():
            raise ValueError("every row needs a finite logit")


def _kl(logp, logq):
    """sum_i p_i (log p_i - log q_i) per row with 0 log 0 = 0 and +inf where q = 0 < p."""
    p = np.exp(logp)
    has = p > 0
    if (has & np.isneginf(logq)).any(axis=None):
        out = np.where((has & np.isneginf(logq)).any(axis=1), np.inf, 0.0)
    else:
        out = np.zeros(logp.shape[0])
    terms = np.where(has & np.isfinite(logq), p * (np.where(has, logp, 0.0) - np.where(np.isfinite(logq), logq, 0.0)), 0.0)
    return np.where(np.isinf(out), out, terms.sum(axis=1))


def row_stats(a: np.ndarray, b: np.ndarray, neg_inf: bool = False) -> dict:
    """Statistics of each row of verifier logits ``a`` and drafter logits ``b``.

    ``a`` and ``b`` are float64 arrays of shape [R, V] (R may be 0). Returns a
    dict of arrays of length R:

    lse_v, lse_d  log-sum-exp of each model's logits
    kl            KL(p_v || p_d) in nats
    entropy       H(p_v) = -sum p_v log p_v in nats
    conf          max_i p_v,i
    argmax_v/_d   lowest index attaining each row's maximum logit
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    _check_logits(a, b, neg_inf)
    lse_v = log_sum_exp(a)
    lse_d = log_sum_exp(b)
    logp_v = a - lse_v[:, None]
    logp_d = b - lse_d[:, None]
    p_v = np.exp(logp_v)
    kl = _kl(logp_v, logp_d)
    entropy = -np.where(p_v > 0, p_v * np.where(p_v > 0, logp_v, 0.0), 0.0).sum(axis=1)
    conf = np.exp(a.max(axis=1) - lse_v)
    # numpy's argmax returns the first (lowest-index) maximum
    argmax_v = np.argmax(a, axis=1).astype(np.int32) if a.shape[0] else np.zeros(0, np.int32)
    argmax_d = np.argmax(b, axis=1).astype(np.int32) if a.shape[0] else np.zeros(0, np.int32)
    return dict(lse_v=lse_v, lse_d=lse_d, kl=kl, entropy=entropy, conf=conf,
                argmax_v=argmax_v, argmax_d=argmax_d)


def kl_reverse(a: np.ndarray, b: np.ndarray, neg_inf: bool = False) -> np.ndarray:
    """KL(p_drafter || p_verifier) per row, in nats (same conventions as row_stats)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    _check_logits(a, b, neg_inf)
    return _kl(log_softmax(b), log_softmax(a))


def prob_of(a: np.ndarray, tok: np.ndarray) -> np.ndarray:
    """p_v,tok[r] = exp(a[r, tok[r]] - lse(a[r])) per row."""
    a = np.asarray(a, dtype=np.float64)
    tok = np.asarray(tok, dtype=np.int64)
    return np.exp(a[np.arange(a.shape[0]), tok] - log_sum_exp(a))
