"""Shared Gumbel noise and the Gumbel-max tokens of both models (float64).

Test infrastructure: see the package docstring for who may import this.

[SPOT] §1 "Key terms", coupled-noise verification, and §3 "Method": at a
sampling temperature T > 0 the drafter and the target draw with the same
Gumbel noise, so that given the noise the target's transition is a
deterministic function of its logits and the target's distribution is kept.
The Gumbel-max construction draws token argmax_i (x_i / T + g_i) with
g_i i.i.d. standard Gumbel; it samples softmax(x / T) exactly.

The pages do not say where the noise comes from. The reading used here is a
counter-based generator keyed on (seed, position, vocabulary index), called
DV_HASH_V1 below, so that the noise a position sees does not depend on which
row, candidate or shard carries it:

* ``mix32`` is the 32-bit finalizer of Austin Appleby's MurmurHash3
  (public domain): x ^= x>>16; x *= 0x85EBCA6B; x ^= x>>13; x *= 0xC2B2AE35;
  x ^= x>>16, all mod 2^32.
* seed words: A = mix32(seed_hi ^ 0x243F6A88), B = mix32(A ^ seed_lo), where
  seed_hi / seed_lo are the upper / lower 32 bits of the 64-bit seed.
* row key: k = mix32(B ^ mix32(pos ^ 0x85A308D3)), pos taken as the 32-bit
  two's-complement pattern of the int32 position.
* word for vocabulary index i: h_i = mix32(k ^ (i * 0x9E3779B9 mod 2^32)).
* uniform: u_i = (2 * (h_i >> 9) + 1) * 2^-24, i.e. 23 random bits placed at
  the centres of 2^23 equal cells of (0, 1); never 0 or 1.

The Gumbel values (DV_NOISE_V2) come in groups of 8 consecutive vocabulary
indices, group c holding indices 8c .. 8c+7. Any set of n i.i.d. standard
Gumbel values can be drawn largest first: their maximum is Gumbel shifted by
ln n (its CDF is F(x)^n with F(x) = exp(-e^-x)), it sits at a uniformly
chosen place, and given it the other n - 1 are i.i.d. Gumbel truncated above
at it (CDF F(x)/F(max)). The joint law is exactly that of n independent
draws, so Gumbel-max sampling is unchanged; what it buys is that a group's
largest noise value comes from one hash word. Per row:

* group key: kg = mix32(k ^ 0x6A09E667);
* group word: w_c = mix32(kg ^ (c * 0x9E3779B9 mod 2^32));
* for a full group (8c + 8 <= vocab): the maximum sits at j* = w_c & 7 and
  is g_max = -ln(-ln(u_max) / 8) with u_max = (2 * (w_c >> 9) + 1) * 2^-24;
  index i = 8c + j with j != j* gets g_i = -ln(-(ln u_i + ln(u_max) / 8)),
  the inverse of the truncated CDF at u_i;
* the last group when it is partial (vocab not a multiple of 8): each index
  gets g_i = -ln(-ln u_i), independent draws.

Temperature T = 0 means greedy decoding: the token is the argmax of the
logits (lowest index on ties) and no noise is drawn. Ties of the perturbed
score also go to the lowest index.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "MIX_C1", "MIX_C2", "SEED_SALT", "POS_SALT", "INDEX_STEP", "GROUP_SALT", "GROUP",
    "mix32", "seed_words", "row_keys", "hash_words", "group_words", "uniforms", "gumbel",
    "noise", "perturbed_scores", "gumbel_tokens",
]

MIX_C1 = 0x85EBCA6B
MIX_C2 = 0xC2B2AE35
SEED_SALT = 0x243F6A88
POS_SALT = 0x85A308D3
INDEX_STEP = 0x9E3779B9
GROUP_SALT = 0x6A09E667
GROUP = 8  # vocabulary indices per noise group
_M32 = np.uint64(0xFFFFFFFF)


def mix32(x) -> np.ndarray:
    """MurmurHash3 fmix32 on uint32 values (array in, uint32 array out)."""
    x = np.asarray(x, dtype=np.uint64) & _M32
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(MIX_C1)) & _M32
    x ^= x >> np.uint64(13)
    x = (x * np.uint64(MIX_C2)) & _M32
    x ^= x >> np.uint64(16)
    return x.astype(np.uint32)


def seed_words(seed: int) -> tuple[int, int]:
    """(A, B) derived from the 64-bit seed."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    hi, lo = seed >> 32, seed & 0xFFFFFFFF
    a = int(mix32(hi ^ SEED_SALT))
    b = int(mix32(a ^ lo))
    return a, b


def row_keys(seed: int, pos) -> np.ndarray:
    """Per-row key k for int32 positions ``pos``."""
    _, b = seed_words(seed)
    p = np.asarray(pos, dtype=np.int64).astype(np.int32).view(np.uint32)
    return mix32(np.uint32(b) ^ mix32(p ^ np.uint32(POS_SALT)))


def hash_words(seed: int, pos, vocab: int, start: int = 0) -> np.ndarray:
    """uint32 words h[r, i] for vocabulary indices start .. start+vocab-1."""
    k = row_keys(seed, pos)
    i = np.arange(start, start + vocab, dtype=np.uint64)
    step = (i * np.uint64(INDEX_STEP)) & _M32
    return mix32(k.astype(np.uint64)[:, None] ^ step[None, :])


def group_words(seed: int, pos, ngroups: int) -> np.ndarray:
    """uint32 group words w[r, c] for groups 0 .. ngroups-1."""
    kg = mix32(row_keys(seed, pos) ^ np.uint32(GROUP_SALT))
    c = np.arange(ngroups, dtype=np.uint64)
    step = (c * np.uint64(INDEX_STEP)) & _M32
    return mix32(kg.astype(np.uint64)[:, None] ^ step[None, :])


def uniforms(h: np.ndarray) -> np.ndarray:
    """u = (2 * (h >> 9) + 1) * 2^-24 as float64 (exact)."""
    h = np.asarray(h, dtype=np.uint32)
    return ((h >> np.uint32(9)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -24


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel variate from a uniform: g = -ln(-ln u)."""
    return -np.log(-np.log(np.asarray(u, dtype=np.float64)))


def noise(seed: int, pos, vocab: int) -> np.ndarray:
    """The Gumbel values g[r, i] of rows at positions ``pos`` over a vocabulary of ``vocab``
    (DV_NOISE_V2, module docstring), float64."""
    pos = np.asarray(pos)
    u = uniforms(hash_words(seed, pos, vocab))
    g = gumbel(u)
    nfull = vocab // GROUP
    if nfull:
        w = group_words(seed, pos, nfull)
        umax = uniforms(w)
        lm = np.log(umax)[:, :, None] / GROUP                       # ln F(g_max)
        lu = np.log(u[:, :GROUP * nfull]).reshape(len(pos), nfull, GROUP)
        gf = -np.log(-(lu + lm))                                    # truncated below the maximum
        jstar = (w & np.uint32(GROUP - 1)).astype(np.int64)
        gmax = -np.log(-np.log(umax) / GROUP)
        np.put_along_axis(gf, jstar[:, :, None], gmax[:, :, None], axis=2)
        g[:, :GROUP * nfull] = gf.reshape(len(pos), GROUP * nfull)
    return g


def perturbed_scores(x: np.ndarray, temperature: float, g: np.ndarray) -> np.ndarray:
    """x / T + g, the score whose argmax is the Gumbel-max sample at T > 0."""
    return np.asarray(x, dtype=np.float64) / float(temperature) + g


def _argmax_and_margin(s: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Lowest-index argmax of each row and the gap between its two largest values."""
    tok = np.argmax(s, axis=1).astype(np.int32)
    if s.shape[1] == 1:
        return tok, np.full(s.shape[0], np.inf)
    top2 = -np.partition(-s, 1, axis=1)[:, :2]
    return tok, top2[:, 0] - top2[:, 1]


def gumbel_tokens(a: np.ndarray, b: np.ndarray, temperature: float, seed: int, pos) -> dict:
    """Tokens of both models under the same noise.

    ``a``, ``b``: float64 [R, V]; ``pos``: int positions [R]. Returns tok_v,
    tok_d (int32) and margin_v, margin_d: the gap between the best and the
    second-best score of each row (raw logits when T = 0, x/T + g when T > 0),
    which the parity tests use to tell near-ties apart.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    t = float(temperature)
    if not np.isfinite(t) or t < 0:
        raise ValueError("temperature must be finite and >= 0")
    if a.shape[0] == 0:
        z = np.zeros(0, np.int32)
        return dict(tok_v=z, tok_d=z.copy(), margin_v=np.zeros(0), margin_d=np.zeros(0))
    if t == 0.0:
        sa, sb = a, b
    else:
        g = noise(seed, pos, a.shape[1])
        sa = perturbed_scores(a, t, g)
        sb = perturbed_scores(b, t, g)
    tok_v, margin_v = _argmax_and_margin(sa)
    tok_d, margin_d = _argmax_and_margin(sb)
    return dict(tok_v=tok_v, tok_d=tok_d, margin_v=margin_v, margin_d=margin_d)
