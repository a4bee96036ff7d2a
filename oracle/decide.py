"""Per-position decision rules and the accepted prefix per candidate (oracle).

Test infrastructure: see the package docstring for who may import this.

Decision codes: 0 NONE (row not decided), 1 KEEP, 2 REPLACE, 3 REMASK.
Rule codes: 0 TRUST, 1 KL, 2 CONF, 3 KL_OR_CONF, 4 COVER, 5 COUPLED_ACCEPT,
6 CONF_DRAFT, 7 KL_STOCHASTIC.

Sources and readings:

* TRUST, [DualDiffusion] §2 "Verification algorithms" item 1: every drafted
  token is accepted unchanged -> KEEP.
* KL, item 2: a token is remasked when KL(p_v || p_d) exceeds tau. The page
  also names a probabilistic remask condition without giving its
  probability; that condition is not part of this rule. REMASK iff
  kl > tau (strict), else KEEP.
* KL_STOCHASTIC, item 2 with its probabilistic remask condition: the page
  gives no probability, so the reading is the plainest one that contains
  the threshold clause: one Bernoulli draw per row that remasks with
  probability min(1, kl / tau). Its uniform u comes from the same counter
  hash as the Gumbel noise (DV_HASH_V1, see oracle.noise), keyed on the seed
  and the row's position, at vocabulary index 2^32 - 1, which no token uses.
  The decision is taken in float32, as the kernel takes it:
  REMASK iff float32(u * tau) < float32(kl). kl > tau always remasks, since
  u < 1; kl = 0 never does, since u > 0. Requires tau > 0.
* CONF, item 3: low verifier confidence leads to remasking. REMASK iff
  conf < theta, else KEEP.
* KL_OR_CONF: REMASK iff either of the two conditions holds.
* CONF_DRAFT, item 3 read the other way: the verifier's confidence for the
  drafted token itself, p_v(tok_d) (``stats["p_tok"]``). REMASK iff
  p_tok < theta, else KEEP.
* COVER, [COVER] §3 "Adaptive revision outcomes": when the re-predicted token
  equals the current assignment the token is kept; when it differs and the
  verifier is confident it is replaced in place; it is remasked only when it
  is uncertain and likely wrong. Reading: re-predicted token = tok_v (the
  verifier's token; equal to argmax_v at T = 0); KEEP if tok_v == current;
  else REPLACE (with tok_v) if conf >= theta; else REMASK.
* COUPLED_ACCEPT, [SPOT] §1/§3 coupled-noise verification of candidate block
  states: a drafted token is accepted when the target, under the shared
  noise, draws the same token. Rows are grouped into candidates of
  ``group_len`` consecutive rows, in the candidate's commit order. Reading:
  the accepted prefix of a candidate is the number of leading decided rows
  whose tokens agree; the first disagreeing row takes the target's own token
  (REPLACE with tok_v, a valid draw of the target given the accepted
  prefix); decided rows after it are REMASKed.

"Current token" is ``cur_tok`` when given, else the drafter's token tok_d.
Rows with subject == 0 are not decided: NONE, and their output token is the
current token. REMASKed rows output ``mask_token``; REPLACEd rows output
tok_v; KEEP rows output the current token.

Accepted prefix of group c (any rule): the offset of the first decided row
in the group whose decision is not KEEP, or group_len if there is none.
Best group: the largest prefix, lowest group index on ties.
"""

from __future__ import annotations

import numpy as np

from . import noise

NONE, KEEP, REPLACE, REMASK = 0, 1, 2, 3
TRUST, KL, CONF, KL_OR_CONF, COVER, COUPLED_ACCEPT, CONF_DRAFT, KL_STOCHASTIC = 0, 1, 2, 3, 4, 5, 6, 7
REMASK_DRAW_INDEX = 2 ** 32 - 1   # the hash index of the remask draw

__all__ = ["NONE", "KEEP", "REPLACE", "REMASK", "TRUST", "KL", "CONF", "KL_OR_CONF",
           "COVER", "COUPLED_ACCEPT", "CONF_DRAFT", "KL_STOCHASTIC", "REMASK_DRAW_INDEX",
           "remask_uniforms", "decide", "accepted_prefix", "best_group"]


def remask_uniforms(seed: int, pos) -> np.ndarray:
    """The uniform of each row's remask draw (float32, exact): DV_HASH_V1 at
    (seed, pos[r], REMASK_DRAW_INDEX)."""
    h = noise.hash_words(seed, np.asarray(pos), 1, start=REMASK_DRAW_INDEX)[:, 0]
    return noise.uniforms(h).astype(np.float32)


def decide(rule: int, stats: dict, *, tau_kl: float = 0.0, conf_thr: float = 0.0,
           mask_token: int = -1, subject=None, cur_tok=None, group_len: int = 0, seed: int = 0, pos=None):
    """Apply ``rule`` to every row. Returns (decision uint8, out_tok int32).

    ``stats`` holds the row statistics needed by the rule (kl, conf, tok_v,
    tok_d), as float64 / int arrays of length R. ``seed`` and ``pos`` (int32
    positions, default the row index) key the draws of KL_STOCHASTIC.
    """
    rule = int(rule)
    cur = np.asarray(stats["tok_d"] if cur_tok is None else cur_tok).astype(np.int32)
    n = cur.shape[0]
    subj = np.ones(n, bool) if subject is None else (np.asarray(subject) != 0)
    dec = np.full(n, NONE, np.uint8)
    if rule == TRUST:
        dec[subj] = KEEP
    elif rule in (KL, CONF, KL_OR_CONF):
        remask = np.zeros(n, bool)
        if rule in (KL, KL_OR_CONF):
            remask |= np.asarray(stats["kl"], dtype=np.float64) > tau_kl
        if rule in (CONF, KL_OR_CONF):
            remask |= np.asarray(stats["conf"], dtype=np.float64) < conf_thr
        dec[subj] = np.where(remask[subj], REMASK, KEEP)
    elif rule == KL_STOCHASTIC:
        if not tau_kl > 0:
            raise ValueError("KL_STOCHASTIC needs tau_kl > 0")
        kl = np.asarray(stats["kl"]).astype(np.float32)
        u = remask_uniforms(seed, np.arange(n) if pos is None else pos)
        remask = (u * np.float32(tau_kl)).astype(np.float32) < kl
        dec[subj] = np.where(remask[subj], REMASK, KEEP)
    elif rule == CONF_DRAFT:
        p_tok = np.asarray(stats["p_tok"], dtype=np.float64)
        dec[subj] = np.where(p_tok[subj] < conf_thr, REMASK, KEEP)
    elif rule == COVER:
        tok_v = np.asarray(stats["tok_v"]).astype(np.int32)
        conf = np.asarray(stats["conf"], dtype=np.float64)
        d = np.where(tok_v == cur, KEEP, np.where(conf >= conf_thr, REPLACE, REMASK))
        dec[subj] = d[subj]
    elif rule == COUPLED_ACCEPT:
        if group_len <= 0 or n % group_len:
            raise ValueError("COUPLED_ACCEPT needs group_len > 0 dividing the row count")
        tok_v = np.asarray(stats["tok_v"]).astype(np.int32)
        agree = tok_v == cur
        for c in range(n // group_len):
            rejected = False
            for j in range(group_len):
                r = c * group_len + j
                if not subj[r]:
                    continue
                if rejected:
                    dec[r] = REMASK
                elif agree[r]:
                    dec[r] = KEEP
                else:
                    dec[r] = REPLACE
                    rejected = True
    else:
        raise ValueError(f"unknown rule {rule}")
    out = cur.copy()
    tok_v = stats.get("tok_v")
    if (dec == REPLACE).any():
        out[dec == REPLACE] = np.asarray(tok_v).astype(np.int32)[dec == REPLACE]
    out[dec == REMASK] = np.int32(mask_token)
    return dec, out


def accepted_prefix(decision, group_len: int, subject=None) -> np.ndarray:
    """Per group: offset of the first decided, non-KEEP row (group_len if none)."""
    decision = np.asarray(decision)
    n = decision.shape[0]
    if group_len <= 0 or n % group_len:
        raise ValueError("group_len must be positive and divide the row count")
    subj = np.ones(n, bool) if subject is None else (np.asarray(subject) != 0)
    out = np.empty(n // group_len, np.int32)
    for c in range(n // group_len):
        p = group_len
        for j in range(group_len):
            r = c * group_len + j
            if subj[r] and decision[r] != KEEP:
                p = j
                break
        out[c] = p
    return out


def best_group(prefix) -> int:
    """Group with the longest accepted prefix; lowest index on ties (-1 if none)."""
    prefix = np.asarray(prefix)
    if prefix.size == 0:
        return -1
    return int(np.argmax(prefix))
