"""Acceptance over a tree of candidate block states, and the commit it yields (oracle).

Test infrastructure: see the package docstring for who may import this.

Source: [SPOT] §1 "Key Terms & Definitions" and §3 "Method & Key Results". The
drafter proposes a multi-level tree of candidate block states: each state is
its parent's state with one more position committed, following a predicted
commit order. The target verifies every state of the tree in one batched pass.
Under coupled noise, the target's transition from a state is deterministic, so
a proposed child is right exactly when it equals that transition.

The page gives no formulas; these are the readings taken:

* Tree: nodes 0..n-1 in topological order, node 0 is the root (the current
  block state), 0 <= parent[i] < i for i >= 1. Node i >= 1 commits token
  node_tok[i] at block position node_pos[i] on top of its parent's state.
* Masked positions of a node's state: the root's masked positions minus the
  positions committed on the path from the root to that node.
* Target transition from node i's state: the masked position p with the
  highest verifier confidence conf[i][p] (the lowest p among equal
  confidences), committed with the verifier's token tok_v[i][p] (its
  Gumbel-max token under the shared noise; the argmax at T = 0). A state with
  no masked position has no transition (position and token -1).
* Node i >= 1 is accepted iff its parent is accepted and (node_pos[i],
  node_tok[i]) equals the parent's transition. The root is accepted.
  depth[i] = number of commits from the root to i, or -1 when not accepted.
* Best node: the deepest accepted node, lowest index on ties.
* Commit list: the (position, token) of the nodes on the path from the root
  to the best node, in order, then the target's own transition at the best
  node when it has one. The target draws it there whether or not a child
  proposed it, so each verification pass commits depth(best) + 1 positions
  while any remain masked.
* Applying the commit list to the block: each committed position takes its
  token and is no longer masked.
"""

from __future__ import annotations

import numpy as np

__all__ = ["transition", "tree_accept", "apply_commits"]


def transition(masked, conf_row, tok_row):
    """(position, token) the target commits from a state, or (-1, -1) if nothing is masked."""
    best_p, best_c = -1, None
    for p in range(len(masked)):
        if masked[p] and (best_c is None or conf_row[p] > best_c):
            best_p, best_c = p, conf_row[p]
    if best_p < 0:
        return -1, -1
    return best_p, int(tok_row[best_p])


def tree_accept(parent, node_pos, node_tok, root_masked, conf, tok_v):
    """Acceptance of every node of one tree.

    parent, node_pos, node_tok: int [n] (entries of the root are ignored).
    root_masked: bool/uint8 [L]. conf: float [n][L], tok_v: int [n][L], the
    verifier statistics of each node's state.

    Returns a dict with accepted (bool [n]), depth (int32 [n]), target_pos and
    target_tok (int32 [n], each node's transition), best (int) and the commit
    list commit_pos / commit_tok (int32 arrays).
    """
    parent = np.asarray(parent, np.int64)
    n = parent.shape[0]
    L = len(root_masked)
    conf = np.asarray(conf, np.float64).reshape(n, L)
    tok_v = np.asarray(tok_v, np.int64).reshape(n, L)
    if n < 1:
        raise ValueError("a tree has at least its root")
    masked = [None] * n
    masked[0] = [bool(m) for m in root_masked]
    for i in range(1, n):
        if not 0 <= parent[i] < i:
            raise ValueError("nodes must be in topological order (0 <= parent[i] < i)")
        m = list(masked[parent[i]])
        p = int(node_pos[i])
        if 0 <= p < L:
            m[p] = False
        masked[i] = m
    tpos = np.empty(n, np.int32)
    ttok = np.empty(n, np.int32)
    for i in range(n):
        tpos[i], ttok[i] = transition(masked[i], conf[i], tok_v[i])
    accepted = np.zeros(n, bool)
    depth = np.full(n, -1, np.int32)
    accepted[0], depth[0] = True, 0
    for i in range(1, n):
        q = parent[i]
        if accepted[q] and tpos[q] >= 0 and int(node_pos[i]) == tpos[q] and int(node_tok[i]) == ttok[q]:
            accepted[i] = True
            depth[i] = depth[q] + 1
    best = int(np.argmax(depth))  # first maximum: lowest index among the deepest
    path = []
    j = best
    while j > 0:
        path.append(j)
        j = int(parent[j])
    path.reverse()
    cpos = [int(node_pos[j]) for j in path]
    ctok = [int(node_tok[j]) for j in path]
    if tpos[best] >= 0:
        cpos.append(int(tpos[best]))
        ctok.append(int(ttok[best]))
    return dict(accepted=accepted, depth=depth, target_pos=tpos, target_tok=ttok, best=best,
                commit_pos=np.asarray(cpos, np.int32), commit_tok=np.asarray(ctok, np.int32))


def apply_commits(tokens, masked, commit_pos, commit_tok):
    """Block tokens and mask after the commits (new arrays)."""
    tokens = np.array(tokens, np.int32, copy=True)
    masked = np.array(masked, np.uint8, copy=True)
    for p, t in zip(commit_pos, commit_tok):
        tokens[p] = t
        masked[p] = 0
    return tokens, masked
