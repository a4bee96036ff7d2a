"""Pins for oracle.tree: a worked example by hand, the target's own sequential
decode (simulated state by state, without a tree), exhaustive trees over tiny
blocks, and invariants of the acceptance on random trees."""

import itertools

import numpy as np

from oracle import tree as T


def test_hand_example():
    # block of 4 positions, all masked in the root state
    L = 4
    root_masked = [1, 1, 1, 1]
    # nodes: 0 root; 1 = (pos 2, tok 7) right; 2 = (pos 2, tok 5) wrong token; 3 = (pos 1, tok 7) wrong position;
    # 4 = child of 1, (pos 0, tok 9) right; 5 = child of 2 (parent rejected); 6 = child of 4, (pos 3, tok 1) wrong
    parent = [-1, 0, 0, 0, 1, 2, 4]
    node_pos = [0, 2, 2, 1, 0, 0, 3]
    node_tok = [0, 7, 5, 7, 9, 9, 1]
    n = len(parent)
    conf = np.zeros((n, L))
    tok = np.zeros((n, L), np.int64)
    conf[0] = [0.1, 0.3, 0.9, 0.2]; tok[0] = [4, 4, 7, 4]     # root: commit pos 2 with 7
    conf[1] = [0.8, 0.3, 0.99, 0.2]; tok[1] = [9, 4, 0, 4]    # pos 2 is no longer masked: commit pos 0 with 9
    conf[4] = [0.99, 0.3, 0.99, 0.5]; tok[4] = [0, 4, 0, 2]   # masked {1, 3}: commit pos 3 with 2
    r = T.tree_accept(parent, node_pos, node_tok, root_masked, conf, tok)
    assert list(r["accepted"]) == [True, True, False, False, True, False, False]
    assert list(r["depth"]) == [0, 1, -1, -1, 2, -1, -1]
    assert r["best"] == 4
    assert list(r["commit_pos"]) == [2, 0, 3] and list(r["commit_tok"]) == [7, 9, 2]
    assert (r["target_pos"][4], r["target_tok"][4]) == (3, 2)
    toks, m = T.apply_commits([0, 0, 0, 0], root_masked, r["commit_pos"], r["commit_tok"])
    assert list(toks) == [9, 0, 7, 2] and list(m) == [0, 1, 0, 0]


def test_ties_and_empty_block():
    # equal confidences: the lowest position; a state with nothing masked has no transition
    assert T.transition([1, 1, 1], [0.5, 0.7, 0.7], [1, 2, 3]) == (1, 2)
    assert T.transition([0, 0], [0.5, 0.7], [1, 2]) == (-1, -1)
    r = T.tree_accept([-1], [0], [0], [0, 0, 0], np.zeros((1, 3)), np.zeros((1, 3)))
    assert r["best"] == 0 and len(r["commit_pos"]) == 0
    # equally deep accepted nodes: the lowest index wins
    r = T.tree_accept([-1, 0, 0], [0, 1, 1], [0, 5, 5], [1, 1], [[0.1, 0.9], [0, 0], [0, 0]], [[3, 5], [0, 0], [0, 0]])
    assert list(r["accepted"]) == [True, True, True] and r["best"] == 1


class _Target:
    """A deterministic stand-in for the target model: confidence and token of
    every position as a function of the block state (committed tokens)."""

    def __init__(self, L, vocab, seed):
        self.L, self.vocab, self.seed = L, vocab, seed

    def stats(self, tokens, masked):
        key = hash((self.seed, tuple(int(t) for t in tokens), tuple(int(m) for m in masked))) & 0xFFFFFFFF
        g = np.random.default_rng(key)
        return g.random(self.L), g.integers(0, self.vocab, self.L)


def _sequential_decode(target, tokens, masked):
    """The target's own decode from a state, one commit at a time (no tree)."""
    tokens, masked = list(tokens), list(masked)
    out = []
    while any(masked):
        conf, tok = target.stats(tokens, masked)
        cand = [p for p in range(len(masked)) if masked[p]]
        best = max(cand, key=lambda p: (conf[p], -p))
        out.append((best, int(tok[best])))
        tokens[best] = int(tok[best])
        masked[best] = 0
    return out


def _state_stats(target, parent, node_pos, node_tok, tokens0, masked0):
    n = len(parent)
    toks, msk = [None] * n, [None] * n
    toks[0], msk[0] = list(tokens0), list(masked0)
    conf, tok = np.zeros((n, len(masked0))), np.zeros((n, len(masked0)), np.int64)
    for i in range(n):
        if i:
            toks[i], msk[i] = list(toks[parent[i]]), list(msk[parent[i]])
            toks[i][node_pos[i]] = node_tok[i]
            msk[i][node_pos[i]] = 0
        conf[i], tok[i] = target.stats(toks[i], msk[i])
    return conf, tok


def test_tree_containing_the_target_decode_accepts_it():
    rng = np.random.default_rng(7)
    for trial in range(40):
        L, vocab = int(rng.integers(1, 7)), int(rng.integers(1, 4))
        target = _Target(L, vocab, trial)
        tokens0 = list(rng.integers(0, vocab, L))
        masked0 = list((rng.random(L) < 0.8).astype(int))
        truth = _sequential_decode(target, tokens0, masked0)
        # a chain along the truth (up to a random depth) plus random distractor nodes anywhere
        depth = int(rng.integers(0, len(truth) + 1))
        parent, node_pos, node_tok = [-1], [0], [0]
        for d in range(depth):
            parent.append(len(parent) - 1)
            node_pos.append(truth[d][0]); node_tok.append(truth[d][1])
        for _ in range(int(rng.integers(0, 12))):
            parent.append(int(rng.integers(0, len(parent))))
            node_pos.append(int(rng.integers(0, L))); node_tok.append(int(rng.integers(0, vocab)))
        conf, tok = _state_stats(target, parent, node_pos, node_tok, tokens0, masked0)
        r = T.tree_accept(parent, node_pos, node_tok, masked0, conf, tok)
        # the commit list is a prefix of the target's own decode, one longer than the accepted depth
        got = list(zip(r["commit_pos"].tolist(), r["commit_tok"].tolist()))
        assert got == truth[:len(got)]
        assert len(got) == min(int(r["depth"][r["best"]]) + 1, len(truth))
        assert int(r["depth"][r["best"]]) >= depth


def test_exhaustive_tree_reaches_the_end_of_the_decode():
    # every (position, token) child of every node, depth-first: exactly the target's decode is accepted
    for L, vocab in ((2, 2), (3, 2), (2, 3)):
        target = _Target(L, vocab, 100 + L * 10 + vocab)
        tokens0, masked0 = [0] * L, [1] * L
        parent, node_pos, node_tok, msk = [-1], [0], [0], [tuple(masked0)]
        frontier = [0]
        while frontier:
            q = frontier.pop()
            for p, t in itertools.product(range(L), range(vocab)):
                if msk[q][p]:
                    parent.append(q); node_pos.append(p); node_tok.append(t)
                    m = list(msk[q]); m[p] = 0; msk.append(tuple(m))
                    frontier.append(len(parent) - 1)
        # renumber into topological order (parents first): sort by depth, stable
        depth = [0] * len(parent)
        for i in range(1, len(parent)):
            depth[i] = depth[parent[i]] + 1
        order = sorted(range(len(parent)), key=lambda i: depth[i])
        new = {o: k for k, o in enumerate(order)}
        parent = [-1 if i == 0 else new[parent[i]] for i in order]
        node_pos = [node_pos[i] for i in order]; node_tok = [node_tok[i] for i in order]
        conf, tok = _state_stats(target, parent, node_pos, node_tok, tokens0, masked0)
        r = T.tree_accept(parent, node_pos, node_tok, masked0, conf, tok)
        truth = _sequential_decode(target, tokens0, masked0)
        assert int(r["depth"][r["best"]]) == L
        assert list(zip(r["commit_pos"].tolist(), r["commit_tok"].tolist())) == truth
        # one accepted node per depth
        assert np.bincount(r["depth"][r["accepted"]]).tolist() == [1] * (L + 1)


def test_invariants_on_random_trees():
    rng = np.random.default_rng(11)
    for trial in range(200):
        n, L, vocab = int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 3))
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        node_pos = rng.integers(0, L, n); node_tok = rng.integers(0, vocab, n)
        masked = (rng.random(L) < 0.7).astype(np.uint8)
        conf = np.round(rng.random((n, L)), 1); tok = rng.integers(0, vocab, (n, L))
        r = T.tree_accept(parent, node_pos, node_tok, masked, conf, tok)
        acc, dep = r["accepted"], r["depth"]
        for i in range(1, n):
            if acc[i]:
                assert acc[parent[i]] and dep[i] == dep[parent[i]] + 1
                assert (node_pos[i], node_tok[i]) == (r["target_pos"][parent[i]], r["target_tok"][parent[i]])
            else:
                assert dep[i] == -1
        assert dep[r["best"]] == dep.max() and r["best"] == int(np.flatnonzero(dep == dep.max())[0])
        # statistics of states outside the accepted set change nothing
        conf2, tok2 = conf.copy(), tok.copy()
        off = ~acc
        conf2[off] = rng.random((off.sum(), L)); tok2[off] = rng.integers(0, vocab, (off.sum(), L))
        r2 = T.tree_accept(parent, node_pos, node_tok, masked, conf2, tok2)
        assert (r2["accepted"] == acc).all() and r2["best"] == r["best"]
        assert (r2["commit_pos"] == r["commit_pos"]).all() and (r2["commit_tok"] == r["commit_tok"]).all()
        # each committed position was masked and appears once
        cp = r["commit_pos"].tolist()
        assert len(set(cp)) == len(cp) and all(masked[p] for p in cp)
