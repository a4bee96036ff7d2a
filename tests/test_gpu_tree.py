"""GPU parity of dv_tree_accept (acceptance over trees of candidate block states)
against oracle.tree, exact: every output is integer work on the same inputs."""

import numpy as np
import pytest
import torch

import token_verification_row_amd as dv
import workloads as W
from oracle import tree as T

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _t(x, dtype, dev):
    return torch.from_numpy(np.ascontiguousarray(x).astype(dtype)).to(dev)


def _masked_sets(parent, node_pos, root_masked):
    L = len(root_masked)
    out = [np.asarray(root_masked, bool).copy()]
    for i in range(1, len(parent)):
        m = out[parent[i]].copy()
        if 0 <= node_pos[i] < L:
            m[node_pos[i]] = False
        out.append(m)
    return out


def _random_tree(rng, n, L, vocab, p_follow, deep=False):
    """A random tree whose nodes copy their parent's transition with probability p_follow."""
    conf = np.round(rng.random((n, L)), 2).astype(np.float32)      # rounding makes equal confidences common
    tok = rng.integers(0, vocab, (n, L)).astype(np.int32)
    masked0 = (rng.random(L) < 0.8).astype(np.uint8)
    parent = np.zeros(n, np.int32)
    parent[0] = -1
    node_pos = np.zeros(n, np.int32)
    node_tok = np.zeros(n, np.int32)
    masks = [masked0.astype(bool)]
    for i in range(1, n):
        q = i - 1 if deep else int(rng.integers(max(0, i - 8), i))
        parent[i] = q
        tp, tt = T.transition(masks[q], conf[q], tok[q])
        if tp >= 0 and rng.random() < p_follow:
            node_pos[i], node_tok[i] = tp, tt
        else:
            node_pos[i], node_tok[i] = int(rng.integers(0, L)), int(rng.integers(0, vocab))
        m = masks[q].copy()
        m[node_pos[i]] = False
        masks.append(m)
    return parent, node_pos, node_tok, masked0, conf, tok


def _run_batch(trees, dev, with_block=True):
    parent = np.stack([t[0] for t in trees])
    node_pos = np.stack([t[1] for t in trees])
    node_tok = np.stack([t[2] for t in trees])
    masked = np.stack([t[3] for t in trees])
    conf = np.stack([t[4] for t in trees])
    tok = np.stack([t[5] for t in trees])
    L = masked.shape[1]
    block = np.arange(len(trees) * L, dtype=np.int32).reshape(len(trees), L) + 1000
    gm = _t(masked, np.uint8, dev)
    gb = _t(block, np.int32, dev) if with_block else None
    got = dv.dv_tree_accept(_t(parent, np.int32, dev), _t(node_pos, np.int32, dev), _t(node_tok, np.int32, dev), gm,
                            _t(conf, np.float32, dev), _t(tok, np.int32, dev), block_tokens=gb,
                            update_mask=with_block)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items()}
    for b, tr in enumerate(trees):
        ref = T.tree_accept(*tr)
        np.testing.assert_array_equal(got["accepted"][b].astype(bool), ref["accepted"], err_msg=f"tree {b} accepted")
        np.testing.assert_array_equal(got["depth"][b], ref["depth"], err_msg=f"tree {b} depth")
        assert got["best_node"][b] == ref["best"], b
        c = len(ref["commit_pos"])
        assert got["commit_len"][b] == c, b
        np.testing.assert_array_equal(got["commit_pos"][b][:c], ref["commit_pos"])
        np.testing.assert_array_equal(got["commit_tok"][b][:c], ref["commit_tok"])
        assert (got["commit_pos"][b][c:] == -1).all() and (got["commit_tok"][b][c:] == -1).all()
        if with_block:
            rt, rm = T.apply_commits(block[b], masked[b], ref["commit_pos"], ref["commit_tok"])
            np.testing.assert_array_equal(gb[b].cpu().numpy(), rt)
            np.testing.assert_array_equal(gm[b].cpu().numpy(), rm)
    return got


def test_hand_example():
    print("case: tree hand example", flush=True)
    L = 4
    parent = np.array([-1, 0, 0, 0, 1, 2, 4], np.int32)
    node_pos = np.array([0, 2, 2, 1, 0, 0, 3], np.int32)
    node_tok = np.array([0, 7, 5, 7, 9, 9, 1], np.int32)
    conf = np.zeros((7, L), np.float32)
    tok = np.zeros((7, L), np.int32)
    conf[0] = [0.1, 0.3, 0.9, 0.2]; tok[0] = [4, 4, 7, 4]
    conf[1] = [0.8, 0.3, 0.99, 0.2]; tok[1] = [9, 4, 0, 4]
    conf[4] = [0.99, 0.3, 0.99, 0.5]; tok[4] = [0, 4, 0, 2]
    got = _run_batch([(parent, node_pos, node_tok, np.ones(L, np.uint8), conf, tok)], _dev())
    assert got["best_node"][0] == 4 and got["commit_len"][0] == 3


@pytest.mark.parametrize("n,L,vocab,p_follow", [(1, 1, 1, 0.0), (1, 7, 3, 0.0), (5, 3, 2, 0.9), (64, 32, 4, 0.8),
                                                (200, 16, 2, 0.6), (300, 100, 3, 0.95), (1024, 64, 2, 0.9), (1024, 65, 2, 0.9),
                                                (64, 64, 2, 0.9), (65, 64, 2, 0.9), (1024, 4, 2, 0.9), (205, 20, 2, 0.9)])
def test_random_trees(n, L, vocab, p_follow):
    print(f"case: random trees n={n} L={L}", flush=True)
    rng = np.random.default_rng(n * 131 + L)
    trees = [_random_tree(rng, n, L, vocab, p_follow) for _ in range(24 if n < 1000 else 3)]
    got = _run_batch(trees, _dev())
    if p_follow >= 0.8 and n > 1 and L > 1:
        assert got["depth"].max() >= 2           # the cases do reach past the first level


def test_maximum_sizes_and_deep_chains():
    print("case: tree maximum sizes", flush=True)
    rng = np.random.default_rng(5)
    dev = _dev()
    # the largest tree over the largest block; and chains deeper than the block
    _run_batch([_random_tree(rng, 1024, 1024, 3, 0.97)], dev)
    _run_batch([_random_tree(rng, 1024, 8, 2, 0.9, deep=True) for _ in range(4)], dev)
    _run_batch([_random_tree(rng, 1024, 64, 2, 0.99, deep=True) for _ in range(2)], dev)
    _run_batch([_random_tree(rng, 1024, 200, 2, 0.99, deep=True)], dev)
    _run_batch([_random_tree(rng, 600, 1, 1, 1.0, deep=True)], dev, with_block=False)


def test_broken_layout_is_not_accepted():
    print("case: tree broken layout", flush=True)
    dev = _dev()
    rng = np.random.default_rng(9)
    parent, node_pos, node_tok, masked, conf, tok = _random_tree(rng, 40, 12, 2, 1.0)
    bad = parent.copy()
    bad[10], bad[20], bad[30] = 10, 35, -3                        # itself, a later node, negative
    pos = node_pos.copy()
    pos[15] = 12                                                  # outside the block
    got = dv.dv_tree_accept(_t(bad[None], np.int32, dev), _t(pos[None], np.int32, dev), _t(node_tok[None], np.int32, dev),
                            _t(masked[None], np.uint8, dev), _t(conf[None], np.float32, dev), _t(tok[None], np.int32, dev))
    depth = got["depth"].cpu().numpy()[0]
    # reference: the broken nodes hang off the root with an impossible position, so they and their
    # descendants are rejected and nothing else changes
    ref_parent, ref_pos = bad.copy(), pos.copy()
    for i in (10, 20, 30, 15):
        ref_parent[i], ref_pos[i] = 0, 12
    ref = T.tree_accept(ref_parent, ref_pos, node_tok, masked, conf, tok)
    np.testing.assert_array_equal(depth, ref["depth"])
    assert got["best_node"].cpu().numpy()[0] == ref["best"]


def test_chain_from_verify_rows():
    """Acceptance fed by dv_verify_rows under shared noise: 64 node states x 32 positions."""
    print("case: tree from verify rows", flush=True)
    dev = _dev()
    w = W.workload(4)
    nodes, L, V = 64, 32, 4096
    rng = np.random.default_rng(17)
    a = (rng.standard_normal((nodes * L, V)) * 2.0).astype(np.float32)
    a[np.arange(nodes * L), rng.integers(0, V, nodes * L)] += 6.0
    b = a + rng.standard_normal((nodes * L, V)).astype(np.float32) * 0.5
    ta = torch.from_numpy(W.round_bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
    tb = torch.from_numpy(W.round_bf16_bits(b).view(np.int16)).to(dev).view(torch.bfloat16)
    st = dv.dv_verify_rows(ta, tb, temperature=1.0, seed=w.seed, pos_period=L)
    conf = st["conf"].cpu().numpy().reshape(1, nodes, L)
    tok = st["tok_v"].cpu().numpy().reshape(1, nodes, L)
    # a tree whose nodes mostly follow the target's transitions computed from these statistics
    parent = np.zeros(nodes, np.int32); parent[0] = -1
    node_pos = np.zeros(nodes, np.int32); node_tok = np.zeros(nodes, np.int32)
    masks = [np.ones(L, bool)]
    for i in range(1, nodes):
        q = int(rng.integers(max(0, i - 4), i))
        parent[i] = q
        tp, tt = T.transition(masks[q], conf[0, q], tok[0, q])
        if rng.random() < 0.85:
            node_pos[i], node_tok[i] = tp, tt
        else:
            node_pos[i], node_tok[i] = int(rng.integers(0, L)), int(tok[0, q, int(rng.integers(0, L))])
        m = masks[q].copy(); m[node_pos[i]] = False; masks.append(m)
    got = dv.dv_tree_accept(_t(parent[None], np.int32, dev), _t(node_pos[None], np.int32, dev),
                            _t(node_tok[None], np.int32, dev), torch.ones((1, L), dtype=torch.uint8, device=dev),
                            st["conf"], st["tok_v"])
    ref = T.tree_accept(parent, node_pos, node_tok, np.ones(L, np.uint8), conf[0], tok[0])
    np.testing.assert_array_equal(got["depth"].cpu().numpy()[0], ref["depth"])
    assert int(got["best_node"].cpu()[0]) == ref["best"]
    n = int(got["commit_len"].cpu()[0])
    np.testing.assert_array_equal(got["commit_pos"].cpu().numpy()[0][:n], ref["commit_pos"])
    print("accepted depth", int(ref["depth"].max()), "commits", n, flush=True)
