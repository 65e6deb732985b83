"""Pins of the oracle's dynamic token tree against facts it does not define:
a hand-worked fixture, a global sort of every candidate (instead of the
best-first expansion), closed forms for one depth, and structural
invariants of the block it emits."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import verify_oracle as O
from tests.helpers import load_golden


def test_golden_tree():
    g = load_golden("dynamic_tree_v5.txt")
    p = np.array([g["probs"]], dtype=np.float32)
    d, par, dep, n = O.dynamic_tree(p, [g["root"]], g["W"], g["n_mask"])
    assert list(d[0]) == g["draft"] and list(par[0]) == g["parents"]
    assert list(dep[0]) == g["depth"] and n[0] == g["n_nodes"]
    d, par, dep, n = O.dynamic_tree(p, [g["root"]], g["W"], g["n_mask"], g["thr"])
    assert list(d[0]) == g["thr_draft"] and list(par[0]) == g["thr_parents"]
    assert list(dep[0]) == g["thr_depth"] and n[0] == g["thr_n_nodes"]


def random_probs(rng, B, K, V, peak=8.0):
    w = rng.random((B, K, V)) ** peak
    return (w / w.sum(axis=-1, keepdims=True)).astype(np.float32)


def global_sort_tree(p, root, W, n_mask, thr):
    """Every candidate of every depth (children of the depth's top-1 parent),
    sorted once; the first W - 1 - n_mask that reach thr."""
    K, V = p.shape
    spine, c = [root], [np.float32(1.0)]
    cands = []
    for d in range(1, K + 1):
        vs = [v for v in range(V) if v != spine[-1]]
        vs.sort(key=lambda v: (-float(p[d - 1, v]), v))
        for r, v in enumerate(vs):
            cands.append((-float(np.float32(c[-1] * p[d - 1, v])), d, r, v))
        spine.append(vs[0])
        c.append(np.float32(c[-1] * p[d - 1, vs[0]]))
    cands.sort()
    out = []
    for negcp, d, r, v in cands[:W - 1 - n_mask]:
        if -negcp < float(np.float32(thr)):
            break
        out.append((d, v))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_best_first_equals_global_sort(seed):
    rng = np.random.default_rng(100 + seed)
    K, V, W = int(rng.integers(1, 7)), int(rng.integers(3, 40)), int(rng.integers(2, 30))
    n_mask = int(rng.integers(0, W))
    thr = float(rng.choice([0.0, 1e-3, 0.05]))
    p = random_probs(rng, 3, K, V)
    root = rng.integers(0, V, size=3)
    d, par, dep, n = O.dynamic_tree(p, root, W, n_mask, thr)
    for b in range(3):
        want = global_sort_tree(p[b], int(root[b]), W, n_mask, thr)
        got = [(int(dep[b, i]), int(d[b, i])) for i in range(1, int(n[b]))]
        assert got == want


@pytest.mark.parametrize("seed", range(8))
def test_block_invariants(seed):
    rng = np.random.default_rng(200 + seed)
    B, K, V, W, n_mask = 4, 5, 50, 24, 3
    p = random_probs(rng, B, K, V, peak=4.0)
    root = rng.integers(0, V, size=B)
    d, par, dep, n = O.dynamic_tree(p, root, W, n_mask)
    for b in range(B):
        assert O.mask_is_valid(O.TREE, par[b])
        assert d[b, 0] == root[b] and par[b, 0] == -1 and dep[b, 0] == 0
        assert n[b] <= W - n_mask
        for i in range(1, W):
            assert dep[b, i] == dep[b, par[b, i]] + 1
            if i < n[b]:
                assert d[b, i] != d[b, par[b, i]]          # no consecutive repeat
                assert dep[b, i] <= K
            else:
                assert d[b, i] == -1                        # mask-token rows
        # only top-1 nodes have children
        kids = set(int(par[b, i]) for i in range(1, n[b]))
        for k in kids:
            if k > 0:
                dd = dep[b, k]
                sibl = [i for i in range(1, n[b]) if dep[b, i] == dd]
                assert k == min(sibl)


def test_one_depth_is_the_top_tokens_of_the_first_distribution():
    rng = np.random.default_rng(5)
    p = random_probs(rng, 2, 1, 30)
    d, par, dep, n = O.dynamic_tree(p, [7, 0], 10, 2)
    for b, root in enumerate((7, 0)):
        order = [v for v in np.argsort(-p[b, 0], kind="stable") if v != root]
        assert list(d[b, 1:8]) == order[:7]
        assert np.all(par[b, 1:8] == 0) and n[b] == 8
        assert list(par[b, 8:]) == [1, 8] and np.all(d[b, 8:] == -1)


def test_ties_go_to_the_smaller_token():
    p = np.full((1, 2, 6), 1 / 6, dtype=np.float32)
    d, par, dep, n = O.dynamic_tree(p, [0], 8, 0)
    # depth 1: tokens 1..5 (0 is the root); spine 1; the depth-1 nodes all
    # have cumulative probability 1/6, ahead of depth 2 (1/36)
    assert list(d[0, 1:6]) == [1, 2, 3, 4, 5]
    assert list(d[0, 6:8]) == [0, 2] and list(par[0, 6:8]) == [1, 1]


def test_positions_chain_and_segment_are_sequential():
    ids = np.array([[-1, 0, 1, 2, 3], [0, 0, 1, 1, 2]])
    pos = O.block_positions([10, 7], [O.CHAIN, O.SEGMENT], ids)
    assert pos.tolist() == [[10, 11, 12, 13, 14], [7, 8, 9, 10, 11]]


def test_positions_of_a_tree_are_depths_from_the_golden_tree():
    g = load_golden("dynamic_tree_v5.txt")
    pos = O.block_positions([100], [O.TREE], np.array([g["parents"]]))
    assert list(pos[0]) == [100 + d for d in g["depth"]]


def test_positions_of_a_malformed_mask_are_minus_one():
    pos = O.block_positions([5], [O.TREE], np.array([[-1, 0, 2]]))
    assert np.all(pos == -1)


def test_golden_tree_one_token_vocabulary():
    """V = 1: pruning leaves no candidate at any depth (hand-worked fixture)."""
    g = load_golden("dynamic_tree_v1.txt")
    p = np.array([g["probs"]], dtype=np.float32)
    for thr in (0.0, 0.5):
        d, par, dep, n = O.dynamic_tree(p, [g["root"]], g["W"], g["n_mask"], thr)
        assert list(d[0]) == g["draft"] and list(par[0]) == g["parents"]
        assert list(dep[0]) == g["depth"] and n[0] == g["n_nodes"]
