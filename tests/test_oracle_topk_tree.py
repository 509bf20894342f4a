"""Pins for the top-k and tree oracles: brute force, the page's example tree,
P1's second mask construction, and invariants that a wrong index, a missing
ancestor or a transposed mask would break."""
import itertools
import json
import os

import numpy as np
import pytest

from medusa_tree_verification_amd import synth
from oracle import topk, tree


def brute_topk(x, k):
    return sorted(range(len(x)), key=lambda i: (-x[i], i))[:k]


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 17))
    # small integer values force many ties
    x = rng.integers(-3, 4, size=V).astype(np.float64)
    for k in range(1, V + 1):
        assert list(topk.topk(x, k)) == brute_topk(list(x), k)


def test_topk_k1_is_argmax_first_max():
    rng = np.random.default_rng(7)
    for _ in range(50):
        x = rng.integers(0, 5, size=30).astype(np.float32)
        assert topk.topk(x, 1)[0] == np.argmax(x)


def test_topk_ties_and_signed_zero():
    assert list(topk.topk(np.array([1.0, 3.0, 3.0, 2.0, 3.0]), 3)) == [1, 2, 4]
    # -0.0 and +0.0 compare equal: the lower index wins
    assert list(topk.topk(np.array([-0.0, 0.0, -1.0]), 2)) == [0, 1]


def test_head_topk_padding():
    x = np.random.default_rng(8).normal(size=(2, 3, 20))
    out = topk.head_topk(x, [4, 2, 1])
    assert out.shape == (2, 3, 4)
    assert np.all(out[:, 1, 2:] == -1) and np.all(out[:, 2, 1:] == -1)
    assert out[1, 2, 0] == np.argmax(x[1, 2])


def _trees():
    yield synth.chain_tree(5)
    yield synth.cartesian_tree((2, 3, 2))
    for name in synth.WORKLOAD_ORDER:
        w = synth.WORKLOADS[name]
        yield synth.cost_ordered_tree(w.topk, w.T)
    for s in range(6):
        yield synth.random_tree(40, (6, 4, 3, 2), s)
    yield np.array([-1], np.int32), np.array([0], np.int32)


@pytest.mark.parametrize("idx", range(14))
def test_mask_two_constructions_agree(idx):
    parent, rank = list(_trees())[idx]
    T = len(parent)
    vis = tree.visible_bruteforce(parent)
    clo = tree.visible_by_closure(parent)
    np.testing.assert_array_equal(clo, vis)
    mask = tree.additive_mask(clo)
    assert mask.shape == (T, T)
    np.testing.assert_array_equal(mask == 0.0, vis)
    np.testing.assert_array_equal(np.isneginf(mask), ~vis)


@pytest.mark.parametrize("idx", range(14))
def test_mask_invariants(idx):
    parent, rank = list(_trees())[idx]
    vis = tree.visible_bruteforce(parent)
    depth = tree.depth_of(parent)
    T = len(parent)
    assert np.all(vis.sum(axis=1) == depth + 1)          # itself + one ancestor per level
    assert np.all(vis[:, 0])                             # everyone sees the root
    assert np.all(np.diag(vis))
    assert not np.any(np.triu(vis, 1))                   # parent[n] < n: no later node visible
    for i in range(T):                                   # prefix-closed
        for j in np.nonzero(vis[i])[0]:
            assert np.all(vis[i] >= vis[j])


def test_bitmask_rows_bits():
    parent, _ = synth.random_tree(150, (8, 6, 4, 3), 3)
    vis = tree.visible_bruteforce(parent)
    words = tree.bitmask_rows(vis)
    assert words.shape == (150, 3)
    for i in range(150):
        for j in range(150):
            bit = (int(words[i, j // 64]) >> (j % 64)) & 1
            assert bit == int(vis[i, j])


def test_page_example_tree(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_tree_example.json")))
    parent, rank = synth.cartesian_tree(g["topk"])
    tree.validate(parent, rank, g["topk"])
    depth = tree.depth_of(parent)
    assert len(parent) == g["expected_nodes_with_root"]
    assert np.bincount(depth).tolist() == g["expected_nodes_per_depth"]
    leaves = [n for n in range(len(parent)) if n not in set(parent.tolist())]
    assert len(leaves) == g["expected_leaves"]


def test_validate_rejects_bad_topologies():
    k = [3, 2]
    tree.validate([-1, 0, 0, 1], [0, 0, 1, 1], k)
    with pytest.raises(ValueError):
        tree.validate([0, 0], [0, 0], k)                 # root must have parent -1
    with pytest.raises(ValueError):
        tree.validate([-1, 2, 0], [0, 0, 1], k)          # parent after child
    with pytest.raises(ValueError):
        tree.validate([-1, 0, 0], [0, 1, 1], k)          # duplicate sibling rank
    with pytest.raises(ValueError):
        tree.validate([-1, 0, 1], [0, 0, 2], k)          # rank beyond head 2's top-2
    with pytest.raises(ValueError):
        tree.validate([-1, 0, 1, 2], [0, 0, 0, 0], k)    # deeper than K heads


def test_tree_tokens_and_positions_hand_example():
    parent = [-1, 0, 0, 1, 2]
    rank = [0, 0, 1, 1, 0]
    tk = np.array([[[50, 51], [60, 61]], [[70, 71], [80, 81]]])   # [B=2, K=2, kmax=2]
    toks = tree.tree_tokens(tk, [7, 8], parent, rank)
    np.testing.assert_array_equal(toks, [[7, 50, 51, 61, 60], [8, 70, 71, 81, 80]])
    np.testing.assert_array_equal(tree.positions([100, 5], parent),
                                  [[100, 101, 101, 102, 102], [5, 6, 6, 7, 7]])


def test_children_in_rank_order():
    parent = [-1, 0, 0, 0, 1]
    rank = [0, 2, 0, 1, 0]
    assert tree.children_in_rank_order(parent, rank)[0] == [2, 3, 1]


def test_cost_ordered_generator_regression():
    # per-depth node counts of the cost-ordered reading for the five workloads
    expect = {"tiny-fp32": [1, 2, 4, 1], "vicuna7b-shaped": [1, 7, 21, 20, 15],
              "vicuna13b-shaped": [1, 7, 15, 20, 15, 6], "vicuna33b-shaped": [1, 7, 21, 35, 32],
              "zephyr7b-shaped": [1, 7, 15, 20, 15, 6]}
    for name, counts in expect.items():
        w = synth.WORKLOADS[name]
        parent, rank = synth.cost_ordered_tree(w.topk, w.T)
        tree.validate(parent, rank, w.topk)
        assert np.bincount(tree.depth_of(parent)).tolist() == counts
