"""Pins for the tree-attention oracle: the path-causal alternative definition
(every root-to-leaf path run as an ordinary causal sequence), torch's own
scaled_dot_product_attention with a boolean mask (an independent library
implementation), and special cases.  A wrong mask direction, a missing
context, a wrong GQA group or a wrong scale fails at least one of them."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import synth
from oracle import attention, tree


def _inputs(rng, B, T, Hq, Hkv, D, ctx, extra=3):
    S_cap = ctx + T + extra
    q = rng.normal(size=(B, T, Hq, D))
    k = rng.normal(size=(B, Hkv, S_cap, D))
    v = rng.normal(size=(B, Hkv, S_cap, D))
    return q, k, v


CASES = [
    # (tree, B, Hq, Hkv, D, ctx_lens)
    ("cost8", 1, 4, 4, 16, [12]),
    ("random30", 2, 4, 2, 8, [5, 9]),
    ("chain6", 1, 2, 1, 8, [0]),
    ("cart232", 2, 6, 3, 8, [7, 0]),
    ("random30", 1, 8, 1, 4, [3]),
]


def _tree(name):
    if name == "cost8":
        return synth.cost_ordered_tree((2, 2, 2), 8)
    if name == "random30":
        return synth.random_tree(30, (4, 3, 3, 2), 11)
    if name == "chain6":
        return synth.chain_tree(5)
    if name == "cart232":
        return synth.cartesian_tree((2, 3, 2))
    raise KeyError(name)


@pytest.mark.parametrize("case", CASES)
def test_tree_attention_equals_path_causal(case):
    name, B, Hq, Hkv, D, ctx = case
    parent, _ = _tree(name)
    T = len(parent)
    rng = np.random.default_rng(CASES.index(case))
    q, k, v = _inputs(rng, B, T, Hq, Hkv, D, max(ctx))
    vis = tree.visible_bruteforce(parent)
    a = attention.tree_attention(q, k, v, ctx, vis)
    b = attention.path_causal_attention(q, k, v, ctx, parent)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_tree_attention_equals_torch_sdpa(case):
    name, B, Hq, Hkv, D, ctx = case
    parent, _ = _tree(name)
    T = len(parent)
    rng = np.random.default_rng(100 + CASES.index(case))
    q, k, v = _inputs(rng, B, T, Hq, Hkv, D, max(ctx))
    vis = tree.visible_bruteforce(parent)
    got = attention.tree_attention(q, k, v, ctx, vis)
    G = Hq // Hkv
    for b in range(B):
        c = ctx[b]
        mask = torch.from_numpy(np.concatenate([np.ones((T, c), bool), vis], axis=1))
        for h in range(Hq):
            qq = torch.from_numpy(q[b, :, h])[None]
            kk = torch.from_numpy(k[b, h // G, :c + T])[None]
            vv = torch.from_numpy(v[b, h // G, :c + T])[None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)[0]
            np.testing.assert_allclose(got[b, :, h], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_single_node_tree_is_plain_decode_attention():
    rng = np.random.default_rng(3)
    q, k, v = _inputs(rng, 1, 1, 2, 2, 16, 20)
    got = attention.tree_attention(q, k, v, [20], np.ones((1, 1), bool))
    for h in range(2):
        s = (k[0, h, :21] @ q[0, 0, h]) / 4.0
        p = np.exp(s - s.max())
        np.testing.assert_allclose(got[0, 0, h], (p / p.sum()) @ v[0, h, :21], rtol=1e-13)


def test_chain_tree_is_causal_attention():
    rng = np.random.default_rng(4)
    parent, _ = synth.chain_tree(6)
    T = 7
    q, k, v = _inputs(rng, 1, T, 1, 1, 8, 10)
    got = attention.tree_attention(q, k, v, [10], tree.visible_bruteforce(parent))
    # causal attention over the whole 17-token sequence; only the last 7 queries matter
    qs = np.concatenate([np.zeros((10, 8)), q[0, :, 0]])
    ref = attention.causal_attention(qs, k[0, 0, :17], v[0, 0, :17], 1 / np.sqrt(8))
    np.testing.assert_allclose(got[0, :, 0], ref[10:], rtol=1e-12)


def test_identical_value_rows_give_that_row():
    rng = np.random.default_rng(5)
    parent, _ = synth.random_tree(20, (4, 3, 2), 2)
    q, k, v = _inputs(rng, 1, 20, 2, 1, 8, 9)
    v[:] = rng.normal(size=8)
    got = attention.tree_attention(q, k, v, [9], tree.visible_bruteforce(parent))
    np.testing.assert_allclose(got, np.broadcast_to(v[0, 0, 0], got.shape), rtol=1e-13)


def test_pure_tree_root_sees_only_itself():
    rng = np.random.default_rng(6)
    parent, _ = synth.cost_ordered_tree((3, 2), 6)
    q, k, v = _inputs(rng, 1, 6, 1, 1, 4, 0)
    got = attention.tree_attention(q, k, v, [0], tree.visible_bruteforce(parent))
    np.testing.assert_allclose(got[0, 0, 0], v[0, 0, 0], rtol=1e-14)


def test_sibling_permutation_permutes_outputs():
    """Swapping two sibling subtrees (renumbered consistently) permutes the
    outputs the same way: the mask only depends on ancestry."""
    rng = np.random.default_rng(7)
    parent = [-1, 0, 0, 1, 2]
    perm = [0, 2, 1, 4, 3]                    # swap nodes 1<->2 and their children 3<->4
    parent2 = [-1, 0, 0, 1, 2]                # same shape after relabelling
    T, c = 5, 6
    q, k, v = _inputs(rng, 1, T, 2, 2, 8, c, extra=0)
    q2 = q[:, perm]
    k2, v2 = k.copy(), v.copy()
    k2[:, :, c:] = k[:, :, c:][:, :, perm]
    v2[:, :, c:] = v[:, :, c:][:, :, perm]
    a = attention.tree_attention(q, k, v, [c], tree.visible_bruteforce(parent))
    b = attention.tree_attention(q2, k2, v2, [c], tree.visible_bruteforce(parent2))
    np.testing.assert_allclose(b, a[:, perm], rtol=1e-13)


def test_rows_variant_matches_full():
    rng = np.random.default_rng(8)
    parent, _ = synth.random_tree(12, (3, 3, 2), 4)
    q, k, v = _inputs(rng, 2, 12, 4, 2, 8, 7)
    vis = tree.visible_bruteforce(parent)
    ctx = [7, 3]
    full = attention.tree_attention(q, k, v, ctx, vis)
    samples = [(0, 3, 1), (1, 11, 3), (1, 0, 0)]
    got = attention.tree_attention_rows([q[s] for s in samples],
                                        lambda b, g, n: (k[b, g, :n], v[b, g, :n]),
                                        ctx, vis, 1 / np.sqrt(8), 12, 2, samples)
    np.testing.assert_allclose(got, [full[s] for s in samples], rtol=1e-13)
