"""CPU checks of the Python binding's argument validation: a tensor whose
shape or dtype does not match what a call assumes, or one in host memory, is
rejected with ValueError before anything reaches the library (a kernel given a
tensor smaller than the tree or the other operands would read or write past
its end).  No device is touched: the tree is a stand-in with the handle's
attributes, and every case fails before the library call."""
import types

import pytest
import torch

from medusa_tree_verification_amd import api

TREE = types.SimpleNamespace(T=8, K=3, kmax=2, W=1, handle=None)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def bf16(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def test_heads_shape_and_dtype_mismatches():
    with pytest.raises(ValueError, match="w1"):
        api.heads(bf16(2, 64), bf16(3, 64, 32), bf16(3, 100, 64))      # W1 not [K,H,H]
    with pytest.raises(ValueError, match="wlm"):
        api.heads(bf16(2, 64), bf16(3, 64, 64), bf16(3, 100, 32))      # W_lm rows of the wrong width
    with pytest.raises(ValueError, match="w1"):
        api.heads(bf16(2, 64), f32(3, 64, 64), bf16(3, 100, 64))       # mixed dtypes
    with pytest.raises(ValueError, match="hidden"):
        api.heads(torch.zeros((2, 64), dtype=torch.float16), bf16(3, 64, 64), bf16(3, 100, 64))
    with pytest.raises(ValueError, match="logits"):
        api.heads(bf16(2, 64), bf16(3, 64, 64), bf16(100, 64), logits=f32(2, 3, 99))
    with pytest.raises(ValueError, match="device memory"):
        api.heads(bf16(2, 64), bf16(3, 64, 64), bf16(100, 64))         # host tensors


def test_candidates_mismatches():
    with pytest.raises(ValueError, match="head_logits"):
        api.tree_candidates(f32(2, 2, 50), i32(2), i32(2), TREE)       # K differs from the tree's
    with pytest.raises(ValueError, match="root"):
        api.tree_candidates(f32(2, 3, 50), i32(1), i32(2), TREE)
    with pytest.raises(ValueError, match="ctx_len"):
        api.tree_candidates(f32(2, 3, 50), i32(2), f32(2), TREE)
    with pytest.raises(ValueError, match="device memory"):
        api.tree_candidates(f32(2, 3, 50), i32(2), i32(2), TREE)


def test_attention_mismatches():
    kv = bf16(1, 2, 64, 128)
    ctx = i32(1)
    with pytest.raises(ValueError, match="q"):
        api.tree_attention(bf16(1, 7, 4, 128), kv, kv, ctx, 32, TREE)  # T differs from the tree's
    with pytest.raises(ValueError, match="k_cache"):
        api.tree_attention(bf16(1, 8, 4, 128), f32(1, 2, 64, 128), kv, ctx, 32, TREE)
    with pytest.raises(ValueError, match="v_cache"):
        api.tree_attention(bf16(1, 8, 4, 128), kv, bf16(1, 2, 63, 128), ctx, 32, TREE)
    with pytest.raises(ValueError, match="ctx_len"):
        api.tree_attention(bf16(1, 8, 4, 128), kv, kv, i32(2), 32, TREE)
    with pytest.raises(ValueError, match="out"):
        api.tree_attention(bf16(1, 8, 4, 128), kv, kv, ctx, 32, TREE, out=bf16(1, 8, 4, 64))
    with pytest.raises(ValueError, match="device memory"):
        api.tree_attention(bf16(1, 8, 4, 128), kv, kv, ctx, 32, TREE)
    kvl = bf16(3, 1, 2, 64, 128)
    with pytest.raises(ValueError, match="k_cache"):
        api.tree_attention_layers(bf16(2, 1, 8, 4, 128), kvl, kvl, ctx, 32, TREE)  # L differs


def test_accept_mismatches():
    base = f32(2, 8, 50)
    toks = i32(2, 8)
    with pytest.raises(ValueError, match="base_logits"):
        api.accept_paths(f32(2, 7, 50), None, toks, TREE, None, None, 0.0)
    with pytest.raises(ValueError, match="head_logits"):
        api.accept_paths(base, f32(2, 3, 49), toks, TREE, f32(2, 8), f32(2, 8), 1.0)
    with pytest.raises(ValueError, match="tree_tokens"):
        api.accept_paths(base, None, i32(2, 9), TREE, None, None, 0.0)
    with pytest.raises(ValueError, match="u_accept"):
        api.accept_paths(base, f32(2, 3, 50), toks, TREE, f32(2, 7), f32(2, 8), 1.0)
    with pytest.raises(ValueError, match="out_tokens"):
        api.accept_paths(base, None, toks, TREE, None, None, 0.0,
                         outs=(i32(2), i32(2, 3), i32(2, 4)))
    with pytest.raises(ValueError, match="device memory"):
        api.accept_paths(base, None, toks, TREE, None, None, 0.0)


def test_commit_mismatches():
    k = bf16(2, 1, 2, 64, 128)
    with pytest.raises(ValueError, match="v_cache"):
        api.commit_accepted(k, bf16(2, 1, 2, 32, 128), i32(1), i32(1, 4), i32(1, 4), i32(1), TREE)
    with pytest.raises(ValueError, match="out_nodes"):
        api.commit_accepted(k, k.clone(), i32(1), i32(1, 3), i32(1, 4), i32(1), TREE)
    with pytest.raises(ValueError, match="accept_len"):
        api.commit_accepted(k, k.clone(), i32(2), i32(1, 4), i32(1, 4), i32(1), TREE)
    with pytest.raises(ValueError, match="device memory"):
        api.commit_accepted(k, k.clone(), i32(1), i32(1, 4), i32(1, 4), i32(1), TREE)


def test_probe_rejects_host_memory():
    with pytest.raises(ValueError):
        api.read_probe(torch.zeros(64, dtype=torch.int32))
