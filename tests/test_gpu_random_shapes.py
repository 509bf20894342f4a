"""Seeded random shapes through the C ABI against the oracle, beside the
hand-picked cases of the per-call tests:

- tree attention: random topologies (1..5 heads, 1..8 candidates per depth,
  up to 140 nodes), ragged context lengths (0..600), every GQA ratio in
  {1, 2, 3, 5, 8}, cache slack, ctx_max above or below the largest context,
  bf16 and fp32; cache slots past each sequence are NaN, so any read beyond
  the sequence shows;
- tree attention score ranges: random bf16 shapes whose keys are scaled so
  that later scores rise far above, fall far below or spike above those of
  a split's first block, at forced split counts;
- candidates: random vocabulary sizes (from the largest k up to 70000),
  1..6 heads keeping 1..32 candidates, some logits drawn from a handful of
  values so that ties are everywhere;
- heads: random M (1..70), H, V, K, shared or per-head vocab projection,
  bf16 and fp32.
Every configuration is printed before it runs."""
import os

import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from oracle import attention as oattn
from oracle import heads as oheads
from oracle import topk as otopk
from oracle import tree as otree
from helpers import TOL_BF16, TOL_F32, announce, row_rel_err, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _random_tree(rng, max_T=140):
    K = int(rng.integers(1, 6))
    topk = tuple(int(x) for x in rng.integers(1, 9, size=K))
    cap = 1 + int(sum(np.prod(topk[:d + 1]) for d in range(K)))
    T = int(rng.integers(1, min(cap, max_T) + 1))
    parent, rank = synth.random_tree(T, topk, int(rng.integers(1 << 30)))
    return topk, T, parent, rank


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_shapes(seed):
    rng = np.random.default_rng(9000 + seed)
    topk, T, parent, rank = _random_tree(rng)
    bf16 = seed % 4 != 3
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 5, 8]))
    D = 128 if bf16 else int(rng.choice([32, 64, 128]))
    ctx = [int(x) for x in rng.integers(0, 601, size=B)]
    ctx_max = max(ctx) + int(rng.integers(-40, 80))
    ctx_max = max(ctx_max, 0)
    S_cap = max(ctx_max, max(ctx)) + T + int(rng.integers(0, 20))
    w = synth.WORKLOADS["vicuna7b-shaped" if bf16 else "tiny-fp32"].scaled(
        B=B, Hq=G * Hkv, Hkv=Hkv, D=D, T=T, K=len(topk), topk=topk, ctx=max(ctx), cfg_id=600 + seed)
    announce("attention random", seed, dict(B=B, Hkv=Hkv, G=G, D=D, T=T, topk=topk, ctx=ctx,
                                            ctx_max=ctx_max, S_cap=S_cap, bf16=bf16))
    tree = api.Tree(parent, rank, topk)
    q, k, v, ctx_t = synth.attention_inputs(w, 0, DEV, S_cap=S_cap, ctx_lens=ctx)
    for b, c in enumerate(ctx):
        k[b, :, c + T:] = float("nan")
        v[b, :, c + T:] = float("nan")
    out = api.tree_attention(q, k, v, ctx_t, ctx_max, tree)
    torch.cuda.synchronize()
    ref = oattn.tree_attention(to64(q), to64(k), to64(v), ctx, otree.visible_bruteforce(parent))
    got = to64(out)
    assert np.all(np.isfinite(got))
    assert row_rel_err(got.reshape(-1, D), ref.reshape(-1, D)) <= (TOL_BF16 if bf16 else TOL_F32)


@pytest.mark.parametrize("seed", range(24))
def test_attention_random_score_ranges(seed):
    """Random bf16 shapes (grouped-query ones with more than 128 query rows
    per K/V head among them) whose keys are scaled along the sequence: rising
    (later scores far above the first block's: the one-workgroup-per-head
    kernel keeps its first pass or computes the split again), falling (the
    reference stays high, later probabilities are small) or a few spiked
    keys anywhere; forced split counts put the jumps inside and across
    splits."""
    rng = np.random.default_rng(9500 + seed)
    topk, T, parent, rank = _random_tree(rng, max_T=100)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 4, 8]))
    ctx = [int(x) for x in rng.integers(0, 1500, size=B)]
    S_cap = max(ctx) + T + int(rng.integers(0, 20))
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(
        B=B, Hq=G * Hkv, Hkv=Hkv, T=T, K=len(topk), topk=topk, ctx=max(ctx), cfg_id=700 + seed)
    kind = ("rise", "fall", "spike")[seed % 3]
    f = float(rng.uniform(2, 60))
    splits = int(rng.choice([0, 1, 2, 5]))
    announce("attention random score ranges", seed, dict(B=B, Hkv=Hkv, G=G, T=T, ctx=ctx, kind=kind,
                                                          f=round(f, 1), splits=splits))
    tree = api.Tree(parent, rank, topk)
    q, k, v, ctx_t = synth.attention_inputs(w, 0, DEV, S_cap=S_cap, ctx_lens=ctx)
    pos = torch.arange(S_cap, device=DEV, dtype=torch.float32) / S_cap
    if kind == "rise":
        scale = 1 + (f - 1) * pos
    elif kind == "fall":
        scale = f - (f - 1) * pos
    else:
        scale = torch.ones(S_cap, device=DEV)
        scale[torch.from_numpy(rng.integers(0, S_cap, size=3)).to(DEV)] = f
    k = (k.float() * scale[None, None, :, None]).to(torch.bfloat16).contiguous()
    for b, c in enumerate(ctx):
        k[b, :, c + T:] = float("nan")
        v[b, :, c + T:] = float("nan")
    if splits:
        os.environ["MEDUSA_ATTN_SPLITS"] = str(splits)
    try:
        out = api.tree_attention(q, k, v, ctx_t, max(ctx), tree)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("MEDUSA_ATTN_SPLITS", None)
    ref = oattn.tree_attention(to64(q), to64(k), to64(v), ctx, otree.visible_bruteforce(parent))
    got = to64(out)
    assert np.all(np.isfinite(got))
    assert row_rel_err(got.reshape(-1, 128), ref.reshape(-1, 128)) <= TOL_BF16


@pytest.mark.parametrize("seed", range(16))
def test_candidates_random_shapes(seed):
    rng = np.random.default_rng(9100 + seed)
    K = int(rng.integers(1, 7))
    topk = tuple(int(x) for x in rng.integers(1, 33, size=K))
    cap = 1 + int(sum(np.prod(topk[:d + 1], dtype=np.float64) for d in range(K)))
    T = int(rng.integers(1, min(cap, 200) + 1))
    parent, rank = synth.random_tree(T, topk, int(rng.integers(1 << 30)))
    B = int(rng.integers(1, 5))
    V = int(rng.integers(max(topk), 70001))
    tied = seed % 3 == 0
    announce("candidates random", seed, dict(B=B, K=K, topk=topk, T=T, V=V, tied=tied))
    tree = api.Tree(parent, rank, topk)
    x = rng.normal(size=(B, K, V)).astype(np.float32)
    if tied:
        x = np.round(x * 2.0).astype(np.float32)   # a handful of distinct values
    root = rng.integers(0, V, size=B).astype(np.int32)
    ctx = rng.integers(0, 5000, size=B).astype(np.int32)
    tk, toks, pos = api.tree_candidates(torch.from_numpy(x).to(DEV), torch.from_numpy(root).to(DEV),
                                        torch.from_numpy(ctx).to(DEV), tree)
    torch.cuda.synchronize()
    r_tk = otopk.head_topk(x, list(topk))
    assert (tk.cpu().numpy() == r_tk).all()
    assert (toks.cpu().numpy() == otree.tree_tokens(r_tk, root, parent, rank)).all()
    assert (pos.cpu().numpy() == otree.positions(ctx, parent)).all()


@pytest.mark.parametrize("seed", range(12))
def test_heads_random_shapes(seed):
    rng = np.random.default_rng(9200 + seed)
    bf16 = seed % 3 != 2
    M = int(rng.integers(1, 71))
    H = 8 * int(rng.integers(1, 129))
    V = int(rng.integers(1, 5001))
    K = int(rng.integers(1, 6))
    shared = seed % 4 == 1
    w = synth.WORKLOADS["vicuna7b-shaped" if bf16 else "tiny-fp32"].scaled(
        B=M, H=H, V=V, K=K, topk=(1,) * K, cfg_id=700 + seed)
    announce("heads random", seed, dict(M=M, H=H, V=V, K=K, shared=shared, bf16=bf16))
    hidden, w1, wlm = synth.head_inputs(w, DEV, shared_lm_head=shared)
    logits = api.heads(hidden, w1, wlm)
    torch.cuda.synchronize()
    wlm_ref = to64(wlm)
    if shared:
        wlm_ref = np.broadcast_to(wlm_ref, (K,) + wlm_ref.shape)
    ref = oheads.medusa_heads(to64(hidden), to64(w1), wlm_ref, round_r=bf16)
    err = row_rel_err(logits.cpu().numpy().reshape(-1, V), ref.reshape(-1, V))
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err
