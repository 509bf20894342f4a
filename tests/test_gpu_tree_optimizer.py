"""GPU: a tree chosen by the static tree optimiser (medusa_tree_optimize)
taken through the device path against the oracle.

P2 (paper-results ablation) credits an optimised tree configuration with
part of Medusa's speed-up; P1 (tree-size trade-off) says the topology is
chosen by profiling.  Here an acceptance table is profiled on the toy target
(the oracle's greedy walk over a wide cost-ordered tree), the optimiser picks
a 12-node tree for it, and that tree is created on the device and run
through candidates -> tree attention -> acceptance for several steps of the
toy target: mask, top-k, tree tokens, positions and accepted paths bit-exact
(rejection-sampling decisions up to counted fp64 ties), attention within the
bf16 bound."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from oracle import accept as oaccept
from oracle import attention as oattn
from oracle import topk as otopk
from oracle import tree as otree
from helpers import TOL_BF16, announce, assert_same_decisions, row_rel_err, to64
from toy_model import RankedDrafts, ToyTarget, node_prefixes, simulate_accepts

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _optimised_tree(kpd, T):
    target = ToyTarget(V=61)
    drafts = RankedDrafts(hit=[0.95, 0.9, 0.85], q=0.3)
    wide_p, wide_r = synth.cost_ordered_tree(kpd, 30)
    _, tried, hits = simulate_accepts(target, drafts, wide_p, wide_r, kpd, 300, seed=1)
    p_hat = np.where(tried > 0, hits / np.maximum(tried, 1), 0.0)
    parent, rank, e = api.tree_optimize(p_hat, kpd, T)
    otree.validate(parent, rank, kpd)
    assert abs(otree.expected_accepted(parent, rank, p_hat) - e) < 1e-12
    return parent, rank


def test_optimised_tree_through_the_device_step():
    kpd, T, B, V = [4, 3, 3], 12, 3, 2048
    parent, rank = _optimised_tree(kpd, T)
    cp, _ = synth.cost_ordered_tree(kpd, T)
    announce("optimised tree", list(parent), "cost-ordered", list(cp))
    tree = api.Tree(parent, rank, kpd)
    vis = otree.visible_bruteforce(parent)
    assert (tree.mask() == otree.bitmask_rows(vis)).all()

    target = ToyTarget(V=V)
    drafts = RankedDrafts(hit=[0.95, 0.9, 0.85], q=0.3)
    rng = np.random.default_rng(7)
    seqs = [list(rng.integers(0, V, 5)) for _ in range(B)]
    roots = [int(np.argmax(target.logits(s))) for s in seqs]
    ctx = [700, 651, 512]
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=B, T=T, K=len(kpd), topk=tuple(kpd), V=V,
                                                   Hq=8, Hkv=2, ctx=max(ctx), cfg_id=610)
    K = len(kpd)
    accepted, rej_lens = [], []
    for step in range(4):
        heads = np.stack([
            synth.toy_draft_logits_ranked(target.greedy(seqs[b] + [roots[b]], K), V,
                                          drafts.ranks(rng, kpd), 1000 * step + b)
            for b in range(B)])
        announce("optimised tree step", step)
        tk, toks, pos = api.tree_candidates(torch.from_numpy(heads).to(DEV),
                                            torch.tensor(roots, dtype=torch.int32, device=DEV),
                                            torch.tensor(ctx, dtype=torch.int32, device=DEV), tree)
        torch.cuda.synchronize()
        r_tk = otopk.head_topk(heads, kpd)
        r_toks = otree.tree_tokens(r_tk, roots, parent, rank)
        assert (tk.cpu().numpy() == r_tk).all()
        assert (toks.cpu().numpy() == r_toks).all()
        assert (pos.cpu().numpy() == otree.positions(ctx, parent)).all()

        # one attention layer over ragged contexts on this tree's mask
        q, k, v, ctx_t = synth.attention_inputs(w, step, DEV, ctx_lens=ctx)
        out = api.tree_attention(q, k, v, ctx_t, max(ctx), tree)
        torch.cuda.synchronize()
        ref = oattn.tree_attention(to64(q), to64(k), to64(v), ctx, vis)
        assert row_rel_err(to64(out), ref) <= TOL_BF16

        # the target's logits after every tree node; greedy and rejection
        base = np.stack([np.stack([target.logits(p) for p in
                                   node_prefixes(seqs[b], roots[b], r_toks[b], parent)])
                         for b in range(B)]).astype(np.float32)
        base_d = torch.from_numpy(base).to(DEV)
        g = api.accept_paths(base_d, None, toks, tree, None, None, 0.0)
        torch.cuda.synchronize()
        r = oaccept.accept_paths(base, None, r_toks, parent, rank, None, None, 0.0, K)
        for x, y in zip(g, r[:3]):
            assert (x.cpu().numpy() == y).all()
        ua = synth.uniform((B, T), synth.seed_for(610, 1, step))
        us = synth.uniform((B, T), synth.seed_for(610, 2, step))
        # the target's logits sharpened (x30) so that rejection sampling
        # accepts some drafts (paths of length 0, 1 and 2 occur here)
        sharp = (30.0 * base).astype(np.float32)
        gr = api.accept_paths(torch.from_numpy(sharp).to(DEV), torch.from_numpy(heads).to(DEV),
                              toks, tree, ua.to(DEV), us.to(DEV), 1.0)
        torch.cuda.synchronize()
        rr = oaccept.accept_paths(sharp, heads, r_toks, parent, rank, ua.numpy(), us.numpy(), 1.0, K)
        assert_same_decisions(tuple(x.cpu().numpy() for x in gr), rr[:3], rr[3])
        rej_lens.extend(int(x) for x in rr[0])

        # commit the greedy result (the oracle's) and move on
        for b in range(B):
            n = int(r[0][b])
            accepted.append(n)
            seqs[b] = seqs[b] + [roots[b]] + [int(t) for t in r[1][b][:n]]
            roots[b] = int(r[1][b][n])
    assert max(accepted) >= 2      # the optimised tree's deeper nodes were reached
    assert max(rej_lens) >= 1      # and rejection sampling accepted along it
