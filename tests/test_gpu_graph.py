"""The verify step captured as a HIP graph (as the benchmark runs it):
several replays, with eager work and synchronisations between them, each
checked against the eager result.  Attention and greedy acceptance keep
arrival counters in their workspaces, so replays also check that those
counters return to zero."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager():
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(L=3, ctx=900, H=1024, V=5000, cfg_id=300)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    tree = api.Tree(parent, rank, w.topk)
    hidden, w1, wlm = synth.head_inputs(w, DEV)
    root = synth.roots(w, DEV)
    ctx = torch.full((w.B,), w.ctx, dtype=torch.int32, device=DEV)
    layers = [synth.attention_inputs(w, l, DEV)[:3] for l in range(w.L)]
    base = synth.normal((w.B, w.T, w.V), 1.0, 7, DEV)
    logits = torch.empty((w.B, w.K, w.V), device=DEV)
    topk = torch.empty((w.B, w.K, tree.kmax), dtype=torch.int32, device=DEV)
    toks = torch.empty((w.B, w.T), dtype=torch.int32, device=DEV)
    pos = torch.empty((w.B, w.T), dtype=torch.int32, device=DEV)
    outs = [torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.bfloat16, device=DEV) for _ in range(w.L)]
    acc = (torch.empty(w.B, dtype=torch.int32, device=DEV),
           torch.empty((w.B, w.K + 1), dtype=torch.int32, device=DEV),
           torch.empty((w.B, w.K + 1), dtype=torch.int32, device=DEV))
    z = lambda n: torch.zeros(max(n, 256), dtype=torch.uint8, device=DEV)
    ws_h = z(api.heads_workspace_size(w.B, w.H, w.K, torch.bfloat16))
    ws_a = z(api.tree_attention_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.ctx, tree, torch.bfloat16))
    ws_c = z(api.accept_workspace_size(w.B, w.V, tree, 0.0))

    def step():
        api.heads(hidden, w1, wlm, logits=logits, ws=ws_h)
        api.tree_candidates(logits, root, ctx, tree, topk, toks, pos)
        for l, (q, k, v) in enumerate(layers):
            api.tree_attention(q, k, v, ctx, w.ctx, tree, out=outs[l], ws=ws_a)
        api.accept_paths(base, None, toks, tree, None, None, 0.0, outs=acc, ws=ws_c)

    def snapshot():
        return [x.clone() for x in [logits, topk, toks, pos, *outs, *acc]]

    announce("graph: eager reference")
    step()
    torch.cuda.synchronize()
    ref = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    announce("graph: capture")
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for x in [logits, topk, toks, pos, *outs, *acc]:
            x.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        announce("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), ref):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        step()                              # eager step between replays
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), ref):
            assert torch.equal(a, b), f"eager step after replay {rep} differs"
