"""Calls on two streams at once, each with its own workspace, compute exactly
what the same calls compute one after the other: no call keeps state on the
device between calls or shares it with another (tree attention at an MHA and
a grouped-query shape with split partials, and the dense-variant heads)."""
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("wl,hq,hkv", [("vicuna7b-shaped", 8, 8), ("zephyr7b-shaped", 32, 8)])
def test_attention_two_streams(wl, hq, hkv):
    w = synth.WORKLOADS[wl].scaled(B=2, Hq=hq, Hkv=hkv, ctx=1800, cfg_id=340)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    ins = [synth.attention_inputs(w, l, DEV, ctx_lens=[1800, 1111 + 97 * l]) for l in range(2)]
    nb = api.tree_attention_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.ctx, t, torch.bfloat16)
    announce("attention on two streams", wl)
    serial = [api.tree_attention(q, k, v, c, w.ctx, t) for (q, k, v, c) in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ws = [torch.zeros(max(nb, 256), dtype=torch.uint8, device=DEV) for _ in range(2)]
    outs = [torch.empty_like(ins[l][0]) for l in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for l in range(2):
            q, k, v, c = ins[l]
            with torch.cuda.stream(streams[l]):
                api.tree_attention(q, k, v, c, w.ctx, t, out=outs[l], ws=ws[l])
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(outs[l], serial[l]), (rep, l)


def test_heads_dense_two_streams():
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=2, H=512, V=3000, K=3, topk=(10, 5, 5), cfg_id=341)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    _, w1, wlm = synth.head_inputs(w, DEV)
    rows = [synth.normal((w.B * w.T, w.H), 1.0, synth.seed_for(w.cfg_id, synth.T_HIDDEN, 0, 1 + i), DEV,
                         torch.bfloat16) for i in range(2)]
    announce("dense heads on two streams")
    serial = [api.heads_dense(r, w1, wlm, t) for r in rows]
    torch.cuda.synchronize()
    M = w.B * w.T
    nb = api._lib.load().medusa_heads_dense_workspace_size(M, w.H, w.V, w.K, t.handle, 1)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ws = [torch.zeros(nb, dtype=torch.uint8, device=DEV) for _ in range(2)]
    outs = [(torch.empty((M, w.K, t.kmax), dtype=torch.int32, device=DEV),
             torch.empty((M, w.K, t.kmax), dtype=torch.float32, device=DEV)) for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                api.heads_dense(rows[i], w1, wlm, t, outs=outs[i], ws=ws[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i][0], serial[i][0]), (rep, i)
            assert torch.equal(outs[i][1], serial[i][1]), (rep, i)
