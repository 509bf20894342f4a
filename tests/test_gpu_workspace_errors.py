"""Workspace errors of the calls that take one (tree attention with split
partials, candidates, acceptance): a workspace that is too small or not
256-byte aligned is refused on the host with MEDUSA_EWORKSPACE before any
launch, the message names the bytes needed, and the same call then succeeds
with a proper workspace (no state is left behind)."""
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _refused(fn, need):
    with pytest.raises(api.MedusaError) as e:
        fn(torch.zeros(16, dtype=torch.uint8, device=DEV))
    assert e.value.code == api.EWORKSPACE
    assert str(need).encode() in api._lib.load().medusa_last_error()
    big = torch.zeros(need + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(api.MedusaError) as e:  # large enough but 256-byte misaligned
        fn(big[16:16 + need])
    assert e.value.code == api.EWORKSPACE
    fn(torch.zeros(need, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()


def test_attention_workspace_refused(monkeypatch):
    w = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=2, ctx=700, cfg_id=330)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    q, k, v, ctx = synth.attention_inputs(w, 0, DEV)
    monkeypatch.setenv("MEDUSA_ATTN_SPLITS", "4")
    need = api.tree_attention_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.ctx, t, torch.bfloat16)
    assert need > 0
    announce("attention workspace errors")
    _refused(lambda ws: api.tree_attention(q, k, v, ctx, w.ctx, t, ws=ws), need)


def test_candidates_workspace_refused():
    w = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=2, cfg_id=331)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    logits = torch.randn((w.B, w.K, w.V), device=DEV)
    root = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    ctx = torch.full((w.B,), 100, dtype=torch.int32, device=DEV)
    need = api.tree_candidates_workspace_size(w.B, w.V, t)
    assert need > 0
    announce("candidates workspace errors")
    _refused(lambda ws: api.tree_candidates(logits, root, ctx, t, ws=ws), need)


@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_accept_workspace_refused(tau):
    w = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=2, cfg_id=332)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    toks = synth.tree_tokens_input(w, parent)
    base, head, ua, us = synth.accept_inputs(w, parent, toks, DEV)
    toks = torch.from_numpy(toks).to(DEV)
    need = api.accept_workspace_size(w.B, w.V, t, tau)
    assert need > 0
    announce("acceptance workspace errors", tau)
    _refused(lambda ws: api.accept_paths(base, head, toks, t, ua, us, tau, ws=ws), need)
