"""GPU: medusa_tree_attention_noalloc (split partials in the library's fixed
per-device scratch, for callers that cannot allocate) against
medusa_tree_attention with a caller's workspace, through the C ABI.

Both run the same kernels and launch plan, so the outputs must be equal bit
for bit; two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents), and the smaller one also against the
oracle.  A request whose partials exceed the scratch is rejected before
anything runs."""
import ctypes

import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from oracle import attention as oattn
from oracle import tree as otree
from helpers import TOL_BF16, announce, row_rel_err, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc_c(q, k, v, ctx, ctx_max, tree, out):
    """The entry point called through the C ABI directly (no binding logic)."""
    lib = api._lib.load()
    B, T, Hq, D = q.shape
    Hkv, S_cap = k.shape[1], k.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.medusa_tree_attention_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(ctx.data_ptr()), ctx_max, tree.handle, B, Hq, Hkv, D, S_cap,
        float(1.0 / np.sqrt(D)), api.BF16, ctypes.c_void_p(out.data_ptr()), stream)


def _case(w, ctx_lens, seed_layer):
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    tree = api.Tree(parent, rank, w.topk)
    q, k, v, ctx = synth.attention_inputs(w, seed_layer, DEV, ctx_lens=ctx_lens)
    return parent, tree, q, k, v, ctx


def test_noalloc_equals_workspace_call_twice_second_smaller():
    big = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=4, ctx=6000, cfg_id=800)
    small = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=2, Hq=8, Hkv=2, ctx=900, cfg_id=801)
    for label, w, ctx_lens in (("big", big, [6000, 5900, 4000, 17]), ("small", small, [900, 333])):
        parent, tree, q, k, v, ctx = _case(w, ctx_lens, 0)
        need = api.tree_attention_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.ctx, tree, torch.bfloat16)
        assert 0 < need <= api.ATTENTION_SCRATCH_BYTES, need   # the call really uses the scratch
        announce("noalloc attention", label, "partials", need)
        ref_out = api.tree_attention(q, k, v, ctx, w.ctx, tree)
        out = torch.empty_like(q)
        rc = _noalloc_c(q, k, v, ctx, w.ctx, tree, out)
        torch.cuda.synchronize()
        assert rc == api.OK, api._lib.load().medusa_last_error()
        assert torch.equal(out, ref_out), label
        if label == "small":
            vis = otree.visible_bruteforce(parent)
            ref = oattn.tree_attention(to64(q), to64(k), to64(v), ctx_lens, vis)
            assert row_rel_err(to64(out), ref) <= TOL_BF16


def test_noalloc_binding_and_f32_path():
    w = synth.WORKLOADS["tiny-fp32"].scaled(B=2, cfg_id=802)
    parent, tree, q, k, v, ctx = _case(w, [128, 40], 0)
    announce("noalloc attention fp32")
    a = api.tree_attention(q, k, v, ctx, w.ctx, tree)
    b = api.tree_attention_noalloc(q, k, v, ctx, w.ctx, tree)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_rejects_partials_beyond_the_scratch(monkeypatch):
    w = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=8, ctx=4096, cfg_id=803)
    parent, tree, q, k, v, ctx = _case(w, [4096] * 8, 0)
    monkeypatch.setenv("MEDUSA_ATTN_SPLITS", "64")      # 64 splits: far more partials than fit
    need = api.tree_attention_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.ctx, tree, torch.bfloat16)
    assert need > api.ATTENTION_SCRATCH_BYTES
    out = torch.zeros_like(q)
    announce("noalloc attention too large", need)
    rc = _noalloc_c(q, k, v, ctx, w.ctx, tree, out)
    torch.cuda.synchronize()
    assert rc == api.EWORKSPACE
    assert b"scratch" in api._lib.load().medusa_last_error()
    assert not out.any()                                 # nothing was enqueued
