"""GPU parity of medusa_tree_attention_layers (every layer in one grid)
against the oracle, layer by layer: small shapes in full with strided layer
blocks, NaN-filled unused slots and ragged contexts; the workload shapes on
sampled (layer, b, node, head) rows; bit-identity with one call per layer at
the same split count; argument errors."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from oracle import attention as oattn
from oracle import tree as otree
from helpers import TOL_BF16, TOL_F32, announce, row_rel_err, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _stacked_inputs(w, L, S_cap=None, ctx_lens=None, pad=0):
    """[L,...] Q/K/V views whose layer blocks sit ``pad`` elements apart beyond
    their extent (pad=0: contiguous), layer l drawn with the layer-l seeds."""
    per = [synth.attention_inputs(w, l, DEV, S_cap=S_cap, ctx_lens=ctx_lens) for l in range(L)]
    ctx = per[0][3]

    def stack(i):
        one = per[0][i]
        n = one.numel()
        buf = torch.full((L, n + pad), float("nan"), dtype=one.dtype, device=DEV)
        for l in range(L):
            buf[l, :n] = per[l][i].reshape(-1)
        return buf[:, :n].view(L, *one.shape)

    q, k, v = stack(0), stack(1), stack(2)
    del per
    return q, k, v, ctx


def _check_layers_full(q, k, v, ctx, parent, out, tol):
    vis = otree.visible_bruteforce(parent)
    for l in range(q.shape[0]):
        ref = oattn.tree_attention(to64(q[l]), to64(k[l]), to64(v[l]), ctx.tolist(), vis)
        got = to64(out[l])
        assert np.all(np.isfinite(got)), l
        err = row_rel_err(got, ref)
        assert err <= tol, (l, err)


SMALL = [
    # (label, L, B, Hq, Hkv, tree(topk, T), ctx list, layer padding in elements)
    ("l3-mha", 3, 1, 4, 4, ((10, 10, 5, 5), 64), [300], 0),
    ("l4-gqa-ragged-padded", 4, 3, 8, 2, ((10, 10, 5, 5, 5), 64), [5, 77, 130], 24),
    ("l2-ctx0", 2, 2, 2, 2, ((4, 3, 2), 20), [0, 33], 8),
    ("l5-t96", 5, 1, 3, 3, ((10, 10, 5, 5), 96), [257], 0),
]


@pytest.mark.parametrize("label,L,B,Hq,Hkv,tr,ctx,pad", SMALL, ids=[c[0] for c in SMALL])
def test_layers_bf16_small_full(label, L, B, Hq, Hkv, tr, ctx, pad):
    topk, T = tr
    parent, rank = synth.cost_ordered_tree(topk, T)
    t = api.Tree(parent, rank, topk)
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=B, Hq=Hq, Hkv=Hkv, T=T, ctx=max(ctx),
                                                  cfg_id=300 + len(label))
    S_cap = max(ctx) + T + 3
    q, k, v, ctx_t = _stacked_inputs(w, L, S_cap=S_cap, ctx_lens=ctx, pad=pad)
    for b, c in enumerate(ctx):   # slots past ctx+T are never read
        k[:, b, :, c + T:] = float("nan")
        v[:, b, :, c + T:] = float("nan")
    announce("attention layers bf16", label)
    out_buf = torch.full((L, q[0].numel() + pad), float("nan"), dtype=q.dtype, device=DEV)
    out = out_buf[:, :q[0].numel()].view(q.shape)
    api.tree_attention_layers(q, k, v, ctx_t, max(ctx), t, out=out)
    torch.cuda.synchronize()
    _check_layers_full(q, k, v, ctx_t, parent, out, TOL_BF16)
    if pad:   # the gaps between layers are left alone
        assert torch.isnan(out_buf[:, q[0].numel():].float()).all()


def test_layers_fp32_small_full():
    w = synth.WORKLOADS["tiny-fp32"]
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    q, k, v, ctx = _stacked_inputs(w, 3, pad=4)
    announce("attention layers f32")
    out = api.tree_attention_layers(q, k, v, ctx, w.ctx, t)
    torch.cuda.synchronize()
    _check_layers_full(q, k, v, ctx, parent, out, TOL_F32)


@pytest.mark.parametrize("hq,hkv", [(8, 4), (16, 4)])
@pytest.mark.parametrize("splits", [1, 3, 11])
def test_layers_equal_per_layer_calls(splits, hq, hkv, monkeypatch):
    """At a fixed split count, one grid over L layers computes exactly what L
    single-layer calls compute (same arithmetic per query row)."""
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=2, Hq=hq, Hkv=hkv, ctx=900, cfg_id=320)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    L = 3
    q, k, v, ctx = _stacked_inputs(w, L, ctx_lens=[900, 411])
    monkeypatch.setenv("MEDUSA_ATTN_SPLITS", str(splits))
    announce("attention layers vs per-layer", splits)
    out = api.tree_attention_layers(q, k, v, ctx, w.ctx, t)
    for l in range(L):
        one = api.tree_attention(q[l], k[l], v[l], ctx, w.ctx, t)
        torch.cuda.synchronize()
        assert torch.equal(out[l], one), l


def test_layers_gqa_recomputed_pass_equal_per_layer(monkeypatch):
    """The one-workgroup-per-K/V-head kernel in one grid over layers when some
    workgroups recompute their split: layer 0's keys grow along the sequence
    (its first pass overflows, so its workgroups compute again checking every
    half), layer 1's are plain.  At a fixed split count each layer equals its
    single-layer call bit for bit, and layer 0 matches the oracle."""
    w = synth.WORKLOADS["zephyr7b-shaped"].scaled(B=2, ctx=1500, cfg_id=321)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    L = 2
    q, k, v, ctx = _stacked_inputs(w, L, ctx_lens=[1500, 1301])
    ramp = 1 + 47 * torch.arange(k.shape[3], device=DEV, dtype=torch.float32) / k.shape[3]
    k[0] = (k[0].float() * ramp[None, None, :, None]).to(torch.bfloat16)
    monkeypatch.setenv("MEDUSA_ATTN_SPLITS", "2")
    announce("attention layers, recomputed first pass")
    out = api.tree_attention_layers(q, k, v, ctx, w.ctx, t)
    for l in range(L):
        one = api.tree_attention(q[l], k[l], v[l], ctx, w.ctx, t)
        torch.cuda.synchronize()
        assert torch.equal(out[l], one), l
    vis = otree.visible_bruteforce(parent)
    ref = oattn.tree_attention(to64(q[0]), to64(k[0]), to64(v[0]), ctx.tolist(), vis)
    got = to64(out[0])
    assert np.all(np.isfinite(got))
    assert row_rel_err(got, ref) <= TOL_BF16


@pytest.mark.parametrize("name", ["vicuna7b-shaped", "vicuna13b-shaped", "zephyr7b-shaped"])
def test_layers_full_size_sampled_rows(name):
    """Every layer of the workload in one call, in the planner's own split
    count; the oracle recomputes sampled (layer, b, node, head) rows."""
    w = synth.WORKLOADS[name]
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    ctx_lens = [w.ctx - 5 * b for b in range(w.B)]
    q, k, v, ctx = _stacked_inputs(w, w.L, ctx_lens=ctx_lens)
    announce("attention layers full", name, w.L)
    out = api.tree_attention_layers(q, k, v, ctx, w.ctx, t)
    torch.cuda.synchronize()
    vis = otree.visible_bruteforce(parent)
    rng = np.random.default_rng(w.cfg_id + 7)
    layers = sorted({0, w.L - 1, *[int(x) for x in rng.integers(w.L, size=4)]})
    for l in layers:
        samples = [(int(rng.integers(w.B)), int(rng.integers(w.T)), int(rng.integers(w.Hq)))
                   for _ in range(8)]
        samples += [(0, 0, 0), (w.B - 1, w.T - 1, w.Hq - 1)]
        cache = {}

        def fetch(b, g, n):
            if (b, g) not in cache:
                cache[(b, g)] = (to64(k[l, b, g, :n]), to64(v[l, b, g, :n]))
            return cache[(b, g)]

        ref = oattn.tree_attention_rows([to64(q[l][s]) for s in samples], fetch, ctx_lens, vis,
                                        1 / np.sqrt(w.D), w.T, w.Hq // w.Hkv, samples)
        got = np.stack([to64(out[l][s]) for s in samples])
        err = row_rel_err(got, ref)
        assert err <= TOL_BF16, (l, err)
    del q, k, v, out
    torch.cuda.empty_cache()


def test_layers_argument_errors():
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, Hq=4, Hkv=4, ctx=64, cfg_id=330)
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    t = api.Tree(parent, rank, w.topk)
    lib = api._lib.load()
    q = torch.zeros((2, 1, w.T, 4, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((2, 1, 4, 64 + w.T, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(q)
    ctx = torch.tensor([64], dtype=torch.int32, device=DEV)
    nb = api.tree_attention_layers_workspace_size(2, 1, 4, 4, 128, 64, t, torch.bfloat16)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=DEV)

    def call(L, qs, kvs, os_):
        return lib.medusa_tree_attention_layers(
            q.data_ptr(), kv.data_ptr(), kv.data_ptr(), qs, kvs, os_, L, ctx.data_ptr(), 64,
            t.handle, 1, 4, 4, 128, 64 + w.T, 0.1, api.BF16, out.data_ptr(), ws.data_ptr(),
            ws.numel(), None)

    qs, kvs = q.stride(0), kv.stride(0)
    assert call(0, qs, kvs, qs) == api.EINVAL               # no layers
    assert call(2, qs - 8, kvs, qs) == api.EINVAL           # q layers overlap
    assert call(2, qs, kvs - 8, qs) == api.EINVAL           # cache layers overlap
    assert call(2, qs, kvs, qs + 3) == api.EINVAL           # breaks 16-byte alignment
    assert call(2, qs, kvs, qs) == api.OK
    torch.cuda.synchronize()
