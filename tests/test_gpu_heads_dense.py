"""GPU parity of medusa_heads_dense (the heads on every tree row, each head's
top-k) against the oracle.

The ranking is decided on the fp32 logits the kernel computes, so each case
also asks for those logits: they are checked against the oracle's fp64
logits within the dtype's tolerance, and the returned indices must equal,
bit for bit, the oracle's top-k of those same fp32 logits (descending, ties
to the lower index); the values must be those logits exactly, and the run
without the logits output must return the same top-k."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from oracle import dense_heads as odense
from oracle import heads as oheads
from oracle import topk as otopk
from helpers import TOL_BF16, TOL_F32, announce, row_rel_err, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tree(topk, T):
    parent, rank = synth.cost_ordered_tree(topk, T)
    return api.Tree(parent, rank, topk)


def _check(hidden, w1, wlm, t, topk, tol, round_r, full_oracle=True, sample_rows=None):
    M = hidden.shape[0]
    K = w1.shape[0]
    V = wlm.shape[-2]
    logits = torch.empty((M, K, V), dtype=torch.float32, device=DEV)
    idx, val = api.heads_dense(hidden, w1, wlm, t, logits=logits)
    idx2, val2 = api.heads_dense(hidden, w1, wlm, t)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(val, val2)
    g_logits = logits.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_val = val.cpu().numpy()
    # indices: the oracle's top-k of the kernel's own fp32 logits, bit for bit
    ref_idx = otopk.head_topk(g_logits, list(topk))
    assert (g_idx == ref_idx).all()
    # values: exactly those logits; padding 0
    for m in range(M):
        for d in range(K):
            kd = topk[d]
            assert (g_val[m, d, :kd] == g_logits[m, d, g_idx[m, d, :kd]]).all()
            assert (g_val[m, d, kd:] == 0).all()
    # logits against the fp64 oracle
    if full_oracle:
        ref_logits = oheads.medusa_heads(to64(hidden), to64(w1), to64(wlm), round_r=round_r)
        err = row_rel_err(g_logits.reshape(-1, V), ref_logits.reshape(-1, V))
        assert err <= tol, err
        # the oracle's own ranking where it is decided: the kernel ranks its
        # logits exactly (checked above) and they are within e_row of the
        # fp64 ones, so a position whose fp64 value is more than 2 e_row from
        # both neighbours in the ranking must hold the same index
        o_idx, _ = odense.dense_candidates(to64(hidden), to64(w1), to64(wlm), topk, round_r=round_r)
        e_row = np.max(np.abs(g_logits - ref_logits), axis=-1)
        checked = 0
        for m in range(M):
            for d in range(K):
                kd = topk[d]
                srt = np.sort(ref_logits[m, d])[::-1][:kd + 1]
                for j in range(kd):
                    lo = np.inf if j == 0 else srt[j - 1] - srt[j]
                    if min(lo, srt[j] - srt[j + 1]) > 2 * e_row[m, d]:
                        assert g_idx[m, d, j] == o_idx[m, d, j], (m, d, j)
                        checked += 1
        print(f"[dense ranking] {checked} of {M * sum(topk)} ranked positions decided in fp64",
              flush=True)
    else:
        # sampled (row, head) pairs: the oracle's residual block, then its
        # vocab product r @ W^T taken over chunks of the vocabulary
        h64 = to64(hidden)
        for (m, d) in sample_rows:
            r = oheads.residual_block(h64[m:m + 1], to64(w1[d]), round_r)[0]
            wd = wlm if wlm.dim() == 2 else wlm[d]
            ref = np.concatenate([to64(wd[v0:v0 + 4096]) @ r for v0 in range(0, V, 4096)])
            err = row_rel_err(g_logits[m, d][None], ref[None])
            assert err <= tol, (m, d, err)


def test_dense_tiny_fp32():
    w = synth.WORKLOADS["tiny-fp32"]
    M = w.B * w.T
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=M)
    t = _tree(w.topk, w.T)
    announce("dense heads tiny-fp32", M)
    _check(hidden, w1, wlm, t, w.topk, TOL_F32, round_r=False)


SMALL = [
    # (label, M, H, V, topk, shared)
    ("m64-v1000", 64, 256, 1000, (10, 5, 3), False),
    ("m200-ragged", 200, 256, 1000, (10, 10, 5), False),
    ("m16-shared", 16, 128, 512, (4, 4), True),
    ("m130-k32", 130, 128, 640, (32, 8), False),
    ("m1-k1", 1, 128, 256, (1, 1, 1), False),
    # 256-row tiles: rows past M in the second row tile, one ragged column
    # tile of 200, a head keeping one candidate next to one keeping twelve
    ("m300-v200", 300, 128, 200, (12, 1), False),
    # 313 tile lists per (row, head): more than the merge's 256 staged lists
    ("m16-v40000", 16, 128, 40000, (10, 4), False),
]


@pytest.mark.parametrize("label,M,H,V,topk,shared", SMALL, ids=[c[0] for c in SMALL])
def test_dense_bf16_small(label, M, H, V, topk, shared):
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=H, V=V, K=len(topk), topk=topk, T=8,
                                                  cfg_id=400 + len(label))
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=M, shared_lm_head=shared)
    T = min(1 + sum(np.cumprod(topk)), 60)
    t = _tree(topk, T)
    announce("dense heads bf16", label)
    _check(hidden, w1, wlm, t, topk, TOL_BF16, round_r=True)


def test_dense_ties_go_to_the_lower_index():
    """Duplicate vocab rows give identical fp32 logits (same products, same
    order); the lower index must come first."""
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=128, V=512, K=1, topk=(6,), T=7, cfg_id=430)
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=32)
    wlm[0, 300] = wlm[0, 17]
    wlm[0, 451] = wlm[0, 17]
    wlm[0, 129] = wlm[0, 400]
    t = _tree((6,), 7)
    announce("dense heads ties")
    logits = torch.empty((32, 1, 512), dtype=torch.float32, device=DEV)
    idx, _ = api.heads_dense(hidden, w1, wlm, t, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert (lg[:, 0, 300] == lg[:, 0, 17]).all() and (lg[:, 0, 451] == lg[:, 0, 17]).all()
    assert (idx.cpu().numpy() == otopk.head_topk(lg, [6])).all()


def test_dense_ties_large_tiles():
    """256-row tiles (M = 256): a large duplicated vocab row makes equal
    logits among each row's largest (within one 4-column granule, across
    tiles and in the ragged last tile), so the tile's ranking must order
    them by index whatever order they were gathered in; head 1 has one
    all-zero 256-column tile, which takes the general ranking path while the
    others do not."""
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=256, V=1000, K=2, topk=(10, 5), T=12,
                                                  cfg_id=435)
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=256)
    big = 4.0 * wlm[0, 17]
    for c in (17, 18, 300, 640, 999):
        wlm[0, c] = big
    wlm[1, 256:512] = 0
    t = _tree((10, 5), 12)
    announce("dense heads ties, 256-row tiles")
    _check(hidden, w1, wlm, t, (10, 5), TOL_BF16, round_r=True)
    logits = torch.empty((256, 2, 1000), dtype=torch.float32, device=DEV)
    idx, _ = api.heads_dense(hidden, w1, wlm, t, logits=logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert (lg[:, 0, 999] == lg[:, 0, 17]).all()
    top = idx[:, 0].cpu().numpy()
    pos = lg[:, 0, 17] >= lg[:, 0].max(axis=1)   # rows where the tied value is the largest
    assert pos.sum() > 20
    assert (top[pos, :5] == np.array([17, 18, 300, 640, 999])).all()


@pytest.mark.parametrize("name", ["vicuna7b-shaped", "vicuna13b-shaped", "vicuna33b-shaped", "zephyr7b-shaped"])
def test_dense_full_size(name):
    """M = B*T rows at the workload's shape; the oracle recomputes sampled
    (row, head) logit rows in full."""
    w = synth.WORKLOADS[name]
    M = w.B * w.T
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=M)
    t = _tree(w.topk, w.T)
    announce("dense heads full", name, M)
    rng = np.random.default_rng(w.cfg_id + 11)
    rows = [(0, 0), (M - 1, w.K - 1)] + [(int(rng.integers(M)), int(rng.integers(w.K))) for _ in range(2)]
    _check(hidden, w1, wlm, t, w.topk, TOL_BF16, round_r=True, full_oracle=False, sample_rows=rows)
    del hidden, w1, wlm
    torch.cuda.empty_cache()


def test_dense_argument_errors():
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=192, V=256, K=2, topk=(4, 2), T=7, cfg_id=440)
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=8)
    t = _tree((4, 2), 7)
    with pytest.raises(api.MedusaError) as e:            # bf16 needs H % 128 == 0
        api.heads_dense(hidden, w1, wlm, t)
    assert e.value.code == api.EINVAL
    t3 = _tree((4, 2, 2), 9)
    w2 = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=128, V=256, K=2, topk=(4, 2), T=7, cfg_id=441)
    hidden, w1, wlm = synth.head_inputs(w2, DEV, M=8)
    with pytest.raises(api.MedusaError) as e:            # K differs from the tree's
        api.heads_dense(hidden, w1, wlm, t3)
    assert e.value.code == api.EINVAL
    lib = api._lib.load()
    idx = torch.empty((8, 2, 4), dtype=torch.int32, device=DEV)
    ws = torch.zeros(256, dtype=torch.uint8, device=DEV)
    rc = lib.medusa_heads_dense(hidden.data_ptr(), w1.data_ptr(), 128 * 128, wlm.data_ptr(), 256 * 128,
                                8, 128, 256, 2, t.handle, api.BF16, idx.data_ptr(), None, None,
                                ws.data_ptr(), ws.numel(), None)
    assert rc == api.EWORKSPACE


@pytest.mark.parametrize("M", [64, 256])
def test_dense_heavy_ties(M):
    """Head 0's projection is zero (every logit exactly 0: the lowest indices
    win); head 1's vocab rows repeat with period 7 (every logit has exact
    duplicates).  Both tile shapes (M = 64 and M = 256)."""
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=128, V=1024, K=2, topk=(10, 10), T=12,
                                                  cfg_id=450 + M)
    hidden, w1, wlm = synth.head_inputs(w, DEV, M=M)
    wlm[0].zero_()
    wlm[1] = wlm[1][torch.arange(1024, device=DEV) % 7]
    t = _tree((10, 10), 12)
    announce("dense heads heavy ties", M)
    idx, _ = api.heads_dense(hidden, w1, wlm, t)
    torch.cuda.synchronize()
    assert (idx[:, 0].cpu().numpy() == np.arange(10)).all()
    _check(hidden, w1, wlm, t, (10, 10), TOL_BF16, round_r=True)


def test_dense_deterministic():
    """Two calls on the same inputs give identical indices, values and
    logits, on both tile shapes (M = 64 and M = 256)."""
    for M in (64, 256):
        w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=1, H=256, V=3000, K=3, topk=(10, 5, 3), T=16,
                                                      cfg_id=460 + M)
        hidden, w1, wlm = synth.head_inputs(w, DEV, M=M)
        t = _tree((10, 5, 3), 16)
        announce("dense heads determinism", M)
        runs = []
        for _ in range(2):
            logits = torch.empty((M, 3, 3000), dtype=torch.float32, device=DEV)
            idx, val = api.heads_dense(hidden, w1, wlm, t, logits=logits)
            runs.append((idx, val, logits))
        torch.cuda.synchronize()
        for a, b in zip(*runs):
            assert torch.equal(a, b)
