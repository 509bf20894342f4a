"""GPU parity of medusa_tree_create and medusa_heads against the oracle."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api, synth
from oracle import heads as oheads
from oracle import tree as otree
from helpers import TOL_BF16, TOL_F32, announce, row_rel_err, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_tree_upload_and_mask(name):
    w = synth.WORKLOADS[name]
    parent, rank = synth.cost_ordered_tree(w.topk, w.T)
    announce("tree_create", name)
    t = api.Tree(parent, rank, w.topk)
    assert (t.T, t.K, t.kmax) == (w.T, w.K, max(w.topk))
    np.testing.assert_array_equal(t.mask(), otree.bitmask_rows(otree.visible_bruteforce(parent)))


def test_heads_tiny_fp32_full():
    w = synth.WORKLOADS["tiny-fp32"]
    hidden, w1, wlm = synth.head_inputs(w, DEV)
    announce("heads tiny-fp32")
    got = api.heads(hidden, w1, wlm)
    torch.cuda.synchronize()
    ref = oheads.medusa_heads(to64(hidden), to64(w1), to64(wlm), round_r=False)
    assert row_rel_err(to64(got), ref) <= TOL_F32


SMALL_BF16 = [
    # (M, H, V, K, shared)
    (1, 512, 3000, 4, False),
    (3, 1024, 2050, 3, False),      # V not a multiple of 4 -> scalar stores
    (8, 512, 1000, 5, False),
    (20, 256, 777, 2, False),       # two 16-column tiles
    (4, 512, 1500, 5, True),        # shared lm_head: 20 columns in one pass
    (70, 128, 200, 1, False),       # several column passes
    (2, 264, 333, 3, False),        # H not a multiple of the 256-element chunk
    # 8 activation rows of 4104 do not fit the LDS staging: two 16-row weight
    # tiles per workgroup, with ragged ends at R = 4104 and R = 1001
    (8, 4104, 1001, 2, False),
]


@pytest.mark.parametrize("M,H,V,K,shared", SMALL_BF16)
def test_heads_bf16_small_full(M, H, V, K, shared):
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=M, H=H, V=V, K=K, cfg_id=100 + M)
    hidden, w1, wlm = synth.head_inputs(w, DEV, shared_lm_head=shared)
    announce("heads bf16", M, H, V, K, shared)
    got = api.heads(hidden, w1, wlm)
    torch.cuda.synchronize()
    ref = oheads.medusa_heads(to64(hidden), to64(w1), to64(wlm), round_r=True)
    err = row_rel_err(to64(got), ref)
    assert err <= TOL_BF16, err


def test_heads_fp32_shared_and_many_rows():
    w = synth.WORKLOADS["tiny-fp32"].scaled(B=19, cfg_id=150)
    hidden, w1, wlm = synth.head_inputs(w, DEV, shared_lm_head=True)
    announce("heads fp32 shared M=19")
    got = api.heads(hidden, w1, wlm)
    torch.cuda.synchronize()
    ref = oheads.medusa_heads(to64(hidden), to64(w1), to64(wlm), round_r=False)
    assert row_rel_err(to64(got), ref) <= TOL_F32


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER[1:])
def test_heads_full_size_sampled_rows(name):
    """Full workload shapes; the oracle recomputes a few whole (m, k) logit
    rows from the same device-generated weights."""
    w = synth.WORKLOADS[name]
    hidden, w1, wlm = synth.head_inputs(w, DEV)
    announce("heads full", name)
    got = api.heads(hidden, w1, wlm)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.cfg_id)
    pairs = {(int(rng.integers(w.B)), int(rng.integers(w.K))) for _ in range(3)}
    h64 = to64(hidden)
    for (m, k) in sorted(pairs):
        r = oheads.residual_block(h64[m:m + 1], to64(w1[k]), round_r=True)[0]
        ref = to64(wlm[k]) @ r
        err = row_rel_err(to64(got[m, k]), ref)
        assert err <= TOL_BF16, (m, k, err)
    del hidden, w1, wlm, got
    torch.cuda.empty_cache()


def test_heads_deterministic():
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=4, H=1024, V=4000, cfg_id=160)
    hidden, w1, wlm = synth.head_inputs(w, DEV)
    announce("heads determinism")
    a = api.heads(hidden, w1, wlm)
    b = api.heads(hidden, w1, wlm)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_heads_argument_errors():
    w = synth.WORKLOADS["vicuna7b-shaped"].scaled(B=2, H=256, V=100, K=2, cfg_id=170)
    hidden, w1, wlm = synth.head_inputs(w, DEV)
    logits = torch.empty((2, 2, 100), device=DEV)
    lib = api._lib.load()
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    rc = lib.medusa_heads(api._ptr(hidden), api._ptr(w1), 256 * 256, api._ptr(wlm), 100 * 256, 2,
                          256, 100, 2, api.BF16, api._ptr(logits), api._ptr(small), 16, None)
    assert rc == api.EWORKSPACE
    rc = lib.medusa_heads(api._ptr(hidden), api._ptr(w1), 256 * 256, api._ptr(wlm), 100 * 256, 2,
                          250, 100, 2, api.BF16, api._ptr(logits), api._ptr(small), 16, None)
    assert rc == api.EINVAL
    assert b"H % 8" in lib.medusa_last_error()
