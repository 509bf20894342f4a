"""Pins for the heads oracle: closed forms, special cases and an independent
library implementation (torch CPU fp64), chosen so that a dropped residual, a
transposed weight, a wrong activation or a missing bf16 rounding fails."""
import numpy as np
import pytest
import torch

from oracle import heads


def test_silu_closed_form_values():
    # SiLU(a) = a * sigmoid(a): values fixed by the definition
    a = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 2.0])
    got = heads.silu(a)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    assert got[0] == 0.0
    assert got[1] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert got[2] == pytest.approx(-0.2689414213699951, rel=1e-15)
    assert got[3] == pytest.approx(40.0, rel=1e-15)
    assert abs(got[4]) < 1e-15
    assert got[5] == pytest.approx(2.0 * sig(2.0), rel=1e-15)


def test_silu_matches_torch():
    x = np.random.default_rng(0).normal(size=1000) * 6
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(heads.silu(x), ref, rtol=1e-14, atol=1e-300)


def test_hand_worked_two_dim_example():
    # H = 2, W1 = diag(1, -1), h = (1, 1): a = (1, -1), r = SiLU(a) + h
    w1 = np.array([[[1.0, 0.0], [0.0, -1.0]]])
    wlm = np.array([[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]])
    h = np.array([[1.0, 1.0]])
    out = heads.medusa_heads(h, w1, wlm)
    r0 = 1.0 + 0.7310585786300049
    r1 = 1.0 - 0.2689414213699951
    np.testing.assert_allclose(out[0, 0], [r0, r1, r0 + r1], rtol=1e-15)


def test_zero_w1_gives_projection_of_hidden():
    rng = np.random.default_rng(1)
    M, H, V, K = 3, 16, 40, 2
    h = rng.normal(size=(M, H))
    wlm = rng.normal(size=(K, V, H))
    out = heads.medusa_heads(h, np.zeros((K, H, H)), wlm)
    for k in range(K):
        np.testing.assert_allclose(out[:, k], np.matmul(h, wlm[k].T), rtol=1e-13)


def test_zero_hidden_gives_zero_logits():
    rng = np.random.default_rng(2)
    out = heads.medusa_heads(np.zeros((2, 8)), rng.normal(size=(3, 8, 8)), rng.normal(size=(3, 11, 8)))
    assert np.all(out == 0.0)


def test_shared_lm_head_equals_identical_copies():
    rng = np.random.default_rng(3)
    M, H, V, K = 2, 12, 30, 3
    h = rng.normal(size=(M, H))
    w1 = rng.normal(size=(K, H, H)) * 0.3
    shared = rng.normal(size=(V, H))
    a = heads.medusa_heads(h, w1, shared)
    b = heads.medusa_heads(h, w1, np.stack([shared] * K))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("round_r", [False, True])
def test_against_torch_linear_fp64(round_r):
    """torch.nn.functional.linear uses the same [out, in] convention; a
    transposed W1 or W_lm in the oracle would fail here (weights are not
    symmetric)."""
    rng = np.random.default_rng(4)
    M, H, V, K = 3, 24, 50, 2
    h = rng.normal(size=(M, H))
    w1 = rng.normal(size=(K, H, H)) * 0.2
    wlm = rng.normal(size=(K, V, H)) * 0.2
    got = heads.medusa_heads(h, w1, wlm, round_r=round_r)
    th = torch.from_numpy(h)
    for k in range(K):
        r = torch.nn.functional.silu(torch.nn.functional.linear(th, torch.from_numpy(w1[k]))) + th
        if round_r:
            r = r.to(torch.float32).to(torch.bfloat16).to(torch.float64)
        ref = torch.nn.functional.linear(r, torch.from_numpy(wlm[k])).numpy()
        tol = 1e-12 if not round_r else 1e-6
        np.testing.assert_allclose(got[:, k], ref, rtol=tol, atol=tol)


def test_round_to_bf16_matches_torch_conversion():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(size=5000) * 10.0 ** rng.integers(-8, 8, size=5000),
                        [0.0, -0.0, 1.0, -3.5]])
    # fp32-representable inputs so that torch's fp32 -> bf16 is a single rounding
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(heads.round_to_bf16(x), ref)


def test_round_to_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even (1.0)
    assert heads.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert heads.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_sampled_rows_match_full():
    rng = np.random.default_rng(6)
    M, H, V, K = 2, 16, 33, 3
    h = rng.normal(size=(M, H))
    w1 = rng.normal(size=(K, H, H)) * 0.3
    wlm = rng.normal(size=(K, V, H))
    full = heads.medusa_heads(h, w1, wlm, round_r=True)
    samples = [(1, 2, 5), (0, 0, 32), (1, 1, 0)]
    got = heads.medusa_heads_rows(h, w1, wlm, True, samples)
    np.testing.assert_allclose(got, [full[s] for s in samples], rtol=1e-13)
