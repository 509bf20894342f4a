"""Pins of the dense-variant heads oracle (oracle/dense_heads.py): heads on
every tree row, each head's top-k.  Each check ties it to something other
than its own code: row independence, special cases that reduce to a plain
matrix product and a library sort, tie order, shared vs per-head weights,
padding, and a rank-count brute force on tiny vocabularies."""
import numpy as np
import pytest

from oracle import dense_heads
from oracle import heads as oheads


def _weights(rng, K, H, V, scale=0.3):
    return rng.normal(0, scale, (K, H, H)), rng.normal(0, 1.0, (K, V, H))


def test_rows_are_independent():
    """Row m of the dense result equals the heads run on row m alone."""
    rng = np.random.default_rng(1)
    M, H, V, K = 6, 8, 40, 3
    h = rng.normal(0, 1, (M, H))
    w1, wlm = _weights(rng, K, H, V)
    idx, logits = dense_heads.dense_candidates(h, w1, wlm, (4, 3, 2))
    for m in range(M):
        i1, l1 = dense_heads.dense_candidates(h[m:m + 1], w1, wlm, (4, 3, 2))
        np.testing.assert_allclose(l1[0], logits[m], rtol=1e-12, atol=1e-12)
        assert (i1[0] == idx[m]).all()


def test_zero_residual_weights_reduce_to_plain_product_and_sort():
    """W1 = 0: SiLU(0) = 0, so r = h and the logits are W_lm h; the top-k is
    then numpy's stable argsort of the negated product."""
    rng = np.random.default_rng(2)
    M, H, V, K = 5, 6, 30, 2
    h = rng.normal(0, 1, (M, H))
    w1 = np.zeros((K, H, H))
    wlm = rng.normal(0, 1, (K, V, H))
    idx, logits = dense_heads.dense_candidates(h, w1, wlm, (5, 5))
    for m in range(M):
        for k in range(K):
            ref = wlm[k] @ h[m]
            np.testing.assert_allclose(logits[m, k], ref, rtol=1e-13, atol=1e-13)
            assert (idx[m, k] == np.argsort(-ref, kind="stable")[:5]).all()


def test_ties_go_to_the_lower_index():
    """Duplicate vocab rows give equal logits; the lower index ranks first."""
    rng = np.random.default_rng(3)
    H, V = 4, 10
    h = rng.normal(0, 1, (1, H))
    w1 = np.zeros((1, H, H))
    wlm = rng.normal(0, 1, (1, V, H))
    best = int(np.argmax(wlm[0] @ h[0]))
    wlm[0, 7] = wlm[0, best]                    # an exact copy of the best row
    wlm[0, 2] = wlm[0, best]
    idx, _ = dense_heads.dense_candidates(h, w1, wlm, (3,))
    assert idx[0, 0].tolist() == sorted({best, 2, 7})


def test_shared_vocab_projection_equals_identical_copies():
    rng = np.random.default_rng(4)
    M, H, V, K = 4, 8, 25, 3
    h = rng.normal(0, 1, (M, H))
    w1, _ = _weights(rng, K, H, V)
    shared = rng.normal(0, 1, (V, H))
    a = dense_heads.dense_candidates(h, w1, shared, (3, 2, 2))
    b = dense_heads.dense_candidates(h, w1, np.stack([shared] * K), (3, 2, 2))
    assert (a[0] == b[0]).all()
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)


def test_padding_for_heads_with_fewer_candidates():
    rng = np.random.default_rng(5)
    h = rng.normal(0, 1, (2, 4))
    w1, wlm = _weights(rng, 3, 4, 12)
    idx, _ = dense_heads.dense_candidates(h, w1, wlm, (4, 2, 1))
    assert idx.shape == (2, 3, 4)
    assert (idx[:, 1, 2:] == -1).all() and (idx[:, 2, 1:] == -1).all()
    assert (idx[:, 0] >= 0).all()


@pytest.mark.parametrize("seed", range(5))
def test_rank_count_brute_force(seed):
    """Candidate at position p of head d has exactly p logits ranked above it
    (larger, or equal with a lower index) -- counted pairwise, no sort."""
    rng = np.random.default_rng(10 + seed)
    M, H, V, K = 3, 5, 9, 2
    h = rng.normal(0, 1, (M, H))
    w1, wlm = _weights(rng, K, H, V)
    # a few forced ties
    wlm[0, 4] = wlm[0, 1]
    kd = (4, 3)
    idx, logits = dense_heads.dense_candidates(h, w1, wlm, kd, round_r=bool(seed % 2))
    for m in range(M):
        for k in range(K):
            x = logits[m, k]
            for p in range(kd[k]):
                v = int(idx[m, k, p])
                above = sum(1 for u in range(V) if x[u] > x[v] or (x[u] == x[v] and u < v))
                assert above == p, (m, k, p)


def test_round_r_matches_heads_oracle_reading():
    """With round_r the residual output is rounded to bf16 before the vocab
    projection, exactly as the standard heads oracle does."""
    rng = np.random.default_rng(6)
    h = rng.normal(0, 1, (3, 8))
    w1, wlm = _weights(rng, 2, 8, 20)
    _, logits = dense_heads.dense_candidates(h, w1, wlm, (2, 2), round_r=True)
    ref = oheads.medusa_heads(h, w1, wlm, round_r=True)
    np.testing.assert_array_equal(logits, ref)
