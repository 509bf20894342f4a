"""Per-head top-k, CPU oracle (test infrastructure only).

Follows P1 ("Medusa 심층 아키텍처"), section "소스코드 레벨 구조 분석": each head's
logits go through ``torch.topk(logits, top_k)`` and the indices are kept as
that head's candidates.  P2 ("[vLLM] Medusa"), section "propose()", is the k=1
case: the argmax of every head, stacked per sequence.

Reading: order by descending value; equal values are ordered by ascending
index (the page does not say; this makes the result unique).  A stable sort on
the negated values gives exactly that order.
"""
from __future__ import annotations

import numpy as np


def topk(x: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries of the 1-D array ``x``, largest first,
    ties to the lower index."""
    x = np.asarray(x)
    if x.ndim != 1:
        raise ValueError("topk expects a 1-D array")
    order = np.argsort(-x, kind="stable")
    return order[:k].astype(np.int64)


def head_topk(head_logits: np.ndarray, k_per_depth) -> np.ndarray:
    """head_logits [B, K, V] -> topk_idx [B, K, kmax], padded with -1 where
    head d keeps fewer than kmax candidates."""
    head_logits = np.asarray(head_logits)
    B, K, V = head_logits.shape
    kmax = max(k_per_depth)
    out = np.full((B, K, kmax), -1, dtype=np.int64)
    for b in range(B):
        for d in range(K):
            kd = k_per_depth[d]
            out[b, d, :kd] = topk(head_logits[b, d], kd)
    return out
