"""Dense-variant Medusa heads, CPU oracle (test infrastructure only).

P1 ("Medusa 심층 아키텍처"), section "Medusa의 핵심 철학 ... 잔차 블록을 포함한
Medusa 헤드 구조": head k turns a hidden state into logits through its residual
SiLU block and its vocab projection; section "소스코드 레벨 구조 분석"
(``generate_candidates``) keeps the top-k of every head's logits.

Reading (the pages leave it open): the dense variant runs the same K heads on the
hidden state of every tree token -- M = B*T rows instead of B -- so that the
next step's candidates already exist at whichever node gets accepted.  Head d
keeps k_d candidates (the tree's per-depth top-k), by descending logit with
ties to the lower index, padded with -1 up to kmax.  It is the composition of
``heads.medusa_heads`` and ``topk.head_topk`` over the M rows, nothing more.
"""
from __future__ import annotations

import numpy as np

from .heads import medusa_heads
from .topk import head_topk


def dense_candidates(hidden_rows: np.ndarray, w1: np.ndarray, wlm: np.ndarray,
                     k_per_head, round_r: bool = False):
    """hidden_rows [M, H] -> (topk_idx [M, K, kmax] int64 (-1 padded),
    logits [M, K, V] fp64)."""
    logits = medusa_heads(hidden_rows, w1, wlm, round_r)
    return head_topk(logits, list(k_per_head)), logits
