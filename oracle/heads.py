"""Medusa heads, CPU oracle (test infrastructure only).

Follows P1 ("Medusa 심층 아키텍처"), section "Medusa의 핵심 철학 ... 잔차 블록을
포함한 Medusa 헤드 구조": head k maps the last hidden state h to
h_k = SiLU(h W_res^(k)) + h and its distribution p_k = softmax(h_k W_head^(k)).
The sketch code in P1's section "소스코드 레벨 구조 분석" fixes the details the
equations leave open: both projections are bias-free linear layers stored
[out, in], the activation is SiLU, the residual adds the input, and
``generate_candidates`` takes top-k of the *logits* (softmax is monotone, so it
is deferred to acceptance).

Readings (where the pages are silent):
  * weights are [out, in]; ``h W`` in the equation is W @ h with W [out, in];
  * SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a));
  * in bf16 workloads the residual output r is rounded to bf16 (round to
    nearest even) before the vocab projection; logits stay fp64 here;
  * a shared vocab projection (frozen base unembedding, which P1 allows) is a
    [V, H] matrix used by every head.
"""
from __future__ import annotations

import numpy as np


def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a / (1 + e^{-a}), fp64."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (ties to even), returned as
    fp64.  bf16 keeps the top 16 bits of an IEEE fp32; rounding fp64 straight
    to 8 significand bits is done here on the fp64 value itself."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(x[nz])           # x = m * 2^e, 0.5 <= |m| < 1
    # bf16 has 8 significand bits (1 implicit + 7 stored): scale m to 2^8
    scaled = m * 256.0
    r = np.round(scaled)             # numpy rounds half to even
    out[nz] = np.ldexp(r / 256.0, e)
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def residual_block(hidden: np.ndarray, w1_k: np.ndarray, round_r: bool) -> np.ndarray:
    """r = SiLU(W1 h) + h for every row of ``hidden`` [M, H]; W1 [H_out, H_in]."""
    h = np.asarray(hidden, dtype=np.float64)
    a = h @ np.asarray(w1_k, dtype=np.float64).T          # a[m, o] = sum_i W1[o, i] h[m, i]
    r = silu(a) + h
    return round_to_bf16(r) if round_r else r


def medusa_heads(hidden: np.ndarray, w1: np.ndarray, wlm: np.ndarray,
                 round_r: bool = False) -> np.ndarray:
    """Head logits [M, K, V] from hidden [M, H].

    w1:  [K, H, H]   per-head residual projection ([out, in])
    wlm: [K, V, H]   per-head vocab projection, or [V, H] shared by all heads
    """
    hidden = np.asarray(hidden, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    wlm = np.asarray(wlm, dtype=np.float64)
    M, H = hidden.shape
    K = w1.shape[0]
    shared = wlm.ndim == 2
    V = wlm.shape[0] if shared else wlm.shape[1]
    out = np.empty((M, K, V), dtype=np.float64)
    for k in range(K):
        r = residual_block(hidden, w1[k], round_r)
        W = wlm if shared else wlm[k]
        out[:, k, :] = r @ W.T                              # logits[m, v] = sum_i W[v, i] r[m, i]
    return out


def medusa_heads_rows(hidden: np.ndarray, w1: np.ndarray, wlm, round_r: bool,
                      samples) -> np.ndarray:
    """The logits at selected (m, k, v) positions only, for checks at sizes
    where the full [M, K, V] product is too slow.  ``wlm`` may be a callable
    (k, v) -> row [H] so that callers can fetch single rows lazily."""
    hidden = np.asarray(hidden, dtype=np.float64)
    cache = {}
    out = np.empty(len(samples), dtype=np.float64)
    for i, (m, k, v) in enumerate(samples):
        if (m, k) not in cache:
            w1k = w1(k) if callable(w1) else np.asarray(w1[k], dtype=np.float64)
            cache[(m, k)] = residual_block(hidden[m:m + 1], w1k, round_r)[0]
        row = wlm(k, v) if callable(wlm) else np.asarray(
            wlm[v] if np.ndim(wlm) == 2 else wlm[k, v], dtype=np.float64)
        out[i] = float(np.dot(np.asarray(row, dtype=np.float64), cache[(m, k)]))
    return out
