"""Path acceptance, CPU oracle (test infrastructure only).

Greedy (temperature 0) follows P3 ("Speculative Decoding(투기적 디코딩) 원리와
가속 아키텍처"), section 5, the greedy check: drafts are compared with the
target's argmax and the first mismatch is replaced, so the output equals
target-only greedy decoding.  P4 ("추측 디코딩과 긴 컨텍스트"), section 1.3: tokens
are kept up to the first mismatch, that position gets the target's own
prediction, everything after it is dropped, and when every draft matches the
target's next prediction comes for free (the bonus token).

Rejection sampling follows P1 ("Medusa 심층 아키텍처"), section "수학적 무손실
보장: 기각 샘플링": a draft x is accepted with probability
alpha(x) = min(1, p(x)/q(x)) by comparing a uniform r with alpha (accept when
r < alpha); on rejection a token is drawn from the residual
p'(x) = max(0, p(x) - q(x)) / sum_y max(0, p(y) - q(y)).  P3 section 2 proves
that the result is distributed as p.

On a tree (readings where the pages leave the step open):
  * node 0 is the root (already decided); its base logits give p for depth 1;
  * the children of the current node are tried one by one in rank order; a
    rejection replaces p by the residual max(0, p - q_d) (normalised) before
    the next sibling is tried (with one child this is exactly the pages' rule;
    it stays lossless when the siblings are independent draws from q_d);
  * q_d = softmax(head_logits[d-1] / tau) for a child at depth d, since Medusa
    head d proposes depth-d tokens; p_u = softmax(base_logits[u] / tau);
  * an accepted child becomes the current node and p becomes its p_u;
  * when the current node is a leaf or every child was rejected, one token is
    drawn from the current p by inverse CDF with u_sample[u]: the smallest v
    with cumsum(p)[v] > u * sum(p) (if rounding leaves none, the last v with
    p(v) > 0).  Accepted draws use u_accept[c] of the child tested;
  * q(x) = 0 gives alpha = 1; a residual with zero mass leaves p unchanged;
  * emitted tokens = tokens of the accepted nodes (root excluded) followed by
    the sampled / argmax token, i.e. accept_len + 1 tokens (1..K+1).
Greedy ties: argmax takes the first maximum; if several children carry the
target token, the lowest rank wins.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

from .tree import children_in_rank_order, depth_of


@dataclass
class AcceptResult:
    accept_len: int
    tokens: List[int]          # accept_len + 1 emitted tokens
    nodes: List[int]           # accept_len + 1 tree nodes: root then accepted nodes
    # decision log for near-tie analysis: (kind, node, margin)
    trace: List[Tuple[str, int, float]] = field(default_factory=list)


def accept_greedy(base_logits, tree_tokens, parent, rank) -> AcceptResult:
    """One sequence: base_logits [T, V], tree_tokens [T]."""
    base_logits = np.asarray(base_logits)
    kids = children_in_rank_order(parent, rank)
    u, path = 0, [0]
    while True:
        t = int(np.argmax(base_logits[u]))         # first maximum
        nxt = [c for c in kids[u] if int(tree_tokens[c]) == t]
        if not nxt:
            break
        u = nxt[0]
        path.append(u)
    toks = [int(tree_tokens[n]) for n in path[1:]] + [t]
    return AcceptResult(len(path) - 1, toks, path)


def softmax_t(z, tau: float) -> np.ndarray:
    """softmax(z / tau) in fp64."""
    z = np.asarray(z, dtype=np.float64) / float(tau)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def inverse_cdf(p: np.ndarray, u: float) -> Tuple[int, float]:
    """Smallest v with cumsum(p)[v] > u * sum(p); also the margin
    min |cumsum - u*sum(p)| / sum(p) at the chosen boundary."""
    c = np.cumsum(p)
    thr = float(u) * c[-1]
    hits = np.nonzero(c > thr)[0]
    if len(hits):
        v = int(hits[0])
    else:
        v = int(np.nonzero(p > 0)[0][-1])
    lo = c[v - 1] if v > 0 else 0.0
    margin = min(abs(c[v] - thr), abs(thr - lo)) / c[-1]
    return v, margin


def accept_rejection(base_logits, head_logits, tree_tokens, parent, rank,
                     u_accept, u_sample, tau: float) -> AcceptResult:
    """One sequence: base_logits [T, V], head_logits [K, V], tree_tokens [T],
    u_accept [T], u_sample [T]."""
    kids = children_in_rank_order(parent, rank)
    depth = depth_of(parent)
    q_cache = {}

    def q_of(d):
        if d not in q_cache:
            q_cache[d] = softmax_t(head_logits[d - 1], tau)
        return q_cache[d]

    trace = []
    u, path = 0, [0]
    p = softmax_t(base_logits[0], tau)
    while True:
        accepted = None
        for c in kids[u]:
            q = q_of(int(depth[c]))
            x = int(tree_tokens[c])
            alpha = 1.0 if q[x] == 0.0 else min(1.0, p[x] / q[x])
            r = float(u_accept[c])
            trace.append(("accept", c, abs(r - alpha)))
            if r < alpha:
                accepted = c
                break
            res = np.maximum(0.0, p - q)
            Z = np.sum(res)
            if Z > 0.0:
                p = res / Z
        if accepted is None:
            break
        u = accepted
        path.append(u)
        p = softmax_t(base_logits[u], tau)
    y, margin = inverse_cdf(p, float(u_sample[u]))
    trace.append(("sample", u, margin))
    toks = [int(tree_tokens[n]) for n in path[1:]] + [y]
    return AcceptResult(len(path) - 1, toks, path, trace)


def accept_paths(base_logits, head_logits, tree_tokens, parent, rank, u_accept, u_sample,
                 tau: float, K: int):
    """Batched form matching the library's outputs: accept_len [B],
    out_tokens [B, K+1], out_nodes [B, K+1] (-1 padded), and the per-sequence
    results (with decision traces)."""
    base_logits = np.asarray(base_logits)
    B = base_logits.shape[0]
    acc = np.zeros(B, np.int64)
    toks = np.full((B, K + 1), -1, np.int64)
    nodes = np.full((B, K + 1), -1, np.int64)
    res = []
    for b in range(B):
        if tau == 0.0:
            r = accept_greedy(base_logits[b], tree_tokens[b], parent, rank)
        else:
            r = accept_rejection(base_logits[b], head_logits[b], tree_tokens[b], parent, rank,
                                 u_accept[b], u_sample[b], tau)
        acc[b] = r.accept_len
        toks[b, :len(r.tokens)] = r.tokens
        nodes[b, :len(r.nodes)] = r.nodes
        res.append(r)
    return acc, toks, nodes, res


def expected_tokens_per_step(alpha: float, K: int) -> float:
    """E[N] = 1 + alpha + ... + alpha^K = (1 - alpha^{K+1}) / (1 - alpha) for K
    drafts each accepted independently with probability alpha (P3 section 2,
    expected tokens per step)."""
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)
