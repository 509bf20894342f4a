"""Static candidate tree, CPU oracle (test infrastructure only).

Follows P1 ("Medusa 심층 아키텍처"), section "트리 어텐션 ... 고정 트리 토폴로지와
2차원 어텐션 마스크": head d contributes its top candidates at depth d, a fixed
topology combines them into paths, and the tree mask lets token i see token j
iff j is an ancestor of i or j = i (0, else -inf).  The visible sets are built
two independent ways here: by walking parent pointers, and as the reflexive
transitive closure of the one-hop "parent of" relation (the least fixpoint of
repeated boolean matrix products).

Node numbering: node 0 is the root (the base model's token t+1); a node at
depth d >= 1 carries candidate number rank(n) of Medusa head d (head index
d-1), which predicts token t+d+1 (P1 section "Medusa의 핵심 철학", head list;
P4 section 2.2).  Position of node n = ctx + depth(n).

Reading: P1's sketch of the mask builder lost its indentation; it is read as
requiring parents before children, so every topology here has parent[n] < n.
"""
from __future__ import annotations

from typing import List, Sequence, Set

import numpy as np


def validate(parent: Sequence[int], rank: Sequence[int], k_per_depth: Sequence[int]) -> np.ndarray:
    """Check the topology; return depth[T].  Raises ValueError if invalid."""
    parent = [int(p) for p in parent]
    rank = [int(r) for r in rank]
    T = len(parent)
    if T < 1 or len(rank) != T:
        raise ValueError("need T >= 1 nodes and one rank per node")
    if parent[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    depth = [0] * T
    seen = set()
    for n in range(1, T):
        p = parent[n]
        if not (0 <= p < n):
            raise ValueError(f"parent[{n}]={p} is not an earlier node")
        depth[n] = depth[p] + 1
        if depth[n] > len(k_per_depth):
            raise ValueError(f"node {n} is deeper than the number of heads")
        if not (0 <= rank[n] < k_per_depth[depth[n] - 1]):
            raise ValueError(f"rank[{n}]={rank[n]} outside head {depth[n]}'s top-k")
        if (p, rank[n]) in seen:
            raise ValueError(f"two children of node {p} share rank {rank[n]}")
        seen.add((p, rank[n]))
    return np.asarray(depth, dtype=np.int64)


def ancestors_bruteforce(parent: Sequence[int]) -> List[Set[int]]:
    """anc(i) by walking parent pointers from i to the root (i excluded)."""
    out = []
    for i in range(len(parent)):
        s, u = set(), int(parent[i])
        while u >= 0:
            s.add(u)
            u = int(parent[u])
        out.append(s)
    return out


def visible_bruteforce(parent: Sequence[int]) -> np.ndarray:
    """Boolean [T, T]: vis[i, j] iff j is an ancestor of i or j == i."""
    T = len(parent)
    vis = np.zeros((T, T), dtype=bool)
    for i, s in enumerate(ancestors_bruteforce(parent)):
        vis[i, i] = True
        for j in s:
            vis[i, j] = True
    return vis


def visible_by_closure(parent: Sequence[int]) -> np.ndarray:
    """Boolean [T, T] visibility as the reflexive transitive closure of the
    one-hop relation up[i, parent(i)]: start from the identity and add one
    more hop (a boolean matrix product) until no new pair appears.  A tree has
    no cycles, so the loop ends after at most depth + 1 products."""
    T = len(parent)
    up = np.zeros((T, T), dtype=np.int64)
    for n in range(T):
        if int(parent[n]) >= 0:
            up[n, int(parent[n])] = 1
    vis = np.eye(T, dtype=bool)
    reach = np.eye(T, dtype=np.int64)
    while True:
        reach = (reach @ up > 0).astype(np.int64)   # exactly one hop further
        if not reach.any():
            return vis
        vis |= reach > 0


def additive_mask(vis: np.ndarray) -> np.ndarray:
    """The [T, T] additive form of a visibility matrix: 0 where visible,
    -inf where hidden (P1 tree-attention section)."""
    return np.where(vis, 0.0, -np.inf)


def bitmask_rows(vis: np.ndarray) -> np.ndarray:
    """Pack a boolean [T, T] visibility matrix into uint64 words [T, ceil(T/64)]:
    bit (j % 64) of word j // 64 in row i is vis[i, j]."""
    T = vis.shape[0]
    W = (T + 63) // 64
    out = np.zeros((T, W), dtype=np.uint64)
    for i in range(T):
        for j in range(T):
            if vis[i, j]:
                out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


def children_in_rank_order(parent: Sequence[int], rank: Sequence[int]) -> List[List[int]]:
    T = len(parent)
    kids: List[List[int]] = [[] for _ in range(T)]
    for n in range(1, T):
        kids[int(parent[n])].append(n)
    for u in range(T):
        kids[u].sort(key=lambda n: int(rank[n]))
    return kids


def tree_tokens(topk_idx: np.ndarray, root: Sequence[int], parent, rank) -> np.ndarray:
    """tree_tokens[b, 0] = root[b]; tree_tokens[b, n] = topk_idx[b, depth(n)-1, rank(n)]."""
    depth = depth_of(parent)
    B = topk_idx.shape[0]
    T = len(parent)
    out = np.zeros((B, T), dtype=np.int64)
    for b in range(B):
        out[b, 0] = int(root[b])
        for n in range(1, T):
            out[b, n] = int(topk_idx[b, depth[n] - 1, int(rank[n])])
    return out


def positions(ctx_len: Sequence[int], parent) -> np.ndarray:
    """pos[b, n] = ctx_len[b] + depth(n): node n sits depth(n) tokens after the
    last cached token, whatever branch it is on."""
    depth = depth_of(parent)
    return np.asarray([[int(c) + int(d) for d in depth] for c in ctx_len], dtype=np.int64)


def depth_of(parent) -> np.ndarray:
    T = len(parent)
    d = np.zeros(T, dtype=np.int64)
    for n in range(1, T):
        d[n] = d[int(parent[n])] + 1
    return d


def expected_accepted(parent, rank, p_accept) -> float:
    """Expected accepted nodes per step of a static tree when the rank-r
    candidate of head d is right with probability p_accept[d-1][r]
    independently along a path (P2, paper-results section: an optimised
    tree configuration; P1: topology chosen by profiling): the sum over
    non-root nodes of the product of p along the root-to-node path."""
    depth = depth_of(parent)
    prob = [1.0] * len(parent)
    total = 0.0
    for n in range(1, len(parent)):
        prob[n] = prob[int(parent[n])] * float(p_accept[depth[n] - 1][int(rank[n])])
        total += prob[n]
    return total


def optimal_tree_bruteforce(p_accept, k_per_depth, T: int):
    """Brute force over every prefix-closed set of T-1 rank tuples: the best
    expected accepted nodes (tiny cases only)."""
    import itertools
    K = len(k_per_depth)
    tuples = []
    for d in range(1, K + 1):
        tuples.extend(itertools.product(*[range(k) for k in k_per_depth[:d]]))
    best = -1.0
    for subset in itertools.combinations(tuples, T - 1):
        s = set(subset)
        if any(len(t) > 1 and t[:-1] not in s for t in s):
            continue
        val = 0.0
        for t in s:
            pr = 1.0
            for d, r in enumerate(t):
                pr *= float(p_accept[d][r])
            val += pr
        best = max(best, val)
    return best
