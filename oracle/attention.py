"""Tree-masked attention, CPU oracle (test infrastructure only).

Follows P1 ("Medusa 심층 아키텍처"), section "트리 어텐션 ... 고정 트리 토폴로지와
2차원 어텐션 마스크": all T tree tokens go through one attention pass in which
token i sees the cached context and, among the tree tokens, only its
ancestors and itself (the tree mask).  Each branch is thereby evaluated as if
it were its own sequence.  P4 ("추측 디코딩과 긴 컨텍스트"), section 3.3, states
the property that blockwise partial softmaxes merged through a running max and
exp-sum equal the full softmax; the oracle does not need it (it takes the full
softmax at once) but the pins below exercise the same identity.

Definition computed here, fp64, for every sequence b, query head h and tree
node i:
    keys    = context slots 0..ctx_b-1  and tree slots ctx_b + j, j visible from i
    s_j     = scale * <q[b,i,h], k[b,g(h),slot_j]>
    o[b,i,h]= sum_j softmax(s)_j * v[b,g(h),slot_j]
with g(h) = h // (Hq/Hkv) (grouped-query attention; heads of a group share
one K/V head).

Readings: scale = 1/sqrt(D) unless given; Q and K arrive already
position-encoded (no rotary embedding here); the caller stores the tree
tokens' K/V in cache slots ctx..ctx+T-1 (the pages keep the tree tokens'
K/V next to the cached context without fixing a layout).
"""
from __future__ import annotations

import numpy as np


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def tree_attention(q, k_cache, v_cache, ctx_len, visible, scale=None) -> np.ndarray:
    """q [B,T,Hq,D]; k_cache, v_cache [B,Hkv,S_cap,D]; ctx_len [B];
    visible [T,T] bool (row i: which tree tokens node i may see).
    Returns o [B,T,Hq,D] fp64."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    for b in range(B):
        c = int(ctx_len[b])
        for h in range(Hq):
            g = h // G
            keys = kc[b, g, :c + T]                         # context then tree slots
            vals = vc[b, g, :c + T]
            s = scale * (q[b, :, h, :] @ keys.T)            # [T, c+T]
            allowed = np.concatenate([np.ones((T, c), bool), np.asarray(visible, bool)], axis=1)
            s = np.where(allowed, s, -np.inf)
            out[b, :, h, :] = _softmax_rows(s) @ vals
    return out


def tree_attention_rows(q_rows, kv_fetch, ctx_len, visible, scale, T, G, samples) -> np.ndarray:
    """The same definition for selected (b, i, h) rows only, for checks at
    sizes where the full output is too slow.  ``q_rows[s]`` is the query
    vector of sample s; ``kv_fetch(b, g, n)`` returns (keys, values) of the
    first n cache slots of sequence b, K/V head g, as [n, D] arrays."""
    out = []
    for s_i, (b, i, h) in enumerate(samples):
        g = h // G
        c = int(ctx_len[b])
        keys, vals = kv_fetch(b, g, c + T)
        keys = np.asarray(keys, dtype=np.float64)
        vals = np.asarray(vals, dtype=np.float64)
        s = float(scale) * (keys @ np.asarray(q_rows[s_i], dtype=np.float64))
        allowed = np.concatenate([np.ones(c, bool), np.asarray(visible[i], bool)])
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max())
        out.append((p / p.sum()) @ vals)
    return np.asarray(out)


def causal_attention(q_seq, k_seq, v_seq, scale) -> np.ndarray:
    """Ordinary causal attention of one head over one sequence: query t sees
    keys 0..t.  q_seq, k_seq, v_seq: [N, D]."""
    q_seq = np.asarray(q_seq, np.float64)
    k_seq = np.asarray(k_seq, np.float64)
    v_seq = np.asarray(v_seq, np.float64)
    N = q_seq.shape[0]
    out = np.zeros_like(q_seq)
    for t in range(N):
        s = scale * (k_seq[:t + 1] @ q_seq[t])
        p = np.exp(s - s.max())
        out[t] = (p / p.sum()) @ v_seq[:t + 1]
    return out


def path_causal_attention(q, k_cache, v_cache, ctx_len, parent, scale=None) -> np.ndarray:
    """The alternative definition of tree attention: for every root-to-leaf
    path, lay the context followed by the path's tree tokens out as one
    ordinary sequence and run causal attention over it; node i's output is the
    output at its place on any path through it.  Context queries are not
    needed, so only the path positions are evaluated (a causal query at a path
    position sees the whole context plus the path prefix)."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    parent = [int(p) for p in parent]
    is_parent = set(parent[1:])
    leaves = [n for n in range(T) if n not in is_parent]
    out = np.full((B, T, Hq, D), np.nan)
    for leaf in leaves:
        path = []
        u = leaf
        while u >= 0:
            path.append(u)
            u = parent[u]
        path.reverse()                                     # root ... leaf
        for b in range(B):
            c = int(ctx_len[b])
            for h in range(Hq):
                g = h // G
                ks = np.concatenate([kc[b, g, :c], kc[b, g, [c + n for n in path]]])
                vs = np.concatenate([vc[b, g, :c], vc[b, g, [c + n for n in path]]])
                for pos, n in enumerate(path):
                    s = scale * (ks[:c + pos + 1] @ q[b, n, h])
                    p = np.exp(s - s.max())
                    out[b, n, h] = (p / p.sum()) @ vs[:c + pos + 1]
    return out
