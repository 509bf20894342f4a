"""Commit of an accepted path: KV rollback / compaction -- TEST INFRASTRUCTURE ONLY.

P3 ("Speculative Decoding(투기적 디코딩) 원리와 가속 아키텍처"), architecture
section (the pipeline ends with rollback and the confirmed correction token)
and section 5, Case 2 (K-token verification with early rejection and
rollback); P4 ("추측 디코딩과 긴 컨텍스트"), section 1.3: matched drafts are kept,
everything after the first mismatch is discarded.

With tree node n's K/V in cache slot ctx + n, keeping the accepted path
(root, then the accepted node at each depth d = 1..len) means the sequence
positions ctx, ctx+1, ..., ctx+len now hold root, path[1], ..., path[len];
the next step starts at ctx + len + 1 with the emitted correction / bonus
token as its root.
"""
import numpy as np


def commit(k, v, ctx_len, accept_len, out_nodes, out_tokens):
    """k, v: [L][B][Hkv][S_cap][D] arrays (any dtype).  Returns (k', v',
    ctx_next [B], root_next [B]); every moved row is read from the cache as
    it was before the commit."""
    k2, v2 = k.copy(), v.copy()
    B = k.shape[1]
    ctx_next = np.zeros(B, np.int64)
    root_next = np.zeros(B, np.int64)
    for b in range(B):
        c, n = int(ctx_len[b]), int(accept_len[b])
        for d in range(1, n + 1):
            src = c + int(out_nodes[b][d])
            k2[:, b, :, c + d] = k[:, b, :, src]
            v2[:, b, :, c + d] = v[:, b, :, src]
        ctx_next[b] = c + n + 1
        root_next[b] = int(out_tokens[b][n])
    return k2, v2, ctx_next, root_next

