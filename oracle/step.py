"""One Medusa verify step composed from the oracle's stages (test
infrastructure only): heads -> per-head top-k -> tree tokens/positions ->
tree attention per layer -> acceptance.  The base model itself (which turns
the attention outputs into the verification logits) is not part of the path:
its logits are an input, as are the per-layer Q/K/V.
Pinned on inputs with a closed-form outcome: W1 = 0 and a one-hot hidden
state give every head a prescribed logit order (so the top-k and tree tokens
are known), identical V rows fix every attention output, and planted greedy
argmaxes fix the accepted path.
"""
from __future__ import annotations

import numpy as np

from . import accept, attention, heads, topk, tree


def verify_step(hidden, w1, wlm, round_r, root, ctx_len, parent, rank, k_per_depth,
                layers, base_logits, u_accept, u_sample, tau, scale=None):
    """layers: list of (q, k_cache, v_cache).  Returns a dict of all outputs."""
    logits = heads.medusa_heads(hidden, w1, wlm, round_r)             # [B, K, V]
    tk = topk.head_topk(logits, k_per_depth)                           # [B, K, kmax]
    toks = tree.tree_tokens(tk, root, parent, rank)                    # [B, T]
    pos = tree.positions(ctx_len, parent)
    vis = tree.visible_bruteforce(parent)
    attn = [attention.tree_attention(q, k, v, ctx_len, vis, scale) for (q, k, v) in layers]
    acc, otok, onode, _ = accept.accept_paths(base_logits, logits, toks, parent, rank,
                                              u_accept, u_sample, tau, len(k_per_depth))
    return dict(head_logits=logits, topk=tk, tree_tokens=toks, pos=pos, attn=attn,
                accept_len=acc, out_tokens=otok, out_nodes=onode)
