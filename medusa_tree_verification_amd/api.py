"""Python binding of the Medusa verify-step library (argument marshalling only).

Tensors are torch tensors on the current HIP device (torch supplies device
memory and the stream); every stage runs in the HIP library.  Each function
has the name of its C entry point without the ``medusa_`` prefix.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
_CODES = {EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", EWORKSPACE: "EWORKSPACE", EHIP: "EHIP"}


class MedusaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != OK:
        raise MedusaError(rc, _lib.load().medusa_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_lib.P_i32)


def version() -> str:
    return _lib.load().medusa_version().decode()


def tree_build_host(parent, rank, k_per_depth):
    """Host-only validation + ancestor bitmask: returns (mask [T][W] uint64, depth [T])."""
    lib = _lib.load()
    parent, rank, kpd = _i32(parent), _i32(rank), _i32(k_per_depth)
    T = len(parent)
    W = (T + 63) // 64
    mask = np.zeros((T, W), np.uint64)
    depth = np.zeros(T, np.int32)
    _check(lib.medusa_tree_build_host(_p32(parent), _p32(rank), T, _p32(kpd), len(kpd),
                                      mask.ctypes.data_as(_lib.P_u64), _p32(depth)))
    return mask, depth


class Tree:
    """A static candidate tree resident on the current device."""

    def __init__(self, parent, rank, k_per_depth):
        lib = _lib.load()
        self._lib = lib
        self.parent, self.rank, self.k_per_depth = _i32(parent), _i32(rank), _i32(k_per_depth)
        h = ctypes.c_void_p()
        _check(lib.medusa_tree_create(_p32(self.parent), _p32(self.rank), len(self.parent),
                                      _p32(self.k_per_depth), len(self.k_per_depth),
                                      ctypes.byref(h)))
        self.handle = h
        vals = [ctypes.c_int32() for _ in range(5)]
        _check(lib.medusa_tree_info(h, *[ctypes.byref(v) for v in vals]))
        self.T, self.K, self.W, self.max_depth, self.kmax = [v.value for v in vals]

    def mask(self) -> np.ndarray:
        out = np.zeros((self.T, self.W), np.uint64)
        _check(self._lib.medusa_tree_mask(self.handle, out.ctypes.data_as(_lib.P_u64)))
        return out

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self._lib.medusa_tree_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    """A caller's workspace, or a new one (zero-filled, though no call needs
    that)."""
    if ws is None:
        if nbytes == 0:
            return None, 0
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def heads_workspace_size(M: int, H: int, K: int, dtype: torch.dtype) -> int:
    return _lib.load().medusa_heads_workspace_size(M, H, K, F32 if dtype == torch.float32 else BF16)


def heads(hidden: torch.Tensor, w1: torch.Tensor, wlm: torch.Tensor, logits=None, ws=None,
          stream=None) -> torch.Tensor:
    """hidden [M,H]; w1 [K,H,H]; wlm [K,V,H] or [V,H] (shared) -> logits [M,K,V] fp32."""
    lib = _lib.load()
    M, H = hidden.shape
    K = w1.shape[0]
    shared = wlm.dim() == 2
    V = wlm.shape[0] if shared else wlm.shape[1]
    if logits is None:
        logits = torch.empty((M, K, V), dtype=torch.float32, device=hidden.device)
    dt = _dt(hidden)
    ws, nb = _workspace(lib.medusa_heads_workspace_size(M, H, K, dt), hidden.device, ws)
    _check(lib.medusa_heads(_ptr(hidden), _ptr(w1), H * H, _ptr(wlm), 0 if shared else V * H,
                            M, H, V, K, dt, _ptr(logits), _ptr(ws), nb, _stream(stream)))
    return logits


def tree_candidates_workspace_size(B, V, tree: Tree) -> int:
    return _lib.load().medusa_tree_candidates_workspace_size(B, V, tree.handle)


def tree_candidates(head_logits: torch.Tensor, root: torch.Tensor, ctx_len: torch.Tensor,
                    tree: Tree, topk_idx=None, tree_tokens=None, pos=None, ws=None, stream=None):
    """head_logits [B,K,V] fp32 -> (topk_idx [B,K,kmax], tree_tokens [B,T], pos [B,T]) int32."""
    lib = _lib.load()
    B, K, V = head_logits.shape
    dev = head_logits.device
    if topk_idx is None:
        topk_idx = torch.empty((B, tree.K, tree.kmax), dtype=torch.int32, device=dev)
    if tree_tokens is None:
        tree_tokens = torch.empty((B, tree.T), dtype=torch.int32, device=dev)
    if pos is None:
        pos = torch.empty((B, tree.T), dtype=torch.int32, device=dev)
    ws, nb = _workspace(lib.medusa_tree_candidates_workspace_size(B, V, tree.handle), dev, ws)
    _check(lib.medusa_tree_candidates(_ptr(head_logits), _ptr(root), _ptr(ctx_len), tree.handle, B,
                                      V, _ptr(topk_idx), _ptr(tree_tokens), _ptr(pos), _ptr(ws), nb,
                                      _stream(stream)))
    return topk_idx, tree_tokens, pos


def heads_dense(hidden: torch.Tensor, w1: torch.Tensor, wlm: torch.Tensor, tree: "Tree",
                values: bool = True, logits=None, outs=None, ws=None, stream=None):
    """Dense-variant heads: hidden [M,H]; w1 [K,H,H]; wlm [K,V,H] or [V,H]
    (shared) -> (topk_idx [M,K,kmax] int32, topk_val [M,K,kmax] fp32 or None).
    ``logits`` (a [M,K,V] fp32 tensor) also receives every logit."""
    lib = _lib.load()
    M, H = hidden.shape
    K = w1.shape[0]
    shared = wlm.dim() == 2
    V = wlm.shape[0] if shared else wlm.shape[1]
    dt = _dt(hidden)
    dev = hidden.device
    if outs is None:
        outs = (torch.empty((M, K, tree.kmax), dtype=torch.int32, device=dev),
                torch.empty((M, K, tree.kmax), dtype=torch.float32, device=dev) if values else None)
    idx, val = outs
    nbytes = lib.medusa_heads_dense_workspace_size(M, H, V, K, tree.handle, dt)
    ws, nb = _workspace(nbytes, dev, ws)
    _check(lib.medusa_heads_dense(_ptr(hidden), _ptr(w1), H * H, _ptr(wlm), 0 if shared else V * H,
                                  M, H, V, K, tree.handle, dt, _ptr(idx), _ptr(val), _ptr(logits),
                                  _ptr(ws), nb, _stream(stream)))
    return idx, val


def tree_attention_workspace_size(B, Hq, Hkv, D, ctx_max, tree: Tree, dtype) -> int:
    return _lib.load().medusa_tree_attention_workspace_size(
        B, Hq, Hkv, D, ctx_max, tree.handle, F32 if dtype == torch.float32 else BF16)


def tree_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   ctx_len: torch.Tensor, ctx_max: int, tree: Tree, scale: Optional[float] = None,
                   out=None, ws=None, stream=None) -> torch.Tensor:
    """q [B,T,Hq,D]; k_cache/v_cache [B,Hkv,S_cap,D] -> out [B,T,Hq,D]."""
    lib = _lib.load()
    B, T, Hq, D = q.shape
    Hkv, S_cap = k_cache.shape[1], k_cache.shape[2]
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    if out is None:
        out = torch.empty_like(q)
    nbytes = lib.medusa_tree_attention_workspace_size(B, Hq, Hkv, D, ctx_max, tree.handle, dt)
    ws, nb = _workspace(nbytes, q.device, ws)
    _check(lib.medusa_tree_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), ctx_max,
                                     tree.handle, B, Hq, Hkv, D, S_cap, float(scale), dt, _ptr(out),
                                     _ptr(ws), nb, _stream(stream)))
    return out


def tree_attention_layers_workspace_size(L, B, Hq, Hkv, D, ctx_max, tree: Tree, dtype) -> int:
    return _lib.load().medusa_tree_attention_layers_workspace_size(
        L, B, Hq, Hkv, D, ctx_max, tree.handle, F32 if dtype == torch.float32 else BF16)


def tree_attention_layers(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          ctx_len: torch.Tensor, ctx_max: int, tree: Tree,
                          scale: Optional[float] = None, out=None, ws=None, stream=None):
    """Every layer in one call: q [L,B,T,Hq,D]; k_cache/v_cache [L,B,Hkv,S_cap,D]
    -> out [L,B,T,Hq,D].  Each layer's block must be contiguous; the layer
    dimension may be strided."""
    lib = _lib.load()
    L, B, T, Hq, D = q.shape
    Hkv, S_cap = k_cache.shape[2], k_cache.shape[3]
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")

    def layered(t):  # the layer dimension may be strided, each layer's block not
        if not t[0].is_contiguous():
            raise ValueError("each layer's block must be contiguous")
        return ctypes.c_void_p(t.data_ptr())

    nbytes = lib.medusa_tree_attention_layers_workspace_size(L, B, Hq, Hkv, D, ctx_max,
                                                             tree.handle, dt)
    ws, nb = _workspace(nbytes, q.device, ws)
    _check(lib.medusa_tree_attention_layers(
        layered(q), layered(k_cache), layered(v_cache), q.stride(0), k_cache.stride(0),
        out.stride(0), L,
        _ptr(ctx_len), ctx_max, tree.handle, B, Hq, Hkv, D, S_cap, float(scale), dt, layered(out),
        _ptr(ws), nb, _stream(stream)))
    return out


def accept_workspace_size(B, V, tree: Tree, temperature: float) -> int:
    return _lib.load().medusa_accept_workspace_size(B, V, tree.handle, float(temperature))


def accept_paths(base_logits: torch.Tensor, head_logits: Optional[torch.Tensor],
                 tree_tokens: torch.Tensor, tree: Tree, u_accept: Optional[torch.Tensor],
                 u_sample: Optional[torch.Tensor], temperature: float, outs=None, ws=None,
                 stream=None):
    """-> (accept_len [B], out_tokens [B,K+1], out_nodes [B,K+1]) int32."""
    lib = _lib.load()
    B, T, V = base_logits.shape
    dev = base_logits.device
    if outs is None:
        outs = (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, tree.K + 1), dtype=torch.int32, device=dev),
                torch.empty((B, tree.K + 1), dtype=torch.int32, device=dev))
    acc, toks, nodes = outs
    ws, nb = _workspace(lib.medusa_accept_workspace_size(B, V, tree.handle, float(temperature)),
                        dev, ws)
    _check(lib.medusa_accept_paths(_ptr(base_logits), _ptr(head_logits), _ptr(tree_tokens),
                                   tree.handle, _ptr(u_accept), _ptr(u_sample), float(temperature),
                                   B, V, _ptr(acc), _ptr(toks), _ptr(nodes), _ptr(ws), nb,
                                   _stream(stream)))
    return acc, toks, nodes


def commit_accepted(k_cache: torch.Tensor, v_cache: torch.Tensor, accept_len: torch.Tensor,
                    out_nodes: torch.Tensor, out_tokens: torch.Tensor, ctx_len: torch.Tensor,
                    tree: Tree, ctx_next=None, root_next=None, stream=None):
    """k_cache/v_cache [L,B,Hkv,S_cap,D] or [B,Hkv,S_cap,D] (updated in place)
    -> (ctx_next [B], root_next [B]) int32."""
    lib = _lib.load()
    if k_cache.dim() == 4:
        L, (B, Hkv, S_cap, D) = 1, k_cache.shape
        stride = B * Hkv * S_cap * D
    else:
        L, B, Hkv, S_cap, D = k_cache.shape
        stride = k_cache.stride(0)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    dev = k_cache.device
    if ctx_next is None:
        ctx_next = torch.empty(B, dtype=torch.int32, device=dev)
    if root_next is None:
        root_next = torch.empty(B, dtype=torch.int32, device=dev)
    _check(lib.medusa_commit_accepted(_ptr(k_cache), _ptr(v_cache), stride, L, _ptr(accept_len),
                                      _ptr(out_nodes), _ptr(out_tokens), _ptr(ctx_len),
                                      _ptr(ctx_next), _ptr(root_next), tree.handle, B, Hkv, D,
                                      S_cap, _dt(k_cache), _stream(stream)))
    return ctx_next, root_next


def tree_optimize(p_accept, k_per_depth, T: int):
    """Host-only: the T-node tree maximising expected accepted nodes under the
    acceptance table p_accept [K][kmax] -> (parent, rank, expected)."""
    lib = _lib.load()
    p = np.ascontiguousarray(np.asarray(p_accept, dtype=np.float64))
    kpd = _i32(k_per_depth)
    K, kmax = p.shape
    parent = np.zeros(T, np.int32)
    rank = np.zeros(T, np.int32)
    e = ctypes.c_double()
    _check(lib.medusa_tree_optimize(p.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), K, kmax,
                                    _p32(kpd), T, _p32(parent), _p32(rank), ctypes.byref(e)))
    return parent, rank, e.value


def read_probe(buf: torch.Tensor, partials=None, stream=None) -> torch.Tensor:
    """Diagnostics: streaming read of a device tensor (contiguous, bytes a
    multiple of 16) -> per-workgroup XOR folds [medusa_read_probe_partials()]
    uint32 (as int32); their XOR is the XOR of every 32-bit word of buf."""
    lib = _lib.load()
    if partials is None:
        partials = torch.empty(lib.medusa_read_probe_partials(), dtype=torch.int32, device=buf.device)
    _check(lib.medusa_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(partials),
                                 _stream(stream)))
    return partials
