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


def _ptr(t: Optional[torch.Tensor], name: str = "tensor"):
    """Device pointer of a contiguous tensor on the current HIP device."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    _on_device(t, name)
    return ctypes.c_void_p(t.data_ptr())


def _on_device(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory (got a {t.device} tensor)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _expect(t: Optional[torch.Tensor], name: str, shape, dtypes, optional: bool = False):
    """Checks a tensor argument's shape and dtype before anything reaches the
    library (a tensor smaller than the call assumes would be read or written
    past its end)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)} (got {t.dtype})")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)} "
                         f"(got {tuple(t.shape)})")


def _ws_bytes(ws: Optional[torch.Tensor]) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


_FLOAT = (torch.float32, torch.bfloat16)


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
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous torch tensor")
    return ws, _ws_bytes(ws)


def heads_workspace_size(M: int, H: int, K: int, dtype: torch.dtype) -> int:
    return _lib.load().medusa_heads_workspace_size(M, H, K, F32 if dtype == torch.float32 else BF16)


def heads(hidden: torch.Tensor, w1: torch.Tensor, wlm: torch.Tensor, logits=None, ws=None,
          stream=None) -> torch.Tensor:
    """hidden [M,H]; w1 [K,H,H]; wlm [K,V,H] or [V,H] (shared) -> logits [M,K,V] fp32."""
    lib = _lib.load()
    M, H, K, V, shared = _heads_shapes(hidden, w1, wlm)
    if logits is None:
        logits = torch.empty((M, K, V), dtype=torch.float32, device=hidden.device)
    _expect(logits, "logits", (M, K, V), torch.float32)
    dt = _dt(hidden)
    ws, nb = _workspace(lib.medusa_heads_workspace_size(M, H, K, dt), hidden.device, ws)
    _check(lib.medusa_heads(_ptr(hidden, "hidden"), _ptr(w1, "w1"), H * H, _ptr(wlm, "wlm"),
                            0 if shared else V * H, M, H, V, K, dt, _ptr(logits, "logits"),
                            _ptr(ws, "ws"), nb, _stream(stream)))
    return logits


def _heads_shapes(hidden, w1, wlm):
    """(M, H, K, V, shared) of the heads' operands, checked against each other."""
    if hidden.dim() != 2 or w1.dim() != 3 or wlm.dim() not in (2, 3):
        raise ValueError("need hidden [M,H], w1 [K,H,H] and wlm [K,V,H] or [V,H]")
    M, H = hidden.shape
    K = w1.shape[0]
    shared = wlm.dim() == 2
    V = wlm.shape[0] if shared else wlm.shape[1]
    _expect(hidden, "hidden", (M, H), _FLOAT)
    _expect(w1, "w1", (K, H, H), hidden.dtype)
    _expect(wlm, "wlm", (V, H) if shared else (K, V, H), hidden.dtype)
    return M, H, K, V, shared


def tree_candidates_workspace_size(B, V, tree: Tree) -> int:
    return _lib.load().medusa_tree_candidates_workspace_size(B, V, tree.handle)


def tree_candidates(head_logits: torch.Tensor, root: torch.Tensor, ctx_len: torch.Tensor,
                    tree: Tree, topk_idx=None, tree_tokens=None, pos=None, ws=None, stream=None):
    """head_logits [B,K,V] fp32 -> (topk_idx [B,K,kmax], tree_tokens [B,T], pos [B,T]) int32."""
    lib = _lib.load()
    if head_logits.dim() != 3:
        raise ValueError("head_logits must be [B,K,V]")
    B, K, V = head_logits.shape
    _expect(head_logits, "head_logits", (B, tree.K, V), torch.float32)
    _expect(root, "root", (B,), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    dev = head_logits.device
    if topk_idx is None:
        topk_idx = torch.empty((B, tree.K, tree.kmax), dtype=torch.int32, device=dev)
    if tree_tokens is None:
        tree_tokens = torch.empty((B, tree.T), dtype=torch.int32, device=dev)
    if pos is None:
        pos = torch.empty((B, tree.T), dtype=torch.int32, device=dev)
    _expect(topk_idx, "topk_idx", (B, tree.K, tree.kmax), torch.int32)
    _expect(tree_tokens, "tree_tokens", (B, tree.T), torch.int32)
    _expect(pos, "pos", (B, tree.T), torch.int32)
    ws, nb = _workspace(lib.medusa_tree_candidates_workspace_size(B, V, tree.handle), dev, ws)
    _check(lib.medusa_tree_candidates(_ptr(head_logits, "head_logits"), _ptr(root, "root"),
                                      _ptr(ctx_len, "ctx_len"), tree.handle, B, V,
                                      _ptr(topk_idx, "topk_idx"), _ptr(tree_tokens, "tree_tokens"),
                                      _ptr(pos, "pos"), _ptr(ws, "ws"), nb, _stream(stream)))
    return topk_idx, tree_tokens, pos


def heads_dense(hidden: torch.Tensor, w1: torch.Tensor, wlm: torch.Tensor, tree: "Tree",
                values: bool = True, logits=None, outs=None, ws=None, stream=None):
    """Dense-variant heads: hidden [M,H]; w1 [K,H,H]; wlm [K,V,H] or [V,H]
    (shared) -> (topk_idx [M,K,kmax] int32, topk_val [M,K,kmax] fp32 or None).
    ``logits`` (a [M,K,V] fp32 tensor) also receives every logit."""
    lib = _lib.load()
    M, H, K, V, shared = _heads_shapes(hidden, w1, wlm)   # K against the tree: the library
    dt = _dt(hidden)
    dev = hidden.device
    if outs is None:
        outs = (torch.empty((M, K, tree.kmax), dtype=torch.int32, device=dev),
                torch.empty((M, K, tree.kmax), dtype=torch.float32, device=dev) if values else None)
    idx, val = outs
    _expect(idx, "topk_idx", (M, K, tree.kmax), torch.int32)
    _expect(val, "topk_val", (M, K, tree.kmax), torch.float32, optional=True)
    _expect(logits, "logits", (M, K, V), torch.float32, optional=True)
    nbytes = lib.medusa_heads_dense_workspace_size(M, H, V, K, tree.handle, dt)
    ws, nb = _workspace(nbytes, dev, ws)
    _check(lib.medusa_heads_dense(_ptr(hidden, "hidden"), _ptr(w1, "w1"), H * H, _ptr(wlm, "wlm"),
                                  0 if shared else V * H, M, H, V, K, tree.handle, dt,
                                  _ptr(idx, "topk_idx"), _ptr(val, "topk_val"),
                                  _ptr(logits, "logits"), _ptr(ws, "ws"), nb, _stream(stream)))
    return idx, val


def tree_attention_workspace_size(B, Hq, Hkv, D, ctx_max, tree: Tree, dtype) -> int:
    return _lib.load().medusa_tree_attention_workspace_size(
        B, Hq, Hkv, D, ctx_max, tree.handle, F32 if dtype == torch.float32 else BF16)


def tree_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   ctx_len: torch.Tensor, ctx_max: int, tree: Tree, scale: Optional[float] = None,
                   out=None, ws=None, stream=None) -> torch.Tensor:
    """q [B,T,Hq,D]; k_cache/v_cache [B,Hkv,S_cap,D] -> out [B,T,Hq,D]."""
    lib = _lib.load()
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("need q [B,T,Hq,D] and k_cache/v_cache [B,Hkv,S_cap,D]")
    B, T, Hq, D = q.shape
    Hkv, S_cap = k_cache.shape[1], k_cache.shape[2]
    _expect(q, "q", (B, tree.T, Hq, D), _FLOAT)
    _expect(k_cache, "k_cache", (B, Hkv, S_cap, D), q.dtype)
    _expect(v_cache, "v_cache", (B, Hkv, S_cap, D), q.dtype)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", tuple(q.shape), q.dtype)
    nbytes = lib.medusa_tree_attention_workspace_size(B, Hq, Hkv, D, ctx_max, tree.handle, dt)
    ws, nb = _workspace(nbytes, q.device, ws)
    _check(lib.medusa_tree_attention(_ptr(q, "q"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache"),
                                     _ptr(ctx_len, "ctx_len"), ctx_max, tree.handle, B, Hq, Hkv, D,
                                     S_cap, float(scale), dt, _ptr(out, "out"), _ptr(ws, "ws"), nb,
                                     _stream(stream)))
    return out


ATTENTION_SCRATCH_BYTES = 32 << 20


def tree_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           ctx_len: torch.Tensor, ctx_max: int, tree: Tree,
                           scale: Optional[float] = None, out=None, stream=None) -> torch.Tensor:
    """medusa_tree_attention_noalloc: tree_attention with the split partials in
    the library's fixed per-device scratch (no workspace, no allocation in the
    call).  ``out`` must be given by callers that cannot allocate."""
    lib = _lib.load()
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("need q [B,T,Hq,D] and k_cache/v_cache [B,Hkv,S_cap,D]")
    B, T, Hq, D = q.shape
    Hkv, S_cap = k_cache.shape[1], k_cache.shape[2]
    _expect(q, "q", (B, tree.T, Hq, D), _FLOAT)
    _expect(k_cache, "k_cache", (B, Hkv, S_cap, D), q.dtype)
    _expect(v_cache, "v_cache", (B, Hkv, S_cap, D), q.dtype)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", tuple(q.shape), q.dtype)
    _check(lib.medusa_tree_attention_noalloc(_ptr(q, "q"), _ptr(k_cache, "k_cache"),
                                             _ptr(v_cache, "v_cache"), _ptr(ctx_len, "ctx_len"),
                                             ctx_max, tree.handle, B, Hq, Hkv, D, S_cap,
                                             float(scale), dt, _ptr(out, "out"), _stream(stream)))
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
    if q.dim() != 5 or k_cache.dim() != 5:
        raise ValueError("need q [L,B,T,Hq,D] and k_cache/v_cache [L,B,Hkv,S_cap,D]")
    L, B, T, Hq, D = q.shape
    Hkv, S_cap = k_cache.shape[2], k_cache.shape[3]
    _expect(q, "q", (L, B, tree.T, Hq, D), _FLOAT)
    _expect(k_cache, "k_cache", (L, B, Hkv, S_cap, D), q.dtype)
    _expect(v_cache, "v_cache", (L, B, Hkv, S_cap, D), q.dtype)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    dt = _dt(q)
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", tuple(q.shape), q.dtype)

    def layered(t):  # the layer dimension may be strided, each layer's block not
        if not t[0].is_contiguous():
            raise ValueError("each layer's block must be contiguous")
        _on_device(t, "layered tensor")
        return ctypes.c_void_p(t.data_ptr())

    nbytes = lib.medusa_tree_attention_layers_workspace_size(L, B, Hq, Hkv, D, ctx_max,
                                                             tree.handle, dt)
    ws, nb = _workspace(nbytes, q.device, ws)
    _check(lib.medusa_tree_attention_layers(
        layered(q), layered(k_cache), layered(v_cache), q.stride(0), k_cache.stride(0),
        out.stride(0), L,
        _ptr(ctx_len, "ctx_len"), ctx_max, tree.handle, B, Hq, Hkv, D, S_cap, float(scale), dt,
        layered(out), _ptr(ws, "ws"), nb, _stream(stream)))
    return out


def accept_workspace_size(B, V, tree: Tree, temperature: float) -> int:
    return _lib.load().medusa_accept_workspace_size(B, V, tree.handle, float(temperature))


def accept_paths(base_logits: torch.Tensor, head_logits: Optional[torch.Tensor],
                 tree_tokens: torch.Tensor, tree: Tree, u_accept: Optional[torch.Tensor],
                 u_sample: Optional[torch.Tensor], temperature: float, outs=None, ws=None,
                 stream=None):
    """-> (accept_len [B], out_tokens [B,K+1], out_nodes [B,K+1]) int32."""
    lib = _lib.load()
    if base_logits.dim() != 3:
        raise ValueError("base_logits must be [B,T,V]")
    B, T, V = base_logits.shape
    # head logits and uniforms may be absent (greedy); the library rejects a
    # missing one that the temperature needs
    _expect(base_logits, "base_logits", (B, tree.T, V), torch.float32)
    _expect(head_logits, "head_logits", (B, tree.K, V), torch.float32, optional=True)
    _expect(tree_tokens, "tree_tokens", (B, tree.T), torch.int32)
    _expect(u_accept, "u_accept", (B, tree.T), torch.float32, optional=True)
    _expect(u_sample, "u_sample", (B, tree.T), torch.float32, optional=True)
    dev = base_logits.device
    if outs is None:
        outs = (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty((B, tree.K + 1), dtype=torch.int32, device=dev),
                torch.empty((B, tree.K + 1), dtype=torch.int32, device=dev))
    acc, toks, nodes = outs
    _expect(acc, "accept_len", (B,), torch.int32)
    _expect(toks, "out_tokens", (B, tree.K + 1), torch.int32)
    _expect(nodes, "out_nodes", (B, tree.K + 1), torch.int32)
    ws, nb = _workspace(lib.medusa_accept_workspace_size(B, V, tree.handle, float(temperature)),
                        dev, ws)
    _check(lib.medusa_accept_paths(_ptr(base_logits, "base_logits"), _ptr(head_logits, "head_logits"),
                                   _ptr(tree_tokens, "tree_tokens"), tree.handle,
                                   _ptr(u_accept, "u_accept"), _ptr(u_sample, "u_sample"),
                                   float(temperature), B, V, _ptr(acc, "accept_len"),
                                   _ptr(toks, "out_tokens"), _ptr(nodes, "out_nodes"),
                                   _ptr(ws, "ws"), nb, _stream(stream)))
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
    elif k_cache.dim() == 5:
        L, B, Hkv, S_cap, D = k_cache.shape
        stride = k_cache.stride(0)
    else:
        raise ValueError("k_cache must be [L,B,Hkv,S_cap,D] or [B,Hkv,S_cap,D]")
    _expect(k_cache, "k_cache", tuple(k_cache.shape), _FLOAT)
    _expect(v_cache, "v_cache", tuple(k_cache.shape), k_cache.dtype)
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    _expect(accept_len, "accept_len", (B,), torch.int32)
    _expect(out_nodes, "out_nodes", (B, tree.K + 1), torch.int32)
    _expect(out_tokens, "out_tokens", (B, tree.K + 1), torch.int32)
    _expect(ctx_len, "ctx_len", (B,), torch.int32)
    dev = k_cache.device
    if ctx_next is None:
        ctx_next = torch.empty(B, dtype=torch.int32, device=dev)
    if root_next is None:
        root_next = torch.empty(B, dtype=torch.int32, device=dev)
    _expect(ctx_next, "ctx_next", (B,), torch.int32)
    _expect(root_next, "root_next", (B,), torch.int32)

    def base(t, name):  # the layer dimension may be strided, each layer's block not
        blk = t if t.dim() == 4 else t[0]
        if not blk.is_contiguous():
            raise ValueError(f"each layer's block of {name} must be contiguous")
        _on_device(t, name)
        return ctypes.c_void_p(t.data_ptr())

    _check(lib.medusa_commit_accepted(base(k_cache, "k_cache"), base(v_cache, "v_cache"), stride, L,
                                      _ptr(accept_len, "accept_len"), _ptr(out_nodes, "out_nodes"),
                                      _ptr(out_tokens, "out_tokens"), _ptr(ctx_len, "ctx_len"),
                                      _ptr(ctx_next, "ctx_next"), _ptr(root_next, "root_next"),
                                      tree.handle, B, Hkv, D, S_cap, _dt(k_cache), _stream(stream)))
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
    n = lib.medusa_read_probe_partials()
    if partials is None:
        partials = torch.empty(n, dtype=torch.int32, device=buf.device)
    _expect(partials, "partials", (n,), torch.int32)
    _check(lib.medusa_read_probe(_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                 _ptr(partials, "partials"), _stream(stream)))
    return partials
