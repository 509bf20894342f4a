"""Seeded synthetic inputs for the Medusa verify step.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds workload shapes and random-number recipes only: nothing in
it computes any part of the method (no heads, no top-k, no tree masks, no
attention, no acceptance).  The one structural helper, ``cost_ordered_tree``,
produces the *static tree topology* that both sides receive as an input
(parent/rank arrays); the method itself treats the topology as given data.

Recipe (stated once, used everywhere):

* Every tensor slice gets its own seed ``SeedSequence([0x4D454455, cfg_id,
  tensor_id, layer])``; the first 63 bits of its state seed a
  ``torch.Generator`` on the device the tensor is made on.  Host tensors come
  from torch's CPU generator, device tensors from torch's HIP generator; the
  two streams differ, so a test that compares both sides generates once and
  copies the inputs where the oracle needs them.
* Normal draws are fp32 and are rounded to bf16 by torch's round-to-nearest-
  even conversion for the bf16 workloads.
* "N(mu, s)" in the workload descriptions is read with ``s`` as the standard
  deviation.
"""
from __future__ import annotations

import dataclasses
import itertools
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

SEED_TAG = 0x4D454455  # "MEDU"

# tensor ids for SeedSequence
T_HIDDEN, T_W1, T_WLM, T_ROOTVEC, T_Q, T_K, T_V, T_BASE, T_UACC, T_USMP, \
    T_TREETOK, T_PLANT, T_HEADLOG, T_MISC = range(14)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one verify-step workload (Vicuna/Zephyr-shaped or tiny)."""
    cfg_id: int
    name: str
    dtype: str            # "f32" or "bf16": storage type of weights, Q, K/V
    B: int                # sequences per step
    H: int                # hidden size
    V: int                # vocabulary
    K: int                # Medusa heads
    topk: Tuple[int, ...] # candidates per depth (len == K)
    T: int                # tree nodes, root included
    L: int                # attention layers
    Hq: int
    Hkv: int
    D: int
    ctx: int              # cached context tokens per sequence
    temperature: Tuple[float, ...]   # 0.0 means greedy acceptance
    base_logit_std: float = 1.0
    weight_std: float = 0.02

    @property
    def S(self) -> int:
        return self.ctx + self.T

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload(0, "tiny-fp32", "f32", B=1, H=256, V=1024, K=3, topk=(2, 2, 2),
                 T=8, L=1, Hq=4, Hkv=4, D=64, ctx=128, temperature=(0.0, 1.0)),
        Workload(1, "vicuna7b-shaped", "bf16", B=1, H=4096, V=32000, K=4,
                 topk=(10, 10, 5, 5), T=64, L=32, Hq=32, Hkv=32, D=128, ctx=2048,
                 temperature=(0.0,)),
        Workload(2, "vicuna13b-shaped", "bf16", B=4, H=5120, V=32000, K=5,
                 topk=(10, 10, 5, 5, 5), T=64, L=40, Hq=40, Hkv=40, D=128, ctx=4096,
                 temperature=(0.7,), base_logit_std=2.0),
        Workload(3, "vicuna33b-shaped", "bf16", B=1, H=6656, V=32000, K=4,
                 topk=(10, 10, 5, 5), T=96, L=60, Hq=52, Hkv=52, D=128, ctx=8192,
                 temperature=(0.0, 1.0)),
        Workload(4, "zephyr7b-shaped", "bf16", B=8, H=4096, V=32000, K=5,
                 topk=(10, 10, 5, 5, 5), T=64, L=32, Hq=32, Hkv=8, D=128, ctx=16384,
                 temperature=(1.0,)),
    ]
}
WORKLOAD_ORDER = ["tiny-fp32", "vicuna7b-shaped", "vicuna13b-shaped",
                  "vicuna33b-shaped", "zephyr7b-shaped"]


def seed_for(cfg_id: int, tensor_id: int, layer: int = 0, extra: int = 0) -> int:
    ss = np.random.SeedSequence([SEED_TAG, cfg_id, tensor_id, layer, extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0, std) fp32 draws, then cast to ``dtype`` (bf16 cast is RNE)."""
    x = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def uniform(shape, seed: int, device="cpu") -> torch.Tensor:
    """U[0,1) fp32 draws."""
    return torch.rand(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def torch_dtype(w: Workload) -> torch.dtype:
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


# ---------------------------------------------------------------------------
# Static tree topology (an input of the method)
# ---------------------------------------------------------------------------

def cost_ordered_tree(topk: Sequence[int], T: int) -> Tuple[np.ndarray, np.ndarray]:
    """Static tree of T nodes (root included) from per-depth candidate counts.

    Reading of the pages (they never list a topology, only a cartesian example
    and a 32-64 node guideline): among all rank tuples (r_1..r_d), d <= K,
    r_i < topk[i], keep the T-1 with the smallest sum(r_i + 1), ties broken by
    depth and then lexicographically.  A child always costs more than its
    parent, so the kept set is prefix-closed.  Nodes are numbered
    breadth-first by (depth, tuple): parent[n] < n and siblings are contiguous
    in rank order.  Returns (parent, rank) int32 arrays; parent[0] = -1.
    """
    K = len(topk)
    tuples: List[Tuple[int, ...]] = []
    for d in range(1, K + 1):
        tuples.extend(itertools.product(*[range(k) for k in topk[:d]]))
    if T - 1 > len(tuples):
        raise ValueError(f"T={T} exceeds the {len(tuples) + 1} nodes of the full tree")
    tuples.sort(key=lambda t: (sum(r + 1 for r in t), len(t), t))
    kept = sorted(tuples[:T - 1], key=lambda t: (len(t), t))
    index = {(): 0}
    parent = [-1]
    rank = [0]
    for n, t in enumerate(kept, start=1):
        index[t] = n
        parent.append(index[t[:-1]])
        rank.append(t[-1])
    return np.asarray(parent, np.int32), np.asarray(rank, np.int32)


def cartesian_tree(topk: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Full cartesian tree (every rank tuple of every depth), BFS-numbered."""
    tuples = [()]
    for d in range(1, len(topk) + 1):
        tuples.extend(itertools.product(*[range(k) for k in topk[:d]]))
    index = {(): 0}
    parent, rank = [-1], [0]
    for n, t in enumerate(tuples[1:], start=1):
        index[t] = n
        parent.append(index[t[:-1]])
        rank.append(t[-1])
    return np.asarray(parent, np.int32), np.asarray(rank, np.int32)


def chain_tree(depth: int) -> Tuple[np.ndarray, np.ndarray]:
    """Root followed by a single path of ``depth`` nodes."""
    parent = np.arange(-1, depth, dtype=np.int32)
    return parent, np.zeros(depth + 1, np.int32)


def random_tree(T: int, topk: Sequence[int], seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """A random valid tree: each new node attaches to a random node that still
    has a free rank slot and depth < K, taking a random free rank.  Nodes are
    renumbered breadth-first (depth, then creation order) so parent[n] < n."""
    rng = np.random.default_rng(seed)
    K = len(topk)
    par, dep, used, rk = [-1], [0], [set()], [0]
    while len(par) < T:
        cands = [u for u in range(len(par)) if dep[u] < K and len(used[u]) < topk[dep[u]]]
        if not cands:
            raise ValueError("tree is full")
        u = int(rng.choice(cands))
        r = int(rng.choice([r for r in range(topk[dep[u]]) if r not in used[u]]))
        used[u].add(r)
        par.append(u)
        dep.append(dep[u] + 1)
        used.append(set())
        rk.append(r)
    order = sorted(range(T), key=lambda n: (dep[n], n))
    new_id = {old: i for i, old in enumerate(order)}
    parent = np.array([-1 if par[o] < 0 else new_id[par[o]] for o in order], np.int32)
    rank = np.array([rk[o] for o in order], np.int32)
    return parent, rank


def depths_of(parent: np.ndarray) -> np.ndarray:
    """Depth of each node by walking parent pointers (topology bookkeeping)."""
    d = np.zeros(len(parent), np.int32)
    for n in range(1, len(parent)):
        d[n] = d[parent[n]] + 1
    return d


# ---------------------------------------------------------------------------
# Per-stage input bundles
# ---------------------------------------------------------------------------

def head_inputs(w: Workload, device="cpu", M: Optional[int] = None, shared_lm_head=False):
    """hidden [M,H], w1 [K,H,H] ([out,in]), wlm [K,V,H] (or [V,H] if shared)."""
    dt = torch_dtype(w)
    M = w.B if M is None else M
    hidden = normal((M, w.H), 1.0, seed_for(w.cfg_id, T_HIDDEN), device, dt)
    w1 = normal((w.K, w.H, w.H), w.weight_std, seed_for(w.cfg_id, T_W1), device, dt)
    if shared_lm_head:
        wlm = normal((w.V, w.H), w.weight_std, seed_for(w.cfg_id, T_WLM, 0, 1), device, dt)
    else:
        wlm = normal((w.K, w.V, w.H), w.weight_std, seed_for(w.cfg_id, T_WLM), device, dt)
    return hidden, w1, wlm


def head_logits_input(w: Workload, device="cpu", std: float = 1.0, extra: int = 0):
    """Seeded head logits [B,K,V] fp32 (used where a stage consumes logits)."""
    return normal((w.B, w.K, w.V), std, seed_for(w.cfg_id, T_HEADLOG, 0, extra), device)


def roots(w: Workload, device="cpu") -> torch.Tensor:
    """Root token per sequence: position of the largest entry of a separate
    N(0,1) vector of length V (a stand-in for the base model's last pick)."""
    v = normal((w.B, w.V), 1.0, seed_for(w.cfg_id, T_ROOTVEC), device)
    return v.argmax(dim=1).to(torch.int32)


def attention_inputs(w: Workload, layer: int = 0, device="cpu", S_cap: Optional[int] = None,
                     ctx_lens: Optional[Sequence[int]] = None):
    """q [B,T,Hq,D], k_cache/v_cache [B,Hkv,S_cap,D], ctx_len [B] int32.

    The tree tokens' K/V live in slots ctx..ctx+T-1 of the cache; every slot
    (including unused ones past ctx+T) holds N(0,1) data.
    """
    dt = torch_dtype(w)
    S_cap = w.S if S_cap is None else S_cap
    q = normal((w.B, w.T, w.Hq, w.D), 1.0, seed_for(w.cfg_id, T_Q, layer), device, dt)
    k = normal((w.B, w.Hkv, S_cap, w.D), 1.0, seed_for(w.cfg_id, T_K, layer), device, dt)
    v = normal((w.B, w.Hkv, S_cap, w.D), 1.0, seed_for(w.cfg_id, T_V, layer), device, dt)
    if ctx_lens is None:
        ctx_lens = [w.ctx] * w.B
    ctx = torch.tensor(list(ctx_lens), dtype=torch.int32, device=device)
    return q, k, v, ctx


def tree_tokens_input(w: Workload, parent: np.ndarray, seed_extra: int = 0) -> np.ndarray:
    """Random tree tokens [B,T] with distinct tokens among siblings (what a
    per-head top-k would give), for testing acceptance in isolation."""
    rng = np.random.default_rng(seed_for(w.cfg_id, T_TREETOK, 0, seed_extra))
    T = len(parent)
    tok = np.zeros((w.B, T), np.int32)
    for b in range(w.B):
        tok[b, 0] = rng.integers(w.V)
        groups: Dict[int, List[int]] = {}
        for n in range(1, T):
            groups.setdefault(int(parent[n]), []).append(n)
        for u, kids in groups.items():
            picks = rng.choice(w.V, size=len(kids), replace=False)
            tok[b, kids] = picks
    return tok


def accept_inputs(w: Workload, parent: np.ndarray, tree_tokens: np.ndarray, device="cpu",
                  plant: bool = True, plant_boost: float = 8.0, seed_extra: int = 0):
    """base_logits [B,T,V], head_logits [B,K,V], u_accept/u_sample [B,T].

    With ``plant`` the base logits are raised by ``plant_boost`` at the token of
    one child along a random root-to-leaf path, down to a random depth, so
    that long accepted paths occur (plain N(0,1) logits rarely accept).
    """
    B, T, V, K = w.B, len(parent), w.V, w.K
    base = normal((B, T, V), w.base_logit_std, seed_for(w.cfg_id, T_BASE, 0, seed_extra), "cpu")
    head = normal((B, K, V), w.base_logit_std, seed_for(w.cfg_id, T_HEADLOG, 0, seed_extra), "cpu")
    u_acc = uniform((B, T), seed_for(w.cfg_id, T_UACC, 0, seed_extra), "cpu")
    u_smp = uniform((B, T), seed_for(w.cfg_id, T_USMP, 0, seed_extra), "cpu")
    if plant:
        rng = np.random.default_rng(seed_for(w.cfg_id, T_PLANT, 0, seed_extra))
        kids: Dict[int, List[int]] = {}
        for n in range(1, T):
            kids.setdefault(int(parent[n]), []).append(n)
        for b in range(B):
            u = 0
            stop = int(rng.integers(0, K + 1))
            for _ in range(stop):
                if u not in kids:
                    break
                c = int(rng.choice(kids[u]))
                base[b, u, int(tree_tokens[b, c])] += plant_boost
                # make the head distribution like the planted child too, so
                # rejection sampling accepts it often
                head[b, depths_of(parent)[c] - 1, int(tree_tokens[b, c])] += plant_boost * 0.5
                u = c
    return (base.to(device), head.to(device), u_acc.to(device), u_smp.to(device))


# ---------------------------------------------------------------------------
# Toy target model for multi-step tests: a counter-based hash of the prefix.
# SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014) maps a 64-bit state to a 64-bit output; the
# prefix hash folds every token in, and the logits of a prefix are the top
# 24 bits of SplitMix64(hash ^ f(v)) scaled to [0, 1).  Host-only: the tests
# feed its values to the device path and to the oracle alike.
# ---------------------------------------------------------------------------
_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _splitmix64_np(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.uint64) + np.uint64(0x9E3779B97F4A7C15)
    z = x
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def prefix_hash(tokens, seed: int = 0x51ED) -> int:
    h = seed & _M64
    for t in tokens:
        h = splitmix64(h ^ (int(t) & _M64))
    return h


def toy_target_logits(h: int, V: int) -> np.ndarray:
    """Logits [V] float32 in [0, 1) of the toy target after a prefix with hash h."""
    with np.errstate(over="ignore"):
        v = np.arange(V, dtype=np.uint64) * np.uint64(0x100000001B3) + np.uint64(1)
        z = _splitmix64_np(np.uint64(h) ^ v)
    return ((z >> np.uint64(40)).astype(np.float64) / float(1 << 24)).astype(np.float32)


def toy_kv_rows(token: int, pos: int, layer: int, Hkv: int, D: int) -> np.ndarray:
    """The toy model's K (or V) rows [Hkv][D] in [-1, 1) for a token at a
    position: what a base-model forward would write into the cache."""
    h = splitmix64(prefix_hash([token, pos, layer], seed=0xCAC4E))
    with np.errstate(over="ignore"):
        idx = np.arange(Hkv * D, dtype=np.uint64) * np.uint64(0x2545F4914F6CDD1D)
        z = _splitmix64_np(np.uint64(h) ^ idx)
    u = (z >> np.uint64(40)).astype(np.float64) / float(1 << 24)
    return (2.0 * u - 1.0).astype(np.float32).reshape(Hkv, D)


def toy_draft_logits(greedy_path, V: int, K: int, hit: np.ndarray, seed: int) -> np.ndarray:
    """Head logits [K][V] for one step: N(0, 1) noise, plus +6 on the target's
    greedy token at depth d+1 for the heads d with hit[d] true (drafts that
    are right where hit says so)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((K, V)).astype(np.float32)
    for d in range(K):
        if hit[d]:
            x[d, int(greedy_path[d])] += 6.0
    return x


def toy_draft_logits_ranked(greedy_path, V: int, ranks, seed: int) -> np.ndarray:
    """Head logits [K][V]: N(0, 1) noise in which the target's greedy token at
    depth d+1 sits exactly at rank ranks[d] (no placement when ranks[d] < 0)."""
    rng = np.random.default_rng(seed)
    K = len(ranks)
    x = rng.standard_normal((K, V)).astype(np.float32)
    for d in range(K):
        r = int(ranks[d])
        if r < 0:
            continue
        t = int(greedy_path[d])
        others = np.sort(np.delete(x[d], t))[::-1]
        x[d, t] = others[0] + 1.0 if r == 0 else 0.5 * (others[r - 1] + others[r])
    return x
