"""Shared helpers of the GPU parity tests (comparison metrics, transfers)."""
import numpy as np
import torch

# Error metric: per output row (one vocab vector of logits, or one D-vector of
# attention output) max|gpu - oracle| / max|oracle|.  Bounds: fp32 path 1e-4,
# bf16 path 2e-2.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / np.maximum(den, 1e-300)))


def announce(*what):
    """Print (and flush) what the next GPU step runs, so a crash names its case."""
    print("[gpu-case]", *what, flush=True)


# Rejection-sampling decisions are taken in fp64 on both sides, in different
# summation orders.  A GPU path that differs from the oracle's is accepted
# only where the oracle's own margin at the FIRST decision on which the two
# walks part is below this bound (either answer is then correct); every such
# case is counted in TIES.
TIE = 1e-9
TIES = {"count": 0}


def first_divergence_margin(res, g_acc: int, g_nodes) -> float:
    """The oracle's margin at the first decision where the GPU's walk left the
    oracle's.  Both walks test the children of a node in rank order, so up to
    that decision they test the same children; a child's test went the same
    way iff the child is on both accepted paths or on neither.  If every child
    test agrees the paths are equal and the final draw differs."""
    g_path = set(int(n) for n in list(g_nodes)[:int(g_acc) + 1])
    o_path = set(int(n) for n in res.nodes)
    for kind, node, margin in res.trace:
        if kind != "accept" or (node in g_path) != (node in o_path):
            return margin
    raise AssertionError("paths differ but no decision of the oracle's walk does")


def assert_same_decisions(g, r, res, allow_ties: bool = True):
    """GPU (accept_len, out_tokens, out_nodes) equal the oracle's, except a
    sequence whose first diverging decision is an oracle tie (counted)."""
    g_acc, g_tok, g_node = (np.asarray(x) for x in g)
    r_acc, r_tok, r_node = r
    for b in range(len(r_acc)):
        if (g_acc[b] == r_acc[b] and np.array_equal(g_tok[b], r_tok[b])
                and np.array_equal(g_node[b], r_node[b])):
            continue
        m = first_divergence_margin(res[b], g_acc[b], g_node[b])
        msg = (f"b={b}: gpu {g_acc[b]} {g_tok[b]} {g_node[b]} vs oracle {r_acc[b]} {r_tok[b]} "
               f"{r_node[b]}; oracle margin at the first diverging decision {m:.3e}")
        assert allow_ties and m < TIE, msg
        TIES["count"] += 1
        print(f"[tie] {msg}", flush=True)
