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
