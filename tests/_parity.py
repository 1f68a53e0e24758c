"""Helpers of the GPU parity tests: moving seeded inputs to the device,
error metrics, and the tolerances every comparison uses.

Tolerances:
  bf16 outputs       rel-L2 <= 5e-3 and max-abs <= 2e-2 over the tensor
  f32 outputs        rel-L2 <= 1e-5 and max-abs <= 1e-5
  lse                max-abs <= 1e-3 (bf16 inputs), 1e-5 (f32 inputs).  The kernels
                     take the scores from exact bf16 products summed in float32
                     and normalise with float32 sums of the unrounded
                     probabilities, so lse carries only float32 rounding
                     (about 1e-6 relative on values of order 10).
  key_score          rel-L2 <= 1e-4 (bf16 inputs), 1e-6 (f32 inputs)
  selected indices   bit-exact
"""
import sys

import numpy as np
import torch

TOL = {
    "bf16": dict(rel_l2=5e-3, max_abs=2e-2, lse=1e-3, score_rel_l2=1e-4),
    "f32": dict(rel_l2=1e-5, max_abs=1e-5, lse=1e-5, score_rel_l2=1e-6),
}


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, device="cuda:0") -> torch.Tensor:
    """A seeded numpy array on the GPU: uint16 bf16 bits -> bfloat16."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """A GPU result as float64 numpy (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0


def assert_close(x, ref, kind, what=""):
    t = TOL[kind]
    assert np.all(np.isfinite(x)), f"{what}: non-finite output"
    r, m = rel_l2(x, ref), max_abs(x, ref)
    assert r <= t["rel_l2"] and m <= t["max_abs"], f"{what}: rel-L2 {r:.3e}, max-abs {m:.3e} ({kind})"
    return r, m
