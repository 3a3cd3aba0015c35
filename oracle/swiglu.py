"""fp64 CPU oracle for SwiGLU (two MatMuls on one input, then a gated
product).  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
and imports nothing from it; it reads only numpy arrays.

Source: the Cleave paper ("Cleave: Scaling Tensor Program Optimization via
Decoupled Algebraic Search and Operator Scheduling", paperpeel.com text).

* §7.3: SwiGLU is one of the dense transformer subgraphs evaluated, with
  Llama-3 8B shapes.  Both of its MatMuls reduce over K and read the same X,
  so one loop over K can feed both (horizontal fusion).
* §2.2 "Split-K": each MatMul's reduction over K is the sum of partial
  reductions over contiguous parts.  The gate is nonlinear, so the parts of
  both MatMuls are added up before it is applied (``swiglu_combine``).

Readings where the pages are silent (listed with their reasons in the design
notes of the repository): SwiGLU(X) = silu(X W_gate^T) * (X W_up^T) with
silu(z) = z / (1 + exp(-z)), the weights stored [N, K] like linear layers.

Precision: every product and sum is fp64 on the (already rounded) inputs.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

__all__ = ["silu", "swiglu", "swiglu_partials", "swiglu_combine", "swiglu_split"]


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z), written without overflow for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def swiglu(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """H [M, N] = silu(X W_gate^T) * (X W_up^T); X [M, K], W_* [N, K], float64."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wu = np.asarray(w_up, dtype=np.float64)
    if wg.shape != wu.shape or wg.shape[1] != x.shape[1]:
        raise ValueError("shapes: x [M, K], w_gate and w_up [N, K]")
    return silu(np.matmul(x, wg.T)) * np.matmul(x, wu.T)


def swiglu_partials(x, w_gate, w_up, bounds: Sequence[int]):
    """Split-K partials (Cleave §2.2 "Split-K"): for part j over columns
    [c_j, c_{j+1}), G_j = X[:, part] W_gate[:, part]^T and U_j likewise.
    Returns (G [s, M, N], U [s, M, N])."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    wu = np.asarray(w_up, dtype=np.float64)
    k = x.shape[1]
    if bounds[0] != 0 or bounds[-1] != k or any(b > a for a, b in zip(bounds[1:], bounds[:-1])):
        raise ValueError("bounds must run from 0 to K, non-decreasing")
    g, u = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        g.append(np.matmul(x[:, lo:hi], wg[:, lo:hi].T))
        u.append(np.matmul(x[:, lo:hi], wu[:, lo:hi].T))
    return np.stack(g), np.stack(u)


def swiglu_combine(g_parts: np.ndarray, u_parts: np.ndarray) -> np.ndarray:
    """Add the parts of each MatMul over s, then gate: silu(sum G_j) * sum U_j."""
    return silu(np.sum(g_parts, axis=0)) * np.sum(u_parts, axis=0)


def swiglu_split(x, w_gate, w_up, bounds) -> np.ndarray:
    """The split graph end to end: equal to ``swiglu``."""
    g, u = swiglu_partials(x, w_gate, w_up, bounds)
    return swiglu_combine(g, u)
