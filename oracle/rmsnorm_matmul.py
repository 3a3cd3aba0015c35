"""fp64 CPU oracle for RMSNorm followed by a MatMul.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
and imports nothing from it; it reads only numpy arrays.

Source: the Cleave paper ("Cleave: Scaling Tensor Program Optimization via
Decoupled Algebraic Search and Operator Scheduling", paperpeel.com text).

* §1 and Fig. 1: RMSNorm feeds a Matmul; moving RMSNorm's row-wise scaling
  after the Matmul lets the two reductions (the row's sum of squares and the
  Matmul's dot products) consume the same input tile, and the normalised input
  is never materialised.  ``rmsnorm_matmul`` is the graph before that rewrite,
  written out; ``rmsnorm_matmul_split`` is the rewritten graph.
* §2.2 "Split-K" and Fig. 3: a reduction of length K is the sum of s partial
  reductions over contiguous parts.  Both reductions of the rewritten graph run
  over K, so both split: ``rmsnorm_matmul_partials`` gives the per-part dot
  products and sums of squares, ``rmsnorm_matmul_combine`` adds them up and
  then applies the row scale.
* §7.3: the RMSNorm+MatMul subgraph is evaluated with Llama-3 8B shapes in a
  prefill and a decode setting.

Readings where the pages are silent (listed with their reasons in the design
notes of the repository): RMSNorm(x)_k = x_k g_k / sqrt(mean_k(x^2) + eps)
with a per-column gain g and eps = 1e-5 (the Llama-3 value); the Matmul is a
linear layer with weights stored [N, K], so Y = RMSNorm(X) W^T.

Precision: every product and sum is fp64 on the (already rounded) inputs.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

__all__ = ["RMS_EPS", "rmsnorm", "rmsnorm_matmul", "rmsnorm_matmul_partials",
           "rmsnorm_matmul_combine", "rmsnorm_matmul_split"]

RMS_EPS = 1e-5


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Row-wise RMSNorm of x [M, K] with gain g [K] (Cleave §1, Fig. 1)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    mean_sq = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * g[None, :]


def rmsnorm_matmul(x: np.ndarray, g: np.ndarray, w: np.ndarray,
                   eps: float = RMS_EPS) -> np.ndarray:
    """Y [M, N] = RMSNorm(X) W^T with X [M, K], g [K], W [N, K], float64.

    The graph before the rewrite (Cleave Fig. 1): the normalised input is
    materialised, then multiplied.
    """
    w = np.asarray(w, dtype=np.float64)
    if w.shape[1] != np.shape(x)[1] or np.shape(g) != (np.shape(x)[1],):
        raise ValueError("shapes: x [M, K], g [K], w [N, K]")
    return np.matmul(rmsnorm(x, g, eps), w.T)


def rmsnorm_matmul_partials(x: np.ndarray, g: np.ndarray, w: np.ndarray,
                            bounds: Sequence[int]):
    """Split-K partials of the rewritten graph (Cleave §2.2 "Split-K").

    ``bounds`` = [c_0 = 0, c_1, ..., c_s = K]; part j covers columns
    [c_j, c_{j+1}).  Returns U [s, M, N] with U_j = (X * g)[:, part] W[:, part]^T
    (the Matmul on the unnormalised input) and SSQ [s, M], the rows' sums of
    squares over the same part.
    """
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = x.shape[1]
    if bounds[0] != 0 or bounds[-1] != k or any(b > a for a, b in zip(bounds[1:], bounds[:-1])):
        raise ValueError("bounds must run from 0 to K, non-decreasing")
    xg = x * g[None, :]
    u, ssq = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        u.append(np.matmul(xg[:, lo:hi], w[:, lo:hi].T))
        ssq.append(np.sum(x[:, lo:hi] ** 2, axis=1))
    return np.stack(u), np.stack(ssq)


def rmsnorm_matmul_combine(u_parts: np.ndarray, ssq_parts: np.ndarray, k: int,
                           eps: float = RMS_EPS) -> np.ndarray:
    """Reduce the parts over s, then apply RMSNorm's row scale after the
    Matmul (Cleave Fig. 1, right): Y = (sum_j U_j) / sqrt(sum_j SSQ_j / K + eps)."""
    u = np.sum(u_parts, axis=0)
    ssq = np.sum(ssq_parts, axis=0)
    return u / np.sqrt(ssq / k + eps)[:, None]


def rmsnorm_matmul_split(x, g, w, bounds, eps: float = RMS_EPS) -> np.ndarray:
    """The rewritten, split graph end to end: equal to ``rmsnorm_matmul``."""
    u, ssq = rmsnorm_matmul_partials(x, g, w, bounds)
    return rmsnorm_matmul_combine(u, ssq, np.shape(x)[1], eps)
