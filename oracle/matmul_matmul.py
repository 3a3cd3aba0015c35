"""fp64 CPU oracle for MatMul+MatMul (two consecutive reductions).  TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

Source: the Cleave paper ("Cleave: Scaling Tensor Program Optimization via
Decoupled Algebraic Search and Operator Scheduling", paperpeel.com text).

* §7.3 (subgraph list, Table 1): MatMul+MatMul is one of the two
  "consecutive reduction" dense subgraphs, where iterative tiling and memory
  planning matter; the pages give no shapes for it.
* §5.1 / §5.3 (iterative tiling): the second reduction is tiled along its
  reduction axis and only one tile of the intermediate is live at a time.
  The result is the plain product, so the oracle is that product, written
  with the whole intermediate materialised.

Readings where the pages are silent (listed with their reasons in the design
notes of the repository):

* the subgraph is taken at attention's per-head shapes: O = (tau A B^T) C with
  A [Lq, d], B [n, d], C [n, dv] per (request, head), i.e. the two Matmuls of
  attention with no softmax between them (the case where the [Lq, n]
  intermediate is too large to stage, which is what makes iterative tiling
  matter); heads, GQA grouping, ragged key counts and the optional
  bottom-right causal mask follow the attention oracle;
* tau defaults to 1/sqrt(d), as for attention; a key that is not visible
  contributes nothing (its intermediate entry is 0);
* the kernel rounds the intermediate to bf16 as the second product's operand
  (as attention rounds P); ``error_bounds`` states what that rounding and fp32
  accumulation allow.

Precision: every product and sum is fp64 on the (already rounded) inputs.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .attention import visible_mask

__all__ = ["matmul_matmul", "matmul_matmul_rows", "intermediate", "error_bounds",
           "BF16_UNIT_ROUNDOFF", "F32_UNIT_ROUNDOFF"]

BF16_UNIT_ROUNDOFF = 2.0 ** -8   # 8-bit significand, round to nearest even
F32_UNIT_ROUNDOFF = 2.0 ** -24


def _heads(q, k):
    bsz, lq, hq, dqk = q.shape
    hkv = k[0].shape[1] if bsz else 1
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"query heads ({hq}) must be a multiple of KV heads ({hkv})")
    return bsz, lq, hq, dqk, hkv, hq // hkv


def intermediate(q: np.ndarray, kb: np.ndarray, vis: np.ndarray, scale: float) -> np.ndarray:
    """The first product of one (request, head): T = tau Q K^T, invisible entries 0.

    q [Lq, d], kb [n, d], vis [Lq, n] -> T [Lq, n] (float64, materialised).
    """
    t = scale * np.matmul(np.asarray(q, dtype=np.float64), np.asarray(kb, dtype=np.float64).T)
    return np.where(vis, t, 0.0)


def matmul_matmul(q: np.ndarray, k: Sequence[np.ndarray], v: Sequence[np.ndarray],
                  causal: bool, scale: Optional[float] = None) -> np.ndarray:
    """Exact O = (tau Q K^T) V per (request, query head), the intermediate materialised.

    q [B, Lq, Hq, d]; k[b] [L_b, Hkv, d]; v[b] [L_b, Hkv, dv] (ragged lists).
    Query head h uses KV head h // (Hq / Hkv).  Returns O [B, Lq, Hq, dv] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, lq, hq, dqk, hkv, g = _heads(q, k)
    dv = v[0].shape[2] if bsz else 0
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    o = np.zeros((bsz, lq, hq, dv), dtype=np.float64)
    for b in range(bsz):
        kb_all = np.asarray(k[b], dtype=np.float64)
        vb_all = np.asarray(v[b], dtype=np.float64)
        vis = visible_mask(lq, kb_all.shape[0], causal)
        for h in range(hq):
            t = intermediate(q[b, :, h, :], kb_all[:, h // g, :], vis, scale)   # first MatMul
            o[b, :, h, :] = np.matmul(t, vb_all[:, h // g, :])                 # second MatMul
    return o


def matmul_matmul_rows(q, k, v, causal, scale, rows):
    """Exact outputs for selected rows only: rows = [(b, i, h), ...] -> O [n, dv]."""
    q = np.asarray(q)
    bsz, lq, hq, dqk, hkv, g = _heads(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    out = np.zeros((len(rows), v[0].shape[2]))
    for r, (b, i, h) in enumerate(rows):
        kb = np.asarray(k[b][:, h // g, :], dtype=np.float64)
        vis = visible_mask(lq, kb.shape[0], causal)[i:i + 1]
        t = intermediate(np.asarray(q[b, i:i + 1, h, :], dtype=np.float64), kb, vis, scale)
        out[r] = np.matmul(t, np.asarray(v[b][:, h // g, :], dtype=np.float64))[0]
    return out


def error_bounds(q, k, v, causal, scale=None, rounds_intermediate: bool = True):
    """What a kernel may differ from the exact O by, per output element.

    The kernel forms each intermediate entry in fp32 from exact bf16 products
    (d terms) times tau, rounds it to bf16 (unit roundoff u = 2^-8) and
    accumulates T V in fp32 (unit roundoff e = 2^-24) over the n visible keys.
    First-order rounding-error analysis (each fp32 addition or product rounds
    once) bounds the difference by
        worst = (u + n e (1 + u)^2) (|T| |V|) + (d + 1) e (1 + u)(1 + n e) (A |V|)
    per output (i, c), with A = tau |Q| |K|^T over visible keys (the fp32 sum
    of the first product errs relative to A, not to |T|, when terms cancel).
    Treating the bf16 roundings as independent, each at most u |T_ij| in size,
    the typical error has root-mean-square at most
        rms = (u / sqrt(3) + n e) * sqrt(sum_j T_ij^2 V_jc^2)
    (the n e term covers fp32 accumulation, 2^16 times smaller than u).
    With ``rounds_intermediate=False`` (every tau Q K^T entry exactly
    representable in bf16, e.g. small integers) the bf16 term u drops out.
    Returns (worst, rms), both [B, Lq, Hq, dv].
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, lq, hq, dqk, hkv, g = _heads(q, k)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    u, e = (BF16_UNIT_ROUNDOFF if rounds_intermediate else 0.0), F32_UNIT_ROUNDOFF
    dv = v[0].shape[2]
    worst = np.zeros((bsz, lq, hq, dv))
    rms = np.zeros((bsz, lq, hq, dv))
    for b in range(bsz):
        kb_all = np.asarray(k[b], dtype=np.float64)
        vb_all = np.asarray(v[b], dtype=np.float64)
        n = kb_all.shape[0]
        vis = visible_mask(lq, n, causal)
        for h in range(hq):
            t = intermediate(q[b, :, h, :], kb_all[:, h // g, :], vis, scale)
            a_abs = intermediate(np.abs(q[b, :, h, :]), np.abs(kb_all[:, h // g, :]), vis,
                                 abs(scale))
            vb = vb_all[:, h // g, :]
            va = np.abs(vb)
            worst[b, :, h, :] = ((u + n * e * (1 + u) ** 2) * np.matmul(np.abs(t), va)
                                 + (dqk + 1) * e * (1 + u) * (1 + n * e) * np.matmul(a_abs, va))
            rms[b, :, h, :] = (u / math.sqrt(3.0) + n * e) * np.sqrt(np.matmul(t * t, vb * vb))
    return worst, rms
