"""fp64 CPU oracle for the attention hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library
and imports nothing from it; it reads only numpy arrays.

Source: the Cleave paper ("Cleave: Scaling Tensor Program Optimization via
Decoupled Algebraic Search and Operator Scheduling", paperpeel.com text).

* §2.2 "FlashAttention" and Fig. 2: attention is a QK-Matmul, then softmax,
  then a V-Matmul.  The FlashAttention rewrite (division moved after the
  V-Matmul) gives the same O, so the oracle is the plain definition, written
  with the whole score matrix S and the whole softmax P materialised.
* §2.2 "Split-K" and Fig. 3: a reduction of length K is the sum of s partial
  reductions over contiguous parts.
* §4 and Fig. 5(b): the split kernel emits a per-split row-sum and a per-split
  value-product of shape [s, S_Q, D]; the combine reduces both over s and then
  divides.  ``split_partials`` + ``combine`` follow that, with each partial
  taken relative to its own row max and carried as (O_j, LSE_j); the combine
  is the log-sum-exp form, which is the same quantity (see ``combine``).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* scale tau defaults to 1/sqrt(Dqk); the softmax is the numerically stable one
  (max subtracted), which is mathematically the same function;
* GQA maps query head h to KV head h // G with G = Hq / Hkv (contiguous groups);
* causal masking is bottom-right aligned: query row i of a request with Lq
  queries and L_b keys sees keys j <= i + L_b - Lq;
* a row with no visible key has O = 0 and LSE = -inf;
* MLA: V is the first Dv columns of the single latent K head.

Precision: every product and sum is fp64 on the (already rounded) inputs.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = ["visible_mask", "attention", "split_partials", "combine",
           "attention_split", "attention_rows"]


def visible_mask(lq: int, n_keys: int, causal: bool, lo: int = 0,
                 hi: Optional[int] = None) -> np.ndarray:
    """Boolean [lq, n_keys]: may query row i attend to key j?

    Key j is visible when it lies in [lo, hi) (the whole length by default)
    and, for causal attention, when j <= i + n_keys - lq (bottom-right
    alignment; for lq == n_keys this is the usual lower triangle j <= i).
    """
    if hi is None:
        hi = n_keys
    i = np.arange(lq)[:, None]
    j = np.arange(n_keys)[None, :]
    vis = (j >= lo) & (j < hi) & (i >= 0)                 # [lq, n_keys]
    if causal:
        vis = vis & (j <= i + (n_keys - lq))
    return vis


def _group(qg: np.ndarray, kb: np.ndarray, vb: np.ndarray, vis: np.ndarray,
           scale: float):
    """Attention of G query heads sharing one KV head, one request.

    qg [G, Lq, Dqk], kb [n, Dqk], vb [n, Dv], vis [Lq, n] -> O [G, Lq, Dv], LSE [G, Lq]
    """
    g, lq, _ = qg.shape
    dv = vb.shape[1]
    o = np.zeros((g, lq, dv), dtype=np.float64)
    lse = np.full((g, lq), -np.inf, dtype=np.float64)
    if kb.shape[0] == 0:
        return o, lse
    # S = tau * Q K^T, materialised in full (QK-Matmul).
    s = scale * np.matmul(qg, kb.T)                       # [G, Lq, n]
    s = np.where(vis[None, :, :], s, -np.inf)
    has = vis.any(axis=1)                                 # rows with >= 1 key
    m = np.where(has[None, :], s.max(axis=2), 0.0)        # row max (finite)
    e = np.where(vis[None, :, :], np.exp(s - m[:, :, None]), 0.0)
    l = e.sum(axis=2)                                     # row sum
    safe_l = np.where(has[None, :], l, 1.0)
    p = e / safe_l[:, :, None]                            # softmax P, materialised
    rows_sum = p.sum(axis=2)
    err = np.abs(rows_sum - 1.0)[:, has]
    assert err.size == 0 or float(err.max()) <= 1e-12, "softmax rows must sum to 1"
    o = np.matmul(p, vb)                                  # V-Matmul
    o[:, ~has, :] = 0.0
    lse = np.where(has[None, :], m + np.log(safe_l), -np.inf)
    return o, lse


def _check(q, hq, hkv):
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"query heads ({hq}) must be a multiple of KV heads ({hkv})")


def attention(q: np.ndarray, k: Sequence[np.ndarray], v: Sequence[np.ndarray],
              causal: bool, scale: Optional[float] = None,
              key_range: Optional[Sequence[tuple]] = None):
    """Exact attention, materialising S and P.

    q  [B, Lq, Hq, Dqk]; k[b] [L_b, Hkv, Dqk]; v[b] [L_b, Hkv, Dv]
    (ragged lists; pass ``[K[b, :L_b] for b ...]`` for padded arrays).
    ``key_range[b] = (lo, hi)`` additionally restricts request b to keys in
    [lo, hi) (used by the split mode).
    Returns O [B, Lq, Hq, Dv] and LSE [B, Lq, Hq] (natural log), both float64.
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, lq, hq, dqk = q.shape
    hkv = k[0].shape[1] if bsz else 1
    _check(q, hq, hkv)
    g = hq // hkv
    dv = v[0].shape[2] if bsz else 0
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    o = np.zeros((bsz, lq, hq, dv), dtype=np.float64)
    lse = np.full((bsz, lq, hq), -np.inf, dtype=np.float64)
    for b in range(bsz):
        kb_all = np.asarray(k[b], dtype=np.float64)
        vb_all = np.asarray(v[b], dtype=np.float64)
        n = kb_all.shape[0]
        lo, hi = (0, n) if key_range is None else key_range[b]
        vis = visible_mask(lq, n, causal, lo, hi)
        for kvh in range(hkv):
            heads = slice(kvh * g, (kvh + 1) * g)
            qg = np.transpose(q[b, :, heads, :], (1, 0, 2))   # [G, Lq, D]
            og, lg = _group(qg, kb_all[:, kvh, :], vb_all[:, kvh, :], vis, scale)
            o[b, :, heads, :] = np.transpose(og, (1, 0, 2))
            lse[b, :, heads] = lg.T
    return o, lse


def attention_rows(q, k, v, causal, scale, rows):
    """Exact attention for selected outputs only: rows = [(b, i, h), ...].

    Each selected output is the definition evaluated for one query row of one
    head, keeping the row's position i for the causal mask.
    Returns O [n, Dv] and LSE [n].
    """
    q = np.asarray(q)
    bsz, lq, hq, dqk = q.shape
    hkv = k[0].shape[1]
    _check(q, hq, hkv)
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    dv = v[0].shape[2]
    out_o = np.zeros((len(rows), dv))
    out_l = np.zeros(len(rows))
    for r, (b, i, h) in enumerate(rows):
        kb = np.asarray(k[b][:, h // g, :], dtype=np.float64)
        vb = np.asarray(v[b][:, h // g, :], dtype=np.float64)
        n = kb.shape[0]
        vis = visible_mask(lq, n, causal)[i:i + 1]
        qg = np.asarray(q[b, i, h], dtype=np.float64)[None, None, :]
        og, lg = _group(qg, kb, vb, vis, scale)
        out_o[r] = og[0, 0]
        out_l[r] = lg[0, 0]
    return out_o, out_l


def split_partials(q, k, v, causal, scale, bounds):
    """Split-K partials (Cleave §4, Fig. 5(b)).

    ``bounds[b]`` is a non-decreasing list 0 = c_0 <= ... <= c_s = L_b; every
    request must have the same s.  Split j of request b covers keys
    [c_j, c_{j+1}).  Returns O_parts [s, B, Lq, Hq, Dv] (each partial already
    divided by its own row sum) and LSE_parts [s, B, Lq, Hq] (-inf for an
    empty split or a row that sees no key of the split).
    """
    bsz = q.shape[0]
    s = len(bounds[0]) - 1
    for b in range(bsz):
        c = list(bounds[b])
        if len(c) != s + 1 or c[0] != 0 or c[-1] != k[b].shape[0] or any(
                c[t] > c[t + 1] for t in range(s)):
            raise ValueError(f"bad split bounds for request {b}: {c}")
    parts_o, parts_l = [], []
    for j in range(s):
        rng_j = [(bounds[b][j], bounds[b][j + 1]) for b in range(bsz)]
        o_j, l_j = attention(q, k, v, causal, scale, key_range=rng_j)
        parts_o.append(o_j)
        parts_l.append(l_j)
    return np.stack(parts_o), np.stack(parts_l)


def combine(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Log-sum-exp merge of split partials over axis 0.

    With M = max_j LSE_j over finite entries and w_j = exp(LSE_j - M):
    O = sum_j w_j O_j / sum_j w_j and LSE = M + ln(sum_j w_j).  Since
    O_j = U_j / l_j and exp(LSE_j) = exp(m_j) l_j, w_j O_j is the split's
    value-product U_j rescaled to the common reference M, and sum_j w_j is the
    rescaled sum of the per-split row sums: the Cleave §4 combine (reduce both
    over s, then divide).  Rows whose partials are all -inf give O = 0,
    LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    finite = np.isfinite(lse_parts)
    any_f = finite.any(axis=0)
    m = np.where(any_f, np.max(np.where(finite, lse_parts, -np.inf), axis=0), 0.0)
    w = np.where(finite, np.exp(np.where(finite, lse_parts, 0.0) - m[None]), 0.0)
    den = w.sum(axis=0)
    safe = np.where(any_f, den, 1.0)
    o = (w[..., None] * o_parts).sum(axis=0) / safe[..., None]
    o = np.where(any_f[..., None], o, 0.0)
    lse = np.where(any_f, m + np.log(safe), -np.inf)
    return o, lse


def attention_split(q, k, v, causal, scale, bounds):
    """Split partials followed by the combine: equal to ``attention`` (Split-K identity)."""
    po, pl = split_partials(q, k, v, causal, scale, bounds)
    return combine(po, pl)
