"""Seeded synthetic inputs shared by the fp64 oracle and the HIP path.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so the oracle and the GPU path can both take their
inputs from it without sharing any of the method.

Workloads (named by what they are, with their sizes):

* ``tiny_gqa_decode_f32``   fp32, B=1, 8 query heads over 2 KV heads, D=64,
  one query row, 256 keys, split count 4.
* ``llama3_8b_gqa_decode``  bf16, B=32, 32/8 heads, D=128, one query row,
  4096 keys per request.
* ``gqa_causal_prefill``    bf16, B=4, 4096 queries and keys, 32/8 heads,
  D=128, lower-triangular causal mask.
* ``ragged_decode_qwen3_32b`` bf16, 64 requests, 64/8 heads, D=128, one query
  row, per-request KV length log-uniform in [128, 32768], capacity 32768.
* ``mla_decode``            bf16, B=64, 128 query heads over one latent KV head,
  Dqk=576 (512 latent + 64 rotary), Dv=512 (V is the first 512 columns of K),
  8192 keys.
* ``llama3_8b_matmul_matmul_prefill`` (``mm_workload``) bf16, B=4, 4096 queries
  and keys, 32/8 heads, D=128, no mask: MatMul+MatMul, O = (tau Q K^T) V per
  head, at Llama-3 8B's attention shapes.

Recipe (stated once, used by tests, smoke and bench):

* ``numpy.random.default_rng(seed)`` (PCG64); every tensor is i.i.d. N(0,1)
  drawn with ``standard_normal(dtype=float32)``.
* Draw order: ragged lengths (if any), then Q, then K, then V (MLA: Q, then the
  latent K; V is a view of K).  Ragged K rows are drawn per request in request
  order, then V rows in request order, so the valid rows never depend on the
  capacity.
* bf16 workloads are rounded fp32 -> bf16 with round-to-nearest-even (torch's
  cast), so the values handed to the oracle (as float64) and to the GPU (as
  bf16) are the same numbers.
* Log-uniform lengths: ``L = clip(floor(exp(U[ln lo, ln hi)))), lo, hi)``.
* Padding rows past a request's length are filled with ``pad`` (NaN for
  parity runs, so any read past the valid rows poisons the output; zero for
  timing runs).
* Paged K/V caches (``page_layout``): request b's rows fill ceil(L_b / page
  size) pages in order; the pages of all requests, plus a few spare pages,
  are numbered by one ``default_rng(seed).permutation`` of the pool, so
  neighbouring pages of a request sit at unrelated places in the pool.
  Page-table entries a request does not use hold -7 (never read).
* RMSNorm + MatMul (``make_rms_problem``): draw X [M, K] ~ N(0, 1), then the
  gain g [K] = 1 + 0.1 N(0, 1), then W [N, K] ~ N(0, 1) / sqrt(K) (the usual
  initialisation scale, so Y stays of order one), each fp32 and rounded to
  bf16 like the attention inputs.  Workloads:
  ``llama3_8b_rmsnorm_matmul_decode`` M=32 tokens, K=4096 (hidden size),
  N=14336 (MLP projection width), eps 1e-5;
  ``llama3_8b_rmsnorm_matmul_prefill`` the same with M=4096 tokens (one
  4096-token prompt); ``tiny_rmsnorm_matmul`` M=5, K=256, N=200.
* SwiGLU (``make_swiglu_problem``): draw X [M, K] ~ N(0, 1), then W_gate and
  W_up [N, K] ~ N(0, 1) / sqrt(K), bf16-rounded.  Workloads:
  ``llama3_8b_swiglu_decode`` M=32, K=4096, N=14336 (Llama-3 8B's MLP);
  ``llama3_8b_swiglu_prefill`` the same with M=4096; ``tiny_swiglu`` M=5,
  K=256, N=200.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Problem", "WORKLOADS", "workload", "make_problem", "to_bf16_exact",
           "padded", "log_uniform_lengths", "page_layout", "RmsProblem", "RMS_WORKLOADS",
           "make_rms_problem", "rms_workload", "SwigluProblem", "SWIGLU_WORKLOADS",
           "make_swiglu_problem", "swiglu_workload"]


@dataclasses.dataclass
class Problem:
    """One attention problem as plain host arrays.

    q      float32 [B, Lq, Hq, Dqk]
    k      list of B float32 arrays [L_b, Hkv, Dqk]   (valid rows only)
    v      list of B float32 arrays [L_b, Hkv, Dv], or None when V is the
           first ``dv`` columns of K (MLA)
    lens   int64 [B]
    """
    name: str
    dtype: str            # "f32" or "bf16": the element type the GPU sees
    q: np.ndarray
    k: list
    v: Optional[list]
    lens: np.ndarray
    hq: int
    hkv: int
    dqk: int
    dv: int
    lcap: int             # capacity (row count of the padded K/V buffers)
    causal: bool
    scale: float
    s: Optional[int] = None   # fixed split count, where the workload names one

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def lq(self) -> int:
        return int(self.q.shape[1])

    @property
    def v_aliases_k(self) -> bool:
        return self.v is None

    def v_rows(self, b: int) -> np.ndarray:
        """V rows of request b (a view of K's first dv columns for MLA)."""
        if self.v is None:
            return self.k[b][..., : self.dv]
        return self.v[b]


WORKLOADS = {
    "tiny_gqa_decode_f32": dict(dtype="f32", batch=1, lq=1, hq=8, hkv=2, dqk=64,
                                dv=64, kv_len=256, causal=False, s=4),
    "llama3_8b_gqa_decode": dict(dtype="bf16", batch=32, lq=1, hq=32, hkv=8,
                                 dqk=128, dv=128, kv_len=4096, causal=False),
    "gqa_causal_prefill": dict(dtype="bf16", batch=4, lq=4096, hq=32, hkv=8,
                               dqk=128, dv=128, kv_len=4096, causal=True),
    "ragged_decode_qwen3_32b": dict(dtype="bf16", batch=64, lq=1, hq=64, hkv=8,
                                    dqk=128, dv=128, kv_len=(128, 32768),
                                    lcap=32768, causal=False),
    "mla_decode": dict(dtype="bf16", batch=64, lq=1, hq=128, hkv=1, dqk=576,
                       dv=512, kv_len=8192, causal=False, mla=True),
}


def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); return as float32."""
    import torch  # the cast is the only use of torch here
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def log_uniform_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    u = rng.uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int64)


def make_problem(*, name: str = "custom", dtype: str = "bf16", batch: int, lq: int,
                 hq: int, hkv: int, dqk: int, dv: int, kv_len, seed: int = 0,
                 causal: bool = False, mla: bool = False, lcap: Optional[int] = None,
                 scale: Optional[float] = None, s: Optional[int] = None,
                 qk_ternary: bool = False) -> Problem:
    """Draw one problem.

    ``kv_len`` is an int (every request has that many keys), a (lo, hi) tuple
    (log-uniform per request), or an explicit sequence of per-request lengths.
    ``qk_ternary``: Q and K entries drawn uniformly from {-1, 0, 1} instead
    (same draw order), so every Q K^T entry is a small integer.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.default_rng(seed)
    if isinstance(kv_len, tuple) and len(kv_len) == 2:
        lens = log_uniform_lengths(rng, batch, int(kv_len[0]), int(kv_len[1]))
    elif np.isscalar(kv_len):
        lens = np.full(batch, int(kv_len), dtype=np.int64)
    else:
        lens = np.asarray(kv_len, dtype=np.int64)
        if lens.shape != (batch,):
            raise ValueError("explicit kv_len must have one entry per request")
    if lcap is None:
        lcap = int(lens.max()) if batch else 0
    if batch and int(lens.max()) > lcap:
        raise ValueError("a request length exceeds the capacity")
    rnd = (lambda a: to_bf16_exact(a)) if dtype == "bf16" else (lambda a: a)

    if qk_ternary:
        draw = lambda shape: rng.integers(-1, 2, size=shape).astype(np.float32)  # noqa: E731
    else:
        draw = lambda shape: rnd(rng.standard_normal(shape, dtype=np.float32))  # noqa: E731
    q = draw((batch, lq, hq, dqk))
    k = [draw((int(n), hkv, dqk)) for n in lens]
    if mla:
        if dv > dqk:
            raise ValueError("MLA needs dv <= dqk (V is a slice of K)")
        v = None
    else:
        v = [rnd(rng.standard_normal((int(n), hkv, dv), dtype=np.float32)) for n in lens]
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    return Problem(name=name, dtype=dtype, q=q, k=k, v=v, lens=lens, hq=hq, hkv=hkv,
                   dqk=dqk, dv=dv, lcap=int(lcap), causal=causal, scale=float(scale), s=s)


def workload(name: str, seed: int = 0) -> Problem:
    """The named full-size workload, drawn with the recipe above."""
    w = dict(WORKLOADS[name])
    return make_problem(name=name, seed=seed, dtype=w["dtype"], batch=w["batch"],
                        lq=w["lq"], hq=w["hq"], hkv=w["hkv"], dqk=w["dqk"], dv=w["dv"],
                        kv_len=w["kv_len"], causal=w.get("causal", False),
                        mla=w.get("mla", False), lcap=w.get("lcap"), s=w.get("s"))


MM_WORKLOADS = {
    "llama3_8b_matmul_matmul_prefill": dict(dtype="bf16", batch=4, lq=4096, hq=32, hkv=8,
                                            dqk=128, dv=128, kv_len=4096, causal=False),
}


def mm_workload(name: str, seed: int = 0) -> Problem:
    """The named MatMul+MatMul workload (same Problem layout and recipe as attention)."""
    w = dict(MM_WORKLOADS[name])
    return make_problem(name=name, seed=seed, dtype=w["dtype"], batch=w["batch"], lq=w["lq"],
                        hq=w["hq"], hkv=w["hkv"], dqk=w["dqk"], dv=w["dv"], kv_len=w["kv_len"],
                        causal=w["causal"])


def padded(rows: list, lcap: int, pad: float = float("nan")) -> np.ndarray:
    """Stack ragged per-request rows [L_b, H, D] into [B, lcap, H, D] with padding."""
    b = len(rows)
    h, d = rows[0].shape[1], rows[0].shape[2]
    out = np.full((b, lcap, h, d), pad, dtype=np.float32)
    for i, r in enumerate(rows):
        out[i, : r.shape[0]] = r
    return out


def page_layout(lens, page_size: int, seed: int, lcap: Optional[int] = None,
                spare_pages: int = 3):
    """A shuffled page table for per-request key counts ``lens``.

    Returns (table int32 [B, pages_per_req], num_pages).  pages_per_req covers
    ``lcap`` (default: the longest request).
    """
    rng = np.random.default_rng(seed)
    need = [-(-int(n) // page_size) for n in lens]
    cap = max(lens) if lcap is None and len(lens) else (lcap or 0)
    ppr = max([1, -(-int(cap) // page_size)] + need)
    total = sum(need) + spare_pages
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(lens), ppr), -7, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, total


@dataclasses.dataclass
class RmsProblem:
    """RMSNorm(X) W^T as plain host arrays: x [M, K], g [K], w [N, K]."""
    name: str
    dtype: str
    x: np.ndarray
    g: np.ndarray
    w: np.ndarray
    eps: float
    s: Optional[int] = None

    @property
    def m(self) -> int:
        return int(self.x.shape[0])

    @property
    def k(self) -> int:
        return int(self.x.shape[1])

    @property
    def n(self) -> int:
        return int(self.w.shape[0])


RMS_WORKLOADS = {
    "tiny_rmsnorm_matmul": dict(m=5, k=256, n=200),
    "llama3_8b_rmsnorm_matmul_decode": dict(m=32, k=4096, n=14336),
    "llama3_8b_rmsnorm_matmul_prefill": dict(m=4096, k=4096, n=14336),
}


def make_rms_problem(*, name: str = "custom", dtype: str = "bf16", m: int, k: int, n: int,
                     seed: int = 0, eps: float = 1e-5, s: Optional[int] = None) -> RmsProblem:
    """Draw X, then g, then W (see the recipe above)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.default_rng(seed)
    rnd = (lambda a: to_bf16_exact(a)) if dtype == "bf16" else (lambda a: a)
    x = rnd(rng.standard_normal((m, k), dtype=np.float32))
    g = rnd((1.0 + 0.1 * rng.standard_normal(k, dtype=np.float32)).astype(np.float32))
    w = rnd((rng.standard_normal((n, k), dtype=np.float32) / np.float32(math.sqrt(k))).astype(np.float32))
    return RmsProblem(name=name, dtype=dtype, x=x, g=g, w=w, eps=float(eps), s=s)


def rms_workload(name: str, seed: int = 0) -> RmsProblem:
    w = RMS_WORKLOADS[name]
    return make_rms_problem(name=name, seed=seed, m=w["m"], k=w["k"], n=w["n"])


@dataclasses.dataclass
class SwigluProblem:
    """silu(X W_gate^T) * (X W_up^T) as host arrays: x [M, K], w_gate, w_up [N, K]."""
    name: str
    dtype: str
    x: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    s: Optional[int] = None

    @property
    def m(self) -> int:
        return int(self.x.shape[0])

    @property
    def k(self) -> int:
        return int(self.x.shape[1])

    @property
    def n(self) -> int:
        return int(self.w_gate.shape[0])


SWIGLU_WORKLOADS = {
    "tiny_swiglu": dict(m=5, k=256, n=200),
    "llama3_8b_swiglu_decode": dict(m=32, k=4096, n=14336),
    "llama3_8b_swiglu_prefill": dict(m=4096, k=4096, n=14336),
}


def make_swiglu_problem(*, name: str = "custom", m: int, k: int, n: int, seed: int = 0,
                        s: Optional[int] = None) -> SwigluProblem:
    """Draw X, then W_gate, then W_up (see the recipe above), bf16-rounded."""
    rng = np.random.default_rng(seed)
    sc = np.float32(1.0 / math.sqrt(k))
    x = to_bf16_exact(rng.standard_normal((m, k), dtype=np.float32))
    wg = to_bf16_exact((rng.standard_normal((n, k), dtype=np.float32) * sc).astype(np.float32))
    wu = to_bf16_exact((rng.standard_normal((n, k), dtype=np.float32) * sc).astype(np.float32))
    return SwigluProblem(name=name, dtype="bf16", x=x, w_gate=wg, w_up=wu, s=s)


def swiglu_workload(name: str, seed: int = 0) -> SwigluProblem:
    w = SWIGLU_WORKLOADS[name]
    return make_swiglu_problem(name=name, seed=seed, m=w["m"], k=w["k"], n=w["n"])
