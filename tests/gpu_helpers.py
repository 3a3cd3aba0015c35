"""Helpers for the GPU parity tests: device placement and error reports.

Inputs come from ``synthetic.inputs`` (seeded); expected values come from the
fp64 oracle only.  Nothing here computes attention.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import reduction_attention_gqa_amd as ra  # noqa: E402

DEV = "cuda"


def torch_dtype(code: str):
    return torch.bfloat16 if code == "bf16" else torch.float32


class DeviceProblem:
    """A synthetic Problem placed on the GPU.

    layout "token": K/V buffers [B, Lcap, Hkv, D]; "head": [B, Hkv, Lcap, D]
    exposed as a [B, Lcap, Hkv, D] view.  Padding rows past each length hold
    ``pad``.  For MLA, v is a view of k's first Dv columns.
    """

    def __init__(self, prob, layout="token", pad=float("nan"), o_dtype=None, lcap=None):
        self.prob = prob
        dt = torch_dtype(prob.dtype)
        b, lq, hq, dqk = prob.q.shape
        self.lcap = prob.lcap if lcap is None else lcap
        self.q = torch.from_numpy(prob.q).to(DEV).to(dt)
        self.k = self._kv(prob.k, prob.hkv, dqk, dt, layout, pad)
        if prob.v_aliases_k:
            self.v = self.k[..., : prob.dv]
        else:
            self.v = self._kv(prob.v, prob.hkv, prob.dv, dt, layout, pad)
        self.lens = torch.tensor(prob.lens, dtype=torch.int32, device=DEV)
        od = dt if o_dtype is None else torch_dtype(o_dtype)
        self.o_dtype = od
        self.o = torch.full((b, lq, hq, prob.dv), float("nan"), dtype=od, device=DEV)
        self.lse = torch.full((b, lq, hq), float("nan"), dtype=torch.float32, device=DEV)

    def _kv(self, rows, hkv, d, dt, layout, pad):
        b = len(rows)
        if layout == "token":
            buf = torch.full((b, self.lcap, hkv, d), pad, dtype=dt, device=DEV)
            view = buf
        elif layout == "head":
            buf = torch.full((b, hkv, self.lcap, d), pad, dtype=dt, device=DEV)
            view = buf.permute(0, 2, 1, 3)
        else:
            raise ValueError(layout)
        for i, r in enumerate(rows):
            if r.shape[0]:
                view[i, : r.shape[0]] = torch.from_numpy(np.ascontiguousarray(r)).to(DEV).to(dt)
        return view

    def problem(self):
        p = self.prob
        return ra.make_problem(self.q, self.k, self.v, self.o, kv_lens=self.lens,
                               kv_len_max=self.lcap, causal=p.causal, scale=p.scale)

    def decode(self, s_request=0, plan=None, fused=True, ws=None):
        """fused: attn_decode (one launch where the kernel family allows);
        otherwise attn_decode_split then attn_combine."""
        prob = self.problem()
        if plan is None:
            plan = ra.attn_decode_plan(prob, s_request, list(self.prob.lens))
        ws_o, ws_lse, ws_cnt = ra.workspace(plan, DEV) if ws is None else ws
        if fused:
            ra.attn_decode(prob, plan, self.q, self.k, self.v, ws_o, ws_lse, ws_cnt, self.o,
                           self.lse)
        else:
            ra.attn_decode_split(prob, plan, self.q, self.k, self.v, ws_o, ws_lse)
            ra.attn_combine(prob, plan, ws_o, ws_lse, self.o, self.lse)
        torch.cuda.synchronize()
        return plan

    def prefill(self):
        ra.attn_prefill(self.problem(), self.q, self.k, self.v, self.o, self.lse)
        torch.cuda.synchronize()

    def out(self):
        return self.o.float().cpu().numpy().astype(np.float64)

    def lse_out(self):
        return self.lse.cpu().numpy().astype(np.float64)


def _to_dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt)


def _place_queries(obj, prob, q_lens, dt, od, pad, spare):
    """Q, O and LSE on the device: [B, Lq, ...] when q_lens is None, else packed
    [T + spare, ...] with q_indptr (request b keeps its first q_lens[b] rows)."""
    b, lq, hq, dqk = prob.q.shape
    obj.q_lens = q_lens
    if q_lens is None:
        obj.q_indptr = None
        obj.q = _to_dev(prob.q, dt)
        obj.o = torch.full((b, lq, hq, prob.dv), float("nan"), dtype=od, device=DEV)
        obj.lse = torch.full((b, lq, hq), float("nan"), dtype=torch.float32, device=DEV)
        return
    assert len(q_lens) == b and max(q_lens) <= lq
    obj.q_indptr = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32,
                                device=DEV)
    tq = int(sum(q_lens))
    qh = np.full((tq + spare, hq, dqk), pad, dtype=np.float32)
    if tq:
        qh[:tq] = np.concatenate([prob.q[i, :n] for i, n in enumerate(q_lens)])
    obj.q = _to_dev(qh, dt)
    obj.tq = tq
    obj.o = torch.full((tq + spare, hq, prob.dv), float("nan"), dtype=od, device=DEV)
    obj.lse = torch.full((tq + spare, hq), float("nan"), dtype=torch.float32, device=DEV)


class PagedDeviceProblem(DeviceProblem):
    """A synthetic Problem whose K/V live in a shuffled page pool.

    layout "token": pools [num_pages, ps, Hkv, D]; "head": [num_pages, Hkv, ps, D]
    exposed as a [num_pages, ps, Hkv, D] view.  Pool rows no request owns hold
    ``pad``.  Q, O and LSE are as in DeviceProblem.
    """

    def __init__(self, prob, page_size, layout="token", seed=0, pad=float("nan"),
                 o_dtype=None, q_lens=None, spare=5):
        from synthetic.inputs import page_layout
        self.prob = prob
        dt = torch_dtype(prob.dtype)
        b, lq, hq, dqk = prob.q.shape
        self.lcap = prob.lcap
        self.page_size = page_size
        table, self.num_pages = page_layout(prob.lens, page_size, seed, lcap=prob.lcap)
        self.table_host = table
        self.table = torch.from_numpy(table).to(DEV)
        self.k = self._pool(prob.k, prob.hkv, dqk, dt, layout, pad)
        if prob.v_aliases_k:
            self.v = self.k[..., : prob.dv]
        else:
            self.v = self._pool(prob.v, prob.hkv, prob.dv, dt, layout, pad)
        self.lens = torch.tensor(prob.lens, dtype=torch.int32, device=DEV)
        od = dt if o_dtype is None else torch_dtype(o_dtype)
        self.o_dtype = od
        _place_queries(self, prob, q_lens, dt, od, pad, spare)

    def _pool(self, rows, hkv, d, dt, layout, pad):
        ps = self.page_size
        host = np.full((self.num_pages, ps, hkv, d), pad, dtype=np.float32)
        for b, r in enumerate(rows):
            n = r.shape[0]
            npg = -(-n // ps)
            if npg == 0:
                continue
            blk = np.full((npg * ps, hkv, d), pad, dtype=np.float32)
            blk[:n] = r
            host[self.table_host[b, :npg]] = blk.reshape(npg, ps, hkv, d)
        if layout == "token":
            return _to_dev(host, dt)
        if layout == "head":
            return _to_dev(host.transpose(0, 2, 1, 3), dt).permute(0, 2, 1, 3)
        raise ValueError(layout)

    def problem(self):
        p = self.prob
        return ra.make_problem(self.q, self.k, self.v, self.o, kv_lens=self.lens,
                               kv_len_max=self.lcap, causal=p.causal, scale=p.scale,
                               page_table=self.table, q_indptr=self.q_indptr, q_len_max=p.lq)


class PackedDeviceProblem(DeviceProblem):
    """A synthetic Problem with packed keys (kv_indptr) and, when ``q_lens`` is
    given, packed ragged queries (q_indptr): request b keeps its first
    q_lens[b] query rows.  ``spare`` extra rows after the last request in the
    packed K/V, O and LSE tensors hold ``pad`` / NaN."""

    def __init__(self, prob, q_lens=None, pad=float("nan"), spare=5, o_dtype=None):
        self.prob = prob
        dt = torch_dtype(prob.dtype)
        b, lq, hq, dqk = prob.q.shape
        self.lcap = prob.lcap
        lens = [int(n) for n in prob.lens]
        self.kv_indptr = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32,
                                      device=DEV)
        tk = sum(lens)
        kh = np.full((tk + spare, prob.hkv, dqk), pad, dtype=np.float32)
        if tk:
            kh[:tk] = np.concatenate(prob.k)
        self.k = _to_dev(kh, dt)
        if prob.v_aliases_k:
            self.v = self.k[..., : prob.dv]
        else:
            vh = np.full((tk + spare, prob.hkv, prob.dv), pad, dtype=np.float32)
            if tk:
                vh[:tk] = np.concatenate(prob.v)
            self.v = _to_dev(vh, dt)
        od = dt if o_dtype is None else torch_dtype(o_dtype)
        self.o_dtype = od
        _place_queries(self, prob, q_lens, dt, od, pad, spare)

    def problem(self):
        p = self.prob
        return ra.make_problem(self.q, self.k, self.v, self.o, kv_len_max=self.lcap,
                               causal=p.causal, scale=p.scale, kv_indptr=self.kv_indptr,
                               q_indptr=self.q_indptr, q_len_max=p.lq)


def v_rows(prob):
    return [prob.v_rows(b) for b in range(prob.batch)]


def report(name, got, want):
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    print(f"[parity] {name}: max_abs={mx:.3e} mean_abs={mean:.3e} n={err.size}", flush=True)
    return mx, mean


def assert_close(name, got, want, max_tol, mean_tol):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in GPU output"
    mx, mean = report(name, got, want)
    assert mx <= max_tol, f"{name}: max abs error {mx} > {max_tol}"
    assert mean <= mean_tol, f"{name}: mean abs error {mean} > {mean_tol}"


def assert_lse_close(name, got, want, tol=1e-3):
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), f"{name}: -inf pattern of LSE differs"
    if fin.any():
        mx = float(np.abs(got[fin] - want[fin]).max())
        print(f"[parity] {name} lse: max_abs={mx:.3e}", flush=True)
        assert mx <= tol


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


BF16_MAX, BF16_MEAN = 1e-2, 1e-3
F32_MAX, F32_MEAN = 1e-5, 1e-5
