#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

Default run (N = 1), one JSON line:
  * value: split-K decode throughput in algorithmic HBM GB/s on the
    Llama-3-8B-shaped GQA decode (B=32, 32/8 heads, D=128, 4096 keys, bf16);
    one step = plan + one attn_decode call over the whole batch (for this
    kernel family a single launch: one split per (request, KV head) writes O
    directly; with several splits the last split of each (request, KV head)
    merges the partials).  Ablations beside it: a paged cache (16-row pages
    scattered over a pool by a seeded shuffle), the two-launch form (split
    kernel + combine kernel), the token-major cache and the split-off (s = 1)
    plan.
  * ragged_decode: 64 requests with Qwen3-32B heads (64/8, D=128) and
    log-uniform key counts in [128, 32768], GB/s; with the two-launch,
    token-major and split-off ablations (the planner splits every long
    request here).
  * mla_decode: B=64, 128 heads over one latent head (Dqk=576, Dv=512,
    V = K[..., :512]), 8192 keys, GB/s; one launch whose last split per
    request merges; with the two-launch and split-off ablations.
  * tiny_decode_f32: fp32, B=1, 8/2 heads, D=64, 256 keys, s = 4: latency.
  * prefill: causal GQA prefill (B=4, L=4096, 32/8 heads, D=128, bf16) in
    algorithmic TFLOP/s; one step = one fused prefill launch.
  * matmul_matmul: MatMul+MatMul, O = (tau Q K^T) V per head with no softmax
    (B=4, 4096 queries and keys, 32/8 heads, D=128, bf16) in algorithmic
    TFLOP/s; one step = one launch.
  * rmsnorm_matmul: RMSNorm followed by a MatMul on the Llama-3 8B decode
    shape (32 tokens, K=4096, N=14336, bf16) in algorithmic HBM GB/s (W, X, g
    read once, Y written once); one step = one call.
  * swiglu: SwiGLU on Llama-3 8B's MLP at 32 tokens (K=4096, N=14336, bf16)
    in algorithmic HBM GB/s (both weight matrices and X read once, H written
    once); one step = one call.
  * rmsnorm_matmul_prefill, swiglu_prefill: the same two subgraphs in the
    prefill setting, 4096 tokens, in algorithmic TFLOP/s (2 m k n per
    MatMul); one step = one call (the X * g pre-pass and the tiled GEMM, or
    the one GEMM launch of both SwiGLU MatMuls).
Each leg first runs its step untimed for about 0.25 s (GPU clocks and
address translation settle under the new load), then the warm-up steps, then
exactly the timed steps.  Every record carries ms_per_step (host wall clock
over exactly the timed steps), gpu_span_ms_per_step (the GPU time between two
HIP events recorded on the launch stream around the same timed steps, per
step) and the roofline of its dominant kernel: achieved = algorithmic work
per launch / that span per launch (for the two-launch decode ablation, the
split kernel's own event pairs); a second pass with an event pair around
every launch gives the per-launch statistics in launch_ms.  After every GPU leg has run, the fp64 oracle is timed on the host
cores over a bounded sample of each workload (cpu_baseline), and once on a
single BLAS thread for the Llama decode and the tiny fp32 decode; "host"
records the CPU model, core count and numpy / BLAS versions.
Inputs are synthetic (seeded i.i.d. N(0,1), rounded to bf16) and resident in
HBM before timing.  The decode K/V cache is stored head-major, [B, Hkv, L, D]
(each (request, KV head) one contiguous stream; the library takes any
strides); --kv-layout token makes the token-major cache the measured one,
--paged PS a paged one.  Several copies of the inputs are rotated so that a
step never finds its K/V in the 256 MB Infinity Cache from the previous step.

Algorithmic work: bytes = unique Q, K and V reads + O write (the split
workspace is not counted); flops = 2 (Dqk + Dv) per visible (query, key) pair.

--workload NAME benches one named workload instead (its own JSON line).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode attn HBM GB/s + prefill TFLOP/s (fraction of MI355X peak), 1 GPU"
INFINITY_CACHE_BYTES = 256 << 20


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--s", type=int, default=0, help="force the split count (0 = planner)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--paged", type=int, default=0, metavar="PS",
                    help="decode from a paged K/V cache with PS rows per page (0 = contiguous)")
    ap.add_argument("--kv-layout", choices=("token", "head"), default="head",
                    help="decode K/V cache storage: token-major [B, L, Hkv, D] or head-major "
                         "[B, Hkv, L, D] (the kernels take either through strides)")
    ap.add_argument("--two-launch", action="store_true",
                    help="time decode as split kernel + combine kernel instead of one launch")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for PMC byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-calibration --workload W` into profiles/traffic.json")
    return ap.parse_args()


# ----------------------------------------------------------------------- inputs

def kv_buffer(prob, d, dt, dev, layout):
    """A zero K or V cache seen as [B, Lcap, Hkv, d]: token-major storage
    [B, Lcap, Hkv, d], or head-major storage [B, Hkv, Lcap, d] (a permuted view;
    the library takes the strides)."""
    import torch
    if layout == "head":
        return torch.zeros((prob.batch, prob.hkv, prob.lcap, d), dtype=dt, device=dev).permute(0, 2, 1, 3)
    return torch.zeros((prob.batch, prob.lcap, prob.hkv, d), dtype=dt, device=dev)


def pool_buffer(num_pages, page_size, hkv, d, dt, dev, layout):
    """A zero page pool seen as [num_pages, page_size, Hkv, d]: token-major pages,
    or head-major pages [num_pages, Hkv, page_size, d] (a permuted view)."""
    import torch
    if layout == "head":
        return torch.zeros((num_pages, hkv, page_size, d), dtype=dt, device=dev).permute(0, 2, 1, 3)
    return torch.zeros((num_pages, page_size, hkv, d), dtype=dt, device=dev)


def device_copies(prob, n_copies, dev, layout="token", page_size=0):
    """n_copies independent device copies of one synthetic problem (zero padding).
    page_size > 0: K/V live in a page pool whose pages are shuffled by a seeded
    permutation (synthetic.inputs.page_layout); the page table is returned too."""
    import numpy as np
    import torch
    dt = torch.bfloat16 if prob.dtype == "bf16" else torch.float32
    q = torch.from_numpy(prob.q).to(dev).to(dt)
    table = None
    if page_size:
        from synthetic.inputs import page_layout
        table_h, n_pages = page_layout(prob.lens, page_size, seed=1, lcap=prob.lcap)
        table = torch.from_numpy(table_h).to(dev)
        k = pool_buffer(n_pages, page_size, prob.hkv, prob.dqk, dt, dev, layout)
        v = None if prob.v_aliases_k else pool_buffer(n_pages, page_size, prob.hkv, prob.dv, dt,
                                                      dev, layout)
    else:
        k = kv_buffer(prob, prob.dqk, dt, dev, layout)
        v = None if prob.v_aliases_k else kv_buffer(prob, prob.dv, dt, dev, layout)
    for b in range(prob.batch):
        n = int(prob.lens[b])
        if not n:
            continue
        if page_size:
            t = torch.arange(n, device=dev)
            rows = (torch.from_numpy(table_h[b]).to(dev).long()[t // page_size], t % page_size)
        else:
            rows = (b, slice(0, n))
        k[rows] = torch.from_numpy(np.ascontiguousarray(prob.k[b])).to(dev).to(dt)
        if v is not None:
            v[rows] = torch.from_numpy(np.ascontiguousarray(prob.v[b])).to(dev).to(dt)
    copies = []
    for c in range(n_copies):
        qc, kc = (q, k) if c == 0 else (q.clone(), k.clone())
        vc = kc[..., : prob.dv] if v is None else (v if c == 0 else v.clone())
        copies.append((qc, kc, vc))
    lens = torch.tensor(prob.lens, dtype=torch.int32, device=dev)
    return copies, lens, table


def n_copies_for(step_bytes):
    return max(2, math.ceil((INFINITY_CACHE_BYTES * 4) / max(step_bytes, 1)) + 1)


# ------------------------------------------------------------------- algorithmic

def decode_bytes(prob):
    e = 2 if prob.dtype == "bf16" else 4
    sum_l = int(prob.lens.sum())
    q = prob.batch * prob.lq * prob.hq * prob.dqk * e
    o = prob.batch * prob.lq * prob.hq * prob.dv * e
    kv = sum_l * prob.hkv * (prob.dqk if prob.v_aliases_k else prob.dqk + prob.dv) * e
    return q, kv, o


def visible_pairs(prob):
    total = 0
    for n in prob.lens:
        n = int(n)
        if prob.causal:
            for i in range(prob.lq):
                total += max(0, min(n, i + n - prob.lq + 1))
        else:
            total += prob.lq * n
    return total * prob.hq


def attention_flops(prob):
    return 2 * (prob.dqk + prob.dv) * visible_pairs(prob)


def source_sha(relpath):
    with open(os.path.join(ROOT, relpath), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


COPY_CALIBRATION_BYTES = 256 << 20  # bytes read (and written) by the calibration copy

# Kernel-name substring and source file of the dominant kernel of each workload
# family, for the PMC summary.
KERNEL_OF = {
    "gqa_d128": ("decode_gqa_d128_", "reduction_attention_gqa_amd/csrc/kernels/decode_gqa_d128.hip"),
    "mla": ("decode_mla_kernel", "reduction_attention_gqa_amd/csrc/kernels/decode_mla.hip"),
    "generic": ("generic", "reduction_attention_gqa_amd/csrc/kernels/generic.hip"),
    "prefill": ("prefill_d128_kernel", "reduction_attention_gqa_amd/csrc/kernels/prefill_d128.hip"),
    "rms": ("rmsnorm_matmul_split_kernel",
            "reduction_attention_gqa_amd/csrc/kernels/rmsnorm_matmul.hip"),
    "swiglu": ("swiglu_split_kernel", "reduction_attention_gqa_amd/csrc/kernels/swiglu.hip"),
    "gemm": ("gemm_nt_kernel", "reduction_attention_gqa_amd/csrc/kernels/gemm_nt.hip"),
}
GEMM_SRC = KERNEL_OF["gemm"][1]


def copy_calibration(dev):
    """A plain device copy of COPY_CALIBRATION_BYTES (read) into another buffer
    (written), twice: the reference for rocprofv3's FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _pmc_per_dispatch(csv_path, counter):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 csv."""
    import csv
    out = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            d = int(row["Dispatch_Id"])
            name, v = out.get(d, (row["Kernel_Name"], 0.0))
            out[d] = (name, v + float(row["Counter_Value"]))
    return out


def summarize_pmc(fetch_csv, write_csv, workload_name, family, key):
    """HBM bytes per launch of the dominant kernel, each counter scaled by what it
    reads for the calibration copy (COPY_CALIBRATION_BYTES read and written)."""
    sub, src = KERNEL_OF[family]
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = _pmc_per_dispatch(path, counter)
        # The calibration copies are the first two copy dispatches of the run
        # (bench.py runs them before anything else is copied).
        copies = [per[d][1] for d in sorted(per) if "copy" in per[d][0].lower()][:2]
        kern = [v for n, v in per.values() if sub in n]
        if len(copies) < 2 or not kern:
            raise SystemExit(f"{path}: no calibration copy or no {sub} dispatch found")
        copy_kib = sum(copies) / 2
        factor = COPY_CALIBRATION_BYTES / (copy_kib * 1024.0)
        kib = sorted(kern)[len(kern) // 2]  # median over the launches
        res[counter] = dict(kib_per_dispatch=kib, copy_kib=copy_kib, factor=factor,
                            bytes=kib * 1024.0 * factor, dispatches=len(kern))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[key] = {"workload": workload_name, "kernel": sub, "source": src,
                 "source_sha": source_sha(src),
                 "bytes_per_launch": round(res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]),
                 "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"]}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(data[key], indent=1))


def traffic_for(kernel_src, launches_key):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(launches_key)
    if not ent or ent.get("source_sha") != source_sha(kernel_src):
        return None
    return ent.get("bytes_per_launch")


# ----------------------------------------------------------------------- timing

SETTLE_S = 0.25


def settle(step, seconds=SETTLE_S):
    """Untimed steps for about `seconds` before the warm-up steps: GPU clocks
    and address translation reach their steady state under this step's load
    (the first few dozen launches after a change of load run measurably
    slower)."""
    import torch
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        step(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed_region(step, steps, stream):
    """Exactly `steps` steps, synchronised on both sides: the host wall clock
    over them, and the GPU time between two events recorded on the launch
    stream around them (no event between the steps), per step."""
    import torch
    reg = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reg[0].record(stream)
    for i in range(steps):
        step(i)
    reg[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, reg[0].elapsed_time(reg[1]) / steps


def time_decode(prob, steps, warmup, s_request, dev, fused, layout="token", page_size=0):
    """Time `steps` decode steps.  fused: one attn_decode call per step (for the
    GQA family a single launch that merges its own splits); otherwise the split
    launch and the combine launch, timed separately.  page_size > 0: a paged
    K/V cache."""
    import torch
    import reduction_attention_gqa_amd as ra
    qb, kvb, ob = decode_bytes(prob)
    copies, lens, table = device_copies(prob, n_copies_for(qb + kvb + ob), dev, layout,
                                        page_size)
    dt = copies[0][0].dtype
    o = torch.empty((prob.batch, prob.lq, prob.hq, prob.dv), dtype=dt, device=dev)
    lens_host = [int(x) for x in prob.lens]
    probs = [ra.make_problem(q, k, v, o, kv_lens=lens, kv_len_max=prob.lcap, causal=prob.causal,
                             scale=prob.scale, page_table=table) for q, k, v in copies]
    plan = ra.attn_decode_plan(probs[0], s_request, lens_host)
    ws_o, ws_lse, ws_cnt = ra.workspace(plan, dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        q, k, v = copies[i % len(copies)]
        pr = probs[i % len(copies)]
        pl = ra.attn_decode_plan(pr, s_request, lens_host)
        if ev is not None:
            ev[0].record(stream)
        if fused:
            ra.attn_decode(pr, pl, q, k, v, ws_o, ws_lse, ws_cnt, o, None, stream)
            if ev is not None:
                ev[1].record(stream)
            return
        ra.attn_decode_split(pr, pl, q, k, v, ws_o, ws_lse, stream)
        if ev is not None:
            ev[1].record(stream)
        ra.attn_combine(pr, pl, ws_o, ws_lse, o, None, stream)
        if ev is not None:
            ev[2].record(stream)

    settle(step)
    for i in range(warmup):
        step(i)
    wall, region_ms = timed_region(step, steps, stream)
    # Per-kernel durations of a second pass, an event pair around each launch
    # (the pair adds its own overhead; the two-launch form needs it to tell
    # the kernels apart).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    split_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    comb_ms = None if fused else sorted(e[1].elapsed_time(e[2]) for e in evs)
    del copies, probs
    return dict(plan=plan, wall_s=wall, split_ms=split_ms, combine_ms=comb_ms,
                bytes=(qb, kvb, ob), fused=fused, region_ms=region_ms)


def time_prefill(prob, steps, warmup, dev, mm=False):
    """Time `steps` fused prefill launches (mm: MatMul+MatMul launches instead)."""
    import torch
    import reduction_attention_gqa_amd as ra
    qb, kvb, ob = decode_bytes(prob)
    copies, lens, _ = device_copies(prob, n_copies_for(qb + kvb + ob), dev)
    dt = copies[0][0].dtype
    o = torch.empty((prob.batch, prob.lq, prob.hq, prob.dv), dtype=dt, device=dev)
    probs = [ra.make_problem(q, k, v, o, kv_lens=lens, kv_len_max=prob.lcap, causal=prob.causal,
                             scale=prob.scale) for q, k, v in copies]
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        q, k, v = copies[i % len(copies)]
        if ev is not None:
            ev[0].record(stream)
        if mm:
            ra.attn_matmul_matmul(probs[i % len(copies)], q, k, v, o, stream)
        else:
            ra.attn_prefill(probs[i % len(copies)], q, k, v, o, None, stream)
        if ev is not None:
            ev[1].record(stream)

    settle(step)
    for i in range(warmup):
        step(i)
    wall, region_ms = timed_region(step, steps, stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    k_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    del copies, probs
    return dict(wall_s=wall, kernel_ms=k_ms, bytes=(qb, kvb, ob), region_ms=region_ms)


def rms_bytes(prob):
    """Algorithmic bytes of RMSNorm + MatMul: W, X and g read once, Y written once (bf16)."""
    return (prob.n * prob.k + prob.m * prob.k + prob.k) * 2, prob.m * prob.n * 2


def time_rms(prob, steps, warmup, dev, s_request=0):
    """Time `steps` RMSNorm + MatMul calls (the split launch and, with s > 1, the
    combine launch), rotating copies of W so no step finds it in the Infinity Cache."""
    import torch
    import reduction_attention_gqa_amd as ra
    rd, wr = rms_bytes(prob)
    n_copies = n_copies_for(rd + wr)
    bf = torch.bfloat16
    x = torch.from_numpy(prob.x).to(dev).to(bf)
    g = torch.from_numpy(prob.g).to(dev).to(bf)
    w0 = torch.from_numpy(prob.w).to(dev).to(bf)
    ws_copies = [w0] + [w0.clone() for _ in range(n_copies - 1)]
    y = torch.empty((prob.m, prob.n), dtype=bf, device=dev)
    prob_c = ra.make_rms_problem(x, g, w0, y, eps=prob.eps)
    plan = ra.rmsnorm_matmul_plan(prob_c, s_request)
    ws = ra.rms_workspace(plan, dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        w = ws_copies[i % n_copies]
        if ev is not None:
            ev[0].record(stream)
        ra.rmsnorm_matmul(prob_c, ra.rmsnorm_matmul_plan(prob_c, s_request), x, g, w, y, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    settle(step)
    for i in range(warmup):
        step(i)
    wall, region_ms = timed_region(step, steps, stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    del ws_copies
    return dict(plan=plan, wall_s=wall, call_ms=call_ms, bytes=(rd, wr), region_ms=region_ms)


def gemm_roofline(flops, r, traffic_key, kernel):
    """MFMA roofline of a prefill-setting call: algorithmic flops / the call's
    average GPU time over the timed region."""
    achieved = flops / (r["region_ms"] * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_for(GEMM_SRC, traffic_key), "kernel": kernel,
            "algorithmic_flops_per_launch": flops,
            "region_ms_per_launch": round(r["region_ms"], 6),
            "launch_ms": stats(r["call_ms"])}


def rms_record(prob, r, steps):
    rd, wr = r["bytes"]
    total = rd + wr
    ms_step = r["wall_s"] * 1e3 / steps
    call = stats(r["call_ms"])
    achieved = total / (r["region_ms"] * 1e-3) / 1e9
    plan = r["plan"]
    config = {"workload": prob.name, "m": prob.m, "k": prob.k, "n": prob.n, "eps": prob.eps,
              "split_s": plan.s, "k_chunk": plan.k_chunk, "kernel": plan.kernel}
    if plan.kernel == 1:
        # Prefill setting: compute-bound; 2 m k n flops of the MatMul (the
        # hi/lo halves of X * g are one exact operand, not extra work).
        flops = 2.0 * prob.m * prob.k * prob.n
        return {"value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms_step, 5), "gpu_span_ms_per_step": round(r["region_ms"], 5),
        "config": config,
                "roofline": gemm_roofline(flops, r, f"rms:{prob.name}",
                                          "X*g pre-pass + tiled MFMA GEMM (timed together)")}
    return {
        "value": round(total / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(ms_step, 5), "gpu_span_ms_per_step": round(r["region_ms"], 5),
        "config": config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("reduction_attention_gqa_amd/csrc/kernels/"
                                            "rmsnorm_matmul.hip", f"rms:{prob.name}"),
                     "kernel": ("RMSNorm+MatMul kernel, one launch" if plan.s == 1 else
                                "RMSNorm+MatMul split kernel + combine kernel (timed together)"),
                     "algorithmic_bytes_per_launch": total,
                     "region_ms_per_launch": round(r["region_ms"], 6), "launch_ms": call}}


def oracle_rows(prob, rows_cap):
    """The first rows of a workload (all of them if there are at most rows_cap):
    the oracle's rows are independent, so a row sample is a bounded sample of
    the same work."""
    return min(prob.m, rows_cap)


def oracle_rms_baseline(prob, rows_cap=512):
    """The fp64 oracle on the RMSNorm + MatMul workload (at most rows_cap token
    rows of it), in the unit of the GPU leg."""
    from threadpoolctl import threadpool_limits
    from oracle import rmsnorm_matmul
    cores = cpu_cores()
    rows = oracle_rows(prob, rows_cap)
    x = prob.x[:rows]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        reps = 0
        while True:
            rmsnorm_matmul(x, prob.g, prob.w, prob.eps)
            reps += 1
            el = time.perf_counter() - t0
            if el > 10.0 or reps >= 200:
                break
    sample = (f"the whole workload, {reps} call(s) in {el:.1f} s, numpy fp64" if rows == prob.m
              else f"{rows} of {prob.m} token rows, {reps} call(s) in {el:.1f} s, numpy fp64")
    if prob.m >= 256:
        value, unit = round(2.0 * rows * prob.k * prob.n * reps / el / 1e12, 6), "TFLOP/s"
    else:
        rd, wr = rms_bytes(prob)
        value, unit = round((rd + wr) * reps / el / 1e9, 4), "GB/s"
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample}


def swiglu_bytes(prob):
    """Algorithmic bytes of SwiGLU: both weight matrices and X read once, H written once."""
    return (2 * prob.n * prob.k + prob.m * prob.k) * 2, prob.m * prob.n * 2


def time_swiglu(prob, steps, warmup, dev, s_request=0):
    """Time `steps` SwiGLU calls, rotating copies of the weights past the
    Infinity Cache."""
    import torch
    import reduction_attention_gqa_amd as ra
    rd, wr = swiglu_bytes(prob)
    n_copies = n_copies_for(rd + wr)
    bf = torch.bfloat16
    x = torch.from_numpy(prob.x).to(dev).to(bf)
    g0 = torch.from_numpy(prob.w_gate).to(dev).to(bf)
    u0 = torch.from_numpy(prob.w_up).to(dev).to(bf)
    weights = [(g0, u0)] + [(g0.clone(), u0.clone()) for _ in range(n_copies - 1)]
    y = torch.empty((prob.m, prob.n), dtype=bf, device=dev)
    pr = ra.make_swiglu_problem(x, g0, u0, y)
    cfg = ra.swiglu_plan(pr, s_request)
    ws = ra.swiglu_workspace(cfg, dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        wg, wu = weights[i % n_copies]
        if ev is not None:
            ev[0].record(stream)
        ra.swiglu(pr, ra.swiglu_plan(pr, s_request), x, wg, wu, y, ws, stream)
        if ev is not None:
            ev[1].record(stream)

    settle(step)
    for i in range(warmup):
        step(i)
    wall, region_ms = timed_region(step, steps, stream)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    call_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    del weights
    return dict(plan=cfg, wall_s=wall, call_ms=call_ms, bytes=(rd, wr), region_ms=region_ms)


def swiglu_record(prob, r, steps):
    rd, wr = r["bytes"]
    total = rd + wr
    ms_step = r["wall_s"] * 1e3 / steps
    call = stats(r["call_ms"])
    achieved = total / (r["region_ms"] * 1e-3) / 1e9
    cfg = r["plan"]
    config = {"workload": prob.name, "m": prob.m, "k": prob.k, "n": prob.n,
              "split_s": cfg.s, "k_chunk": cfg.k_chunk, "kernel": cfg.kernel}
    if cfg.kernel == 1:
        flops = 4.0 * prob.m * prob.k * prob.n   # both MatMuls
        return {"value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms_step, 5), "gpu_span_ms_per_step": round(r["region_ms"], 5),
        "config": config,
                "roofline": gemm_roofline(flops, r, f"swiglu:{prob.name}",
                                          "tiled MFMA GEMM of both MatMuls, one launch")}
    return {
        "value": round(total / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(ms_step, 5), "gpu_span_ms_per_step": round(r["region_ms"], 5),
        "config": config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("reduction_attention_gqa_amd/csrc/kernels/swiglu.hip",
                                            f"swiglu:{prob.name}"),
                     "kernel": ("SwiGLU kernel, one launch" if cfg.s == 1 else
                                "SwiGLU split kernel + combine kernel (timed together)"),
                     "algorithmic_bytes_per_launch": total,
                     "region_ms_per_launch": round(r["region_ms"], 6), "launch_ms": call}}


def oracle_swiglu_baseline(prob, rows_cap=512):
    """The fp64 oracle on the SwiGLU workload (at most rows_cap token rows of
    it), in the unit of the GPU leg."""
    from threadpoolctl import threadpool_limits
    from oracle import swiglu
    cores = cpu_cores()
    rows = oracle_rows(prob, rows_cap)
    x = prob.x[:rows]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        reps = 0
        while True:
            swiglu(x, prob.w_gate, prob.w_up)
            reps += 1
            el = time.perf_counter() - t0
            if el > 10.0 or reps >= 200:
                break
    sample = (f"the whole workload, {reps} call(s) in {el:.1f} s, numpy fp64" if rows == prob.m
              else f"{rows} of {prob.m} token rows, {reps} call(s) in {el:.1f} s, numpy fp64")
    if prob.m >= 256:
        value, unit = round(4.0 * rows * prob.k * prob.n * reps / el / 1e12, 6), "TFLOP/s"
    else:
        rd, wr = swiglu_bytes(prob)
        value, unit = round((rd + wr) * reps / el / 1e9, 4), "GB/s"
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample}


def stats(ms):
    n = len(ms)
    return dict(mean_ms=sum(ms) / n, median_ms=ms[n // 2], min_ms=ms[0], p10_ms=ms[n // 10],
                p90_ms=ms[min(n - 1, (9 * n) // 10)])


# ------------------------------------------------------------------ CPU oracle

def cpu_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def oracle_decode_baseline(prob, budget_s=10.0):
    """The fp64 oracle, as it stands, over the whole decode batch, repeated for ~budget_s."""
    from threadpoolctl import threadpool_limits
    from oracle import attention
    cores = cpu_cores()
    qb, kvb, ob = decode_bytes(prob)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        reps = 0
        while True:
            attention(prob.q, prob.k, [prob.v_rows(b) for b in range(prob.batch)], prob.causal,
                      prob.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 200000:
                break
    gbs = (qb + kvb + ob) * reps / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"whole batch ({prob.batch} requests) x {reps} repetitions, {el:.1f} s, "
                      f"numpy fp64 with {cores} BLAS threads"}


def oracle_prefill_baseline(prob, groups=24):
    """The fp64 oracle on `groups` (request, KV-head) groups of the prefill workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention
    cores = cpu_cores()
    g = prob.hq // prob.hkv
    done = 0
    flops = 0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for idx in range(groups):
            b, kvh = idx % prob.batch, (idx // prob.batch) % prob.hkv
            heads = slice(kvh * g, (kvh + 1) * g)
            q = np.ascontiguousarray(prob.q[b:b + 1, :, heads, :])
            k = [prob.k[b][:, kvh:kvh + 1, :]]
            v = [prob.v_rows(b)[:, kvh:kvh + 1, :]]
            attention(q, k, v, prob.causal, prob.scale)
            done += 1
        el = time.perf_counter() - t0
    n = int(prob.lens[0])
    pairs = (n * (n + 1) // 2 if prob.causal else n * n) * g * done
    flops = 2 * (prob.dqk + prob.dv) * pairs
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} of {prob.batch * prob.hkv} (request, KV head) groups "
                      f"({g} heads x {prob.lq} queries each), {el:.1f} s, numpy fp64"}


def oracle_mm_baseline(prob, heads=128):
    """The fp64 MatMul+MatMul oracle on `heads` (request, query head) pairs."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import matmul_matmul
    cores = cpu_cores()
    g = prob.hq // prob.hkv
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for idx in range(heads):
            b, h = idx % prob.batch, (idx // prob.batch) % prob.hq
            q = np.ascontiguousarray(prob.q[b:b + 1, :, h:h + 1, :])
            k = [prob.k[b][:, h // g:h // g + 1, :]]
            v = [prob.v_rows(b)[:, h // g:h // g + 1, :]]
            matmul_matmul(q, k, v, prob.causal, prob.scale)
        el = time.perf_counter() - t0
    n = int(prob.lens[0])
    pairs = (n * (n + 1) // 2 if prob.causal else n * n) * heads
    flops = 2 * (prob.dqk + prob.dv) * pairs
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{heads} of {prob.batch * prob.hq} (request, query head) pairs "
                      f"({prob.lq} queries x {n} keys each), {el:.1f} s, numpy fp64"}


def mm_record(prob, r, steps):
    """JSON record of a MatMul+MatMul timing (same kernel source as prefill)."""
    flops = attention_flops(prob)
    ks = stats(r["kernel_ms"])
    ms_step = r["wall_s"] * 1e3 / steps
    achieved = flops / (r["region_ms"] * 1e-3) / 1e12
    return {"value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "ms_per_step": round(ms_step, 5),
            "gpu_span_ms_per_step": round(r["region_ms"], 5),
            "config": {"workload": prob.name, "batch": prob.batch, "q_len": prob.lq,
                       "kv_len": int(prob.lens.max()), "q_heads": prob.hq,
                       "kv_heads": prob.hkv, "head_dim": prob.dqk, "causal": bool(prob.causal)},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_for("reduction_attention_gqa_amd/csrc/kernels/"
                                                "prefill_d128.hip", f"mm:{prob.name}"),
                         "kernel": "MatMul+MatMul kernel (prefill kernel without the softmax)",
                         "algorithmic_flops_per_launch": flops,
                         "region_ms_per_launch": round(r["region_ms"], 6), "launch_ms": ks}}


# ------------------------------------------------------------------------ main

def decode_record(prob, r, steps, extra_src, key_suffix=""):
    qb, kvb, ob = r["bytes"]
    total = qb + kvb + ob
    ms_step = r["wall_s"] * 1e3 / steps
    split = stats(r["split_ms"])
    # The dominant kernel: the single fused launch (Q, K, V read + O written),
    # timed over the timed region, or the split launch of the two-launch path
    # (Q, K, V read), timed by its own event pairs.
    kern_bytes = total if r["fused"] else qb + kvb
    launch_ms = r["region_ms"] if r["fused"] else split["mean_ms"]
    achieved = kern_bytes / (launch_ms * 1e-3) / 1e9
    plan = r["plan"]
    traffic = traffic_for(extra_src, ("decode:" if r["fused"] else "decode_split:") + prob.name
                          + key_suffix)
    return dict(
        value=round(total / (ms_step * 1e-3) / 1e9, 2), ms_per_step=round(ms_step, 5),
        gpu_span_ms_per_step=round(r["region_ms"], 5),
        plan=dict(kernel=plan.kernel, s_max=plan.s_max, chunk=plan.chunk, n_items=plan.n_items,
                  grid=list(plan.grid), ws_bytes=int(plan.ws_o_bytes + plan.ws_lse_bytes)),
        roofline={"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                  "traffic": traffic,
                  "kernel": (("decode kernel, single launch, one split per (request, KV head)"
                              if plan.s_max == 1 else
                              "decode kernel, single launch with in-kernel merge")
                             if r["fused"] else "decode split kernel"),
                  "algorithmic_bytes_per_launch": kern_bytes,
                  "region_ms_per_launch": round(launch_ms, 6),
                  "launch_ms": split},
        combine=None if r["combine_ms"] is None else stats(r["combine_ms"]),
        algorithmic_bytes_per_step=total)


KERNEL_SRC = {0: "generic.hip", 1: "decode_gqa_d128.hip", 2: "decode_mla.hip"}


def single_launch_family(prob):
    """Does attn_decode run this workload as one launch (the merge inside the
    split kernel)?  Every kernel family does (an MLA problem too large for its
    single launch aside, which the workloads here are not)."""
    return True


def decode_leg(prob, a, dev, ablations=(), layout="head", page_size=0, s_request=0):
    """Time one decode workload; `ablations` names the extra timings to add
    ("paged", "two_launch", "token_major", "split_off")."""
    fused = single_launch_family(prob) and not a.two_launch
    log(f"timing decode {prob.name} ({'single launch' if fused else 'split + combine'})")
    r = time_decode(prob, a.steps, a.warmup, s_request, dev, fused, layout, page_size)
    src = "reduction_attention_gqa_amd/csrc/kernels/" + KERNEL_SRC[r["plan"].kernel]
    rec = decode_record(prob, r, a.steps, src, f":paged{page_size}" if page_size else "")
    import reduction_attention_gqa_amd as ra
    out = {"value": rec["value"], "unit": "GB/s", "ms_per_step": rec["ms_per_step"],
           "gpu_span_ms_per_step": rec["gpu_span_ms_per_step"],
           "dtype": "bf16" if prob.dtype == "bf16" else "f32",
           "config": {"workload": prob.name, "batch": prob.batch, "q_heads": prob.hq,
                      "kv_heads": prob.hkv, "head_dim_qk": prob.dqk, "head_dim_v": prob.dv,
                      "kv_len_total": int(prob.lens.sum()), "kv_len_max": int(prob.lens.max()),
                      "q_len": prob.lq, "kv_layout": layout, "page_size": page_size or None,
                      "split_s": rec["plan"]["s_max"], "chunk": rec["plan"]["chunk"],
                      "kernel": ra.KERNEL_NAMES[rec["plan"]["kernel"]]},
           "roofline": rec["roofline"],
           "decode_detail": {"plan": rec["plan"], "single_launch": fused,
                             "combine_launch_ms": rec["combine"],
                             "algorithmic_bytes_per_step": rec["algorithmic_bytes_per_step"],
                             "wall_s_timed": round(r["wall_s"], 4)}}
    n_abl = max(10, a.steps // 2)
    if "paged" in ablations:
        log(f"  {prob.name}: paged-cache ablation (16-row pages, shuffled pool)")
        rp = time_decode(prob, n_abl, 3, 0, dev, fused, layout, 16)
        recp = decode_record(prob, rp, n_abl, src)
        out["paged"] = {"page_size": 16, "value": recp["value"], "unit": "GB/s",
                        "ms_per_step": recp["ms_per_step"],
                        "launch_ms": recp["roofline"]["launch_ms"]["mean_ms"],
                        "frac": recp["roofline"]["frac"], "split_s": recp["plan"]["s_max"],
                        "ratio_to_contiguous": round(recp["value"] / rec["value"], 3)}
    if "two_launch" in ablations and fused:
        log(f"  {prob.name}: two-launch ablation (split kernel + combine kernel)")
        r2 = time_decode(prob, n_abl, 3, s_request, dev, False, layout)
        rec2 = decode_record(prob, r2, n_abl, src)
        out["two_launch"] = {"value": rec2["value"], "unit": "GB/s",
                             "ms_per_step": rec2["ms_per_step"],
                             "split_launch_ms": rec2["roofline"]["launch_ms"]["mean_ms"],
                             "combine_launch_ms": rec2["combine"]["mean_ms"],
                             "speedup_of_single_launch": round(rec["value"] / rec2["value"], 3)}
    if "token_major" in ablations and layout == "head":
        log(f"  {prob.name}: token-major cache ablation")
        r3 = time_decode(prob, n_abl, 3, s_request, dev, fused, "token")
        rec3 = decode_record(prob, r3, n_abl, src)
        out["token_major"] = {"value": rec3["value"], "unit": "GB/s",
                              "ms_per_step": rec3["ms_per_step"],
                              "launch_ms": rec3["roofline"]["launch_ms"]["mean_ms"],
                              "frac": rec3["roofline"]["frac"],
                              "speedup_of_head_major": round(rec["value"] / rec3["value"], 3)}
    if "split_off" in ablations:
        log(f"  {prob.name}: split-off ablation (s = 1)")
        r1 = time_decode(prob, n_abl, 3, 1, dev, fused, layout)
        rec1 = decode_record(prob, r1, n_abl, src)
        out["split_off"] = {"value": rec1["value"], "unit": "GB/s",
                            "ms_per_step": rec1["ms_per_step"],
                            "split_s_planned": rec["plan"]["s_max"],
                            "speedup_of_split": round(rec["value"] / rec1["value"], 3)}
    return out


def prefill_leg(prob, a, dev):
    log(f"timing prefill {prob.name}")
    r = time_prefill(prob, a.steps, a.warmup, dev)
    flops = attention_flops(prob)
    ks = stats(r["kernel_ms"])
    ms_step = r["wall_s"] * 1e3 / a.steps
    achieved = flops / (r["region_ms"] * 1e-3) / 1e12
    return {"value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "ms_per_step": round(ms_step, 5),
            "gpu_span_ms_per_step": round(r["region_ms"], 5),
            "config": {"workload": prob.name, "batch": prob.batch, "q_len": prob.lq,
                       "kv_len": int(prob.lens.max()), "q_heads": prob.hq,
                       "kv_heads": prob.hkv, "head_dim": prob.dqk, "causal": bool(prob.causal)},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 3),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_for("reduction_attention_gqa_amd/csrc/kernels/"
                                                "prefill_d128.hip", f"prefill:{prob.name}"),
                         "kernel": "prefill kernel",
                         "algorithmic_flops_per_launch": flops,
                         "region_ms_per_launch": round(r["region_ms"], 6), "launch_ms": ks}}


# --------------------------------------------------------------- host record

def host_info():
    """CPU model, usable cores, numpy and BLAS versions of the host that runs
    the oracle baselines."""
    import numpy as np
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for e in threadpool_info():
            if e.get("user_api") == "blas":
                blas.append({"library": e.get("internal_api"), "version": e.get("version"),
                             "threading": e.get("threading_layer"),
                             "max_threads": e.get("num_threads")})
    except Exception:  # noqa: BLE001 - metadata only
        pass
    return {"cpu_model": model, "cores": cpu_cores(), "logical_cpus": os.cpu_count(),
            "numpy": np.__version__, "blas": blas}


def oracle_decode_single_thread(prob, budget_s=5.0):
    """The fp64 oracle on one BLAS thread over the whole decode batch: a
    per-core figure."""
    from threadpoolctl import threadpool_limits
    from oracle import attention
    qb, kvb, ob = decode_bytes(prob)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        while True:
            attention(prob.q, prob.k, [prob.v_rows(b) for b in range(prob.batch)], prob.causal,
                      prob.scale)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 200000:
                break
    return {"value": round((qb + kvb + ob) * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"whole batch ({prob.batch} requests) x {reps} repetitions, {el:.2f} s, "
                      f"numpy fp64 on one BLAS thread"}


def base_line(a, data):
    return {"metric": METRIC, "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": data}


DATA_ATTN = "synthetic (seeded i.i.d. N(0,1), bf16-rounded; no model weights needed)"


def main():
    a = parse()
    if a.summarize_pmc:
        from synthetic.inputs import RMS_WORKLOADS as RMS_WORKLOADS_NAMES, workload as _wl
        from synthetic.inputs import SWIGLU_WORKLOADS as SW_NAMES, MM_WORKLOADS as MM_NAMES
        name = a.workload or "llama3_8b_gqa_decode"
        prob = None if (name in RMS_WORKLOADS_NAMES or name in SW_NAMES or
                        name in MM_NAMES) else _wl(name)
        if name in MM_NAMES:
            family, key = "prefill", f"mm:{name}"
        elif name in SW_NAMES:
            family = "gemm" if SW_NAMES[name]["m"] >= 256 else "swiglu"
            key = f"swiglu:{name}"
        elif name in RMS_WORKLOADS_NAMES:
            family = "gemm" if RMS_WORKLOADS_NAMES[name]["m"] >= 256 else "rms"
            key = f"rms:{name}"
        elif prob.lq > 1:
            family, key = "prefill", f"prefill:{name}"
        else:
            family = {128: "gqa_d128", 576: "mla"}.get(prob.dqk, "generic")
            if prob.dtype != "bf16":
                family = "generic"
            fused = single_launch_family(prob) and not a.two_launch
            key = ("decode:" if fused else "decode_split:") + name
            if a.paged:
                key += f":paged{a.paged}"
        summarize_pmc(a.summarize_pmc[0], a.summarize_pmc[1], name, family, key)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import reduction_attention_gqa_amd as ra
    ra.load()
    from synthetic.inputs import (MM_WORKLOADS, RMS_WORKLOADS, SWIGLU_WORKLOADS, WORKLOADS,
                                  mm_workload, rms_workload, swiglu_workload, workload)
    dev = "cuda:0"
    if a.copy_calibration:
        log("calibration copy")
        copy_calibration(dev)
    cpu_jobs = []   # (record, key, function, args): oracle runs, after every GPU leg

    name = a.workload
    if name is not None:
        # One named workload, its own JSON line.
        if name in MM_WORKLOADS:
            prob = mm_workload(name)
            out = base_line(a, DATA_ATTN)
            out.update(mm_record(prob, time_prefill(prob, a.steps, a.warmup, dev, mm=True),
                                 a.steps))
            cpu_jobs.append((out, "cpu_baseline", oracle_mm_baseline, (prob,)))
        elif name in SWIGLU_WORKLOADS:
            prob = swiglu_workload(name)
            out = base_line(a, "synthetic (seeded; X ~ N(0,1), W_gate, W_up ~ N(0,1)/sqrt(K), "
                               "bf16-rounded; no model weights needed)")
            log(f"timing {name}")
            out.update(swiglu_record(prob, time_swiglu(prob, a.steps, a.warmup, dev, a.s),
                                     a.steps))
            cpu_jobs.append((out, "cpu_baseline", oracle_swiglu_baseline, (prob,)))
        elif name in RMS_WORKLOADS:
            prob = rms_workload(name)
            out = base_line(a, "synthetic (seeded; X ~ N(0,1), g ~ 1 + 0.1 N(0,1), "
                               "W ~ N(0,1)/sqrt(K), bf16-rounded; no model weights needed)")
            log(f"timing {name}")
            out.update(rms_record(prob, time_rms(prob, a.steps, a.warmup, dev, a.s), a.steps))
            cpu_jobs.append((out, "cpu_baseline", oracle_rms_baseline, (prob,)))
        elif name in WORKLOADS:
            log(f"generating {name}")
            prob = workload(name)
            out = base_line(a, DATA_ATTN)
            if prob.lq > 1:
                out.update(prefill_leg(prob, a, dev))
                cpu_jobs.append((out, "cpu_baseline", oracle_prefill_baseline, (prob,)))
            else:
                abl = () if a.no_ablation or a.s or a.paged else (
                    "two_launch", "split_off")
                leg = decode_leg(prob, a, dev, abl, a.kv_layout, a.paged, a.s)
                out.update(leg)
                cpu_jobs.append((out, "cpu_baseline", oracle_decode_baseline, (prob,)))
        else:
            sys.exit(f"unknown workload {name}; choose from "
                     f"{sorted(WORKLOADS) + sorted(RMS_WORKLOADS) + sorted(SWIGLU_WORKLOADS)}"
                     f" + {sorted(MM_WORKLOADS)}")
    else:
        # The default run: every workload of the hot path, GPU legs first, then
        # the oracle on the host.
        log("generating llama3_8b_gqa_decode")
        prob2 = workload("llama3_8b_gqa_decode")
        out = base_line(a, DATA_ATTN)
        abl = () if a.no_ablation else ("paged", "two_launch", "token_major", "split_off")
        out.update(decode_leg(prob2, a, dev, abl, a.kv_layout, a.paged, a.s))
        cpu_jobs.append((out, "cpu_baseline", oracle_decode_baseline, (prob2,)))

        log("generating ragged_decode_qwen3_32b")
        prob4 = workload("ragged_decode_qwen3_32b")
        abl = () if a.no_ablation else ("two_launch", "token_major", "split_off")
        out["ragged_decode"] = decode_leg(prob4, a, dev, abl, a.kv_layout)
        cpu_jobs.append((out["ragged_decode"], "cpu_baseline", oracle_decode_baseline, (prob4,)))
        del prob4

        log("generating mla_decode")
        prob5 = workload("mla_decode")
        abl = () if a.no_ablation else ("two_launch", "split_off")
        out["mla_decode"] = decode_leg(prob5, a, dev, abl, "token")
        cpu_jobs.append((out["mla_decode"], "cpu_baseline", oracle_decode_baseline, (prob5,)))

        prob1 = workload("tiny_gqa_decode_f32")
        out["tiny_decode_f32"] = decode_leg(prob1, a, dev, (), "token", 0, prob1.s)
        out["tiny_decode_f32"]["latency_us"] = round(
            out["tiny_decode_f32"]["ms_per_step"] * 1e3, 2)
        cpu_jobs.append((out["tiny_decode_f32"], "cpu_baseline", oracle_decode_baseline,
                         (prob1,)))

        if not a.no_prefill:
            pprob = workload("gqa_causal_prefill")
            out["prefill"] = prefill_leg(pprob, a, dev)
            cpu_jobs.append((out["prefill"], "cpu_baseline", oracle_prefill_baseline, (pprob,)))
            mname = "llama3_8b_matmul_matmul_prefill"
            log(f"timing {mname}")
            mprob = mm_workload(mname)
            out["matmul_matmul"] = mm_record(mprob, time_prefill(mprob, a.steps, a.warmup, dev,
                                                                 mm=True), a.steps)
            cpu_jobs.append((out["matmul_matmul"], "cpu_baseline", oracle_mm_baseline, (mprob,)))
        rname = "llama3_8b_rmsnorm_matmul_decode"
        log(f"timing {rname}")
        rprob = rms_workload(rname)
        out["rmsnorm_matmul"] = rms_record(rprob, time_rms(rprob, a.steps, a.warmup, dev), a.steps)
        cpu_jobs.append((out["rmsnorm_matmul"], "cpu_baseline", oracle_rms_baseline, (rprob,)))
        sname = "llama3_8b_swiglu_decode"
        log(f"timing {sname}")
        sprob = swiglu_workload(sname)
        out["swiglu"] = swiglu_record(sprob, time_swiglu(sprob, a.steps, a.warmup, dev), a.steps)
        cpu_jobs.append((out["swiglu"], "cpu_baseline", oracle_swiglu_baseline, (sprob,)))
        if not a.no_prefill:
            for rname in ("llama3_8b_rmsnorm_matmul_prefill",):
                log(f"timing {rname}")
                rprob = rms_workload(rname)
                out["rmsnorm_matmul_prefill"] = rms_record(
                    rprob, time_rms(rprob, a.steps, a.warmup, dev), a.steps)
                cpu_jobs.append((out["rmsnorm_matmul_prefill"], "cpu_baseline",
                                 oracle_rms_baseline, (rprob,)))
            for sname in ("llama3_8b_swiglu_prefill",):
                log(f"timing {sname}")
                sprob = swiglu_workload(sname)
                out["swiglu_prefill"] = swiglu_record(
                    sprob, time_swiglu(sprob, a.steps, a.warmup, dev), a.steps)
                cpu_jobs.append((out["swiglu_prefill"], "cpu_baseline", oracle_swiglu_baseline,
                                 (sprob,)))
        if not a.no_cpu:
            cpu_jobs.append((out, "cpu_baseline_one_thread", oracle_decode_single_thread,
                             (prob2,)))
            cpu_jobs.append((out["tiny_decode_f32"], "cpu_baseline_one_thread",
                             oracle_decode_single_thread, (prob1,)))

    if not a.no_cpu:
        torch.cuda.synchronize()
        out["host"] = host_info()
        for rec, key, fn, args in cpu_jobs:
            log(f"oracle on the host: {key} of {args[0].name}")
            rec[key] = fn(*args)
    line = json.dumps(out)
    print(line, flush=True)
    if a.json_out:
        with open(a.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
