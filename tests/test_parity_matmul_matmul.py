"""GPU parity of MatMul+MatMul (attn_matmul_matmul, through the C ABI) against the fp64 oracle.

The pages state no tolerance for this subgraph; the bar is derived from the
kernel's arithmetic (``oracle.matmul_matmul.error_bounds``): the intermediate
tau Q K^T is formed in fp32, rounded to bf16 and multiplied by V with fp32
accumulation, so every fp32-output element must lie within the first-order
worst-case bound, and the mean absolute error within the mean of the
independent-rounding RMS bound.  With ternary Q and K and tau = 1 every
intermediate entry is a small integer (exact in bf16) and only fp32
accumulation remains, a bound tight enough that one dropped or misplaced key
fails it.  bf16-output O must equal round-to-nearest-even of the fp32-output O
bit for bit.
"""
import time

import numpy as np
import pytest
import torch

import reduction_attention_gqa_amd as ra
from gpu_helpers import DeviceProblem, PagedDeviceProblem, report, v_rows
from oracle import error_bounds, matmul_matmul
from synthetic.inputs import make_problem, mm_workload

pytestmark = pytest.mark.gpu


def _run(d):
    ra.attn_matmul_matmul(d.problem(), d.q, d.k, d.v, d.o)
    torch.cuda.synchronize()
    return d.out()


def _check(name, got, p, exact_intermediate=False):
    want = matmul_matmul(p.q, p.k, v_rows(p), p.causal, p.scale)
    worst, rms = error_bounds(p.q, p.k, v_rows(p), p.causal, p.scale,
                              rounds_intermediate=not exact_intermediate)
    err = np.abs(got - want)
    report(name, got, want)
    ratio = float(np.max(np.divide(err, worst, out=np.zeros_like(err), where=worst > 0)))
    print(f"[{name}] max err / worst-case bound = {ratio:.3g}; mean err {err.mean():.3g} vs "
          f"mean rms bound {rms.mean():.3g}", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert np.all(err <= worst), f"{name}: error above the worst-case bound (ratio {ratio:.3g})"
    assert err.mean() <= rms.mean(), f"{name}: mean error above the rms bound"


@pytest.mark.parametrize("causal", [False, True])
def test_exact_intermediate(causal):
    # 2 requests x 300 queries x 4 heads per KV head = 1200 rows (five 256-row
    # tiles, a ragged last one); 300 and 77 keys (a ragged key tail; causal
    # rows of request 1 before position 223 see no key); NaN padding past each
    # length and in the unused capacity.
    p = make_problem(dtype="bf16", batch=2, lq=300, hq=8, hkv=2, dqk=128, dv=128,
                     kv_len=[300, 77], lcap=320, seed=51, causal=causal, scale=1.0,
                     qk_ternary=True)
    d = DeviceProblem(p, o_dtype="f32")
    _check(f"mm exact causal={causal}", _run(d), p, exact_intermediate=True)


@pytest.mark.parametrize("causal", [False, True])
def test_normal_inputs(causal):
    p = make_problem(dtype="bf16", batch=2, lq=260, hq=8, hkv=2, dqk=128, dv=128,
                     kv_len=[260, 133], seed=52, causal=causal)
    d = DeviceProblem(p, o_dtype="f32", layout="head")
    _check(f"mm normal causal={causal}", _run(d), p)


def test_bf16_output_is_rne_of_fp32_output():
    p = make_problem(dtype="bf16", batch=1, lq=128, hq=4, hkv=1, dqk=128, dv=128, kv_len=200,
                     seed=53)
    d32 = DeviceProblem(p, o_dtype="f32")
    d16 = DeviceProblem(p, o_dtype="bf16")
    _run(d32)
    _run(d16)
    assert torch.equal(d16.o, d32.o.to(torch.bfloat16)), "bf16 O != RNE(fp32 O)"


@pytest.mark.parametrize("page_size", [16, 1])
def test_paged_kv(page_size):
    p = make_problem(dtype="bf16", batch=3, lq=70, hq=8, hkv=2, dqk=128, dv=128,
                     kv_len=[90, 1, 257], lcap=260, seed=54, causal=True, scale=1.0,
                     qk_ternary=True)
    d = PagedDeviceProblem(p, page_size, o_dtype="f32")
    _check(f"mm paged ps={page_size}", _run(d), p, exact_intermediate=True)


def test_no_keys_gives_zero():
    p = make_problem(dtype="bf16", batch=2, lq=5, hq=4, hkv=2, dqk=128, dv=128,
                     kv_len=[0, 3], lcap=8, seed=55)
    d = DeviceProblem(p, o_dtype="f32")
    got = _run(d)
    assert np.all(got[0] == 0.0)
    _check("mm empty request", got, p)


def test_full_size_whole_output():
    # The full workload (B=4, 4096 queries and keys, 32/8 heads, D=128, no
    # mask) in the launch configuration the benchmark times: every output
    # element within its worst-case bound, the mean error within the mean RMS
    # bound.
    p = mm_workload("llama3_8b_matmul_matmul_prefill")
    print(f"[case] {p.name}: B={p.batch} Lq={p.lq} L={p.lcap} heads {p.hq}/{p.hkv}", flush=True)
    d = DeviceProblem(p, o_dtype="f32", pad=0.0)
    got = _run(d)
    t0 = time.perf_counter()
    _check("mm whole output", got, p)
    print(f"[oracle] {p.name}: whole output and bounds in {time.perf_counter() - t0:.1f} s",
          flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_keys_and_ragged_queries(causal):
    # Packed keys (kv_indptr) and packed ragged queries (q_indptr): request b
    # keeps its first q_lens[b] query rows, bottom-right causal alignment with
    # its own row count; the spare O rows after the last request stay unwritten.
    from gpu_helpers import PackedDeviceProblem
    p = make_problem(dtype="bf16", batch=3, lq=300, hq=8, hkv=2, dqk=128, dv=128,
                     kv_len=[260, 40, 300], seed=57, causal=causal, scale=1.0, qk_ternary=True)
    q_lens = [300, 17, 0]
    d = PackedDeviceProblem(p, q_lens=q_lens, o_dtype="f32")
    ra.attn_matmul_matmul(d.problem(), d.q, d.k, d.v, d.o)
    torch.cuda.synchronize()
    out = d.o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(out[d.tq:])), "rows past the last request were written"
    got = out[:d.tq]
    want, worst = [], []
    vr = v_rows(p)
    for b, n in enumerate(q_lens):
        if n == 0:
            continue
        qb = p.q[b:b + 1, :n]
        want.append(matmul_matmul(qb, [p.k[b]], [vr[b]], causal, p.scale)[0])
        worst.append(error_bounds(qb, [p.k[b]], [vr[b]], causal, p.scale,
                                  rounds_intermediate=False)[0][0])
    want, worst = np.concatenate(want), np.concatenate(worst)
    report(f"mm packed causal={causal}", got, want)
    assert np.all(np.abs(got - want) <= worst)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_shape(causal):
    # One query row per request (the decode setting of Cleave §7.3): G = 4 rows
    # per KV head, key counts from 1 to 3000 (one row tile per (request, KV
    # head), most of its rows empty); for Lq = 1 the causal flag changes nothing.
    p = make_problem(dtype="bf16", batch=4, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[3000, 1, 517, 64], lcap=3008, seed=58, causal=causal, scale=1.0,
                     qk_ternary=True)
    d = DeviceProblem(p, o_dtype="f32", layout="head")
    _check(f"mm decode causal={causal}", _run(d), p, exact_intermediate=True)
