"""GPU parity of split decode against the fp64 oracle (through the C ABI), both
as two launches (attn_decode_split + attn_combine) and as attn_decode (one
launch: the last split of each (request, KV head) merges the partials).

Tolerances: bf16 inputs with fp32 accumulation, max abs 1e-2 and mean abs
1e-3; the fp32 workload, 1e-5.  K/V rows past each request's length hold NaN,
so any read of a row that should not be read poisons the output.
"""
import time

import numpy as np
import pytest
import torch

from gpu_helpers import (BF16_MAX, BF16_MEAN, F32_MAX, F32_MEAN, DeviceProblem, assert_close,
                         assert_lse_close, v_rows)
from oracle import attention
from synthetic.inputs import make_problem, workload

pytestmark = pytest.mark.gpu


def _oracle(p):
    return attention(p.q, p.k, v_rows(p), p.causal, p.scale)


def test_tiny_gqa_decode_f32_s4():
    p = workload("tiny_gqa_decode_f32")
    d = DeviceProblem(p)
    plan = d.decode(s_request=p.s)
    assert plan.s_max == 4 and plan.chunk == 64
    o, lse = _oracle(p)
    assert_close("tiny_gqa_decode_f32", d.out(), o, F32_MAX, F32_MEAN)
    assert_lse_close("tiny_gqa_decode_f32", d.lse_out(), lse, 1e-5)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("s", [0, 1, 2, 3, 4, 7, 8, 16, 1000])
def test_gqa_d128_split_sweep(s, fused):
    # Llama-3-8B heads (32/8, D=128) at reduced batch and ragged lengths that
    # end mid-tile; every split count must give the same answer within tolerance.
    p = make_problem(dtype="bf16", batch=3, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[1000, 2311, 37], lcap=2400, seed=1)
    d = DeviceProblem(p)
    plan = d.decode(s_request=s, fused=fused)
    o, lse = _oracle(p)
    assert_close(f"gqa_d128 s={s} fused={fused} (kernel {plan.kernel}, s_max {plan.s_max})",
                 d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"gqa_d128 s={s} fused={fused}", d.lse_out(), lse)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("layout", ["token", "head"])
def test_gqa_g8_ragged_log_uniform(layout, fused):
    # Qwen3-32B heads (64/8): G = 8 query heads per KV head.
    p = make_problem(dtype="bf16", batch=6, lq=1, hq=64, hkv=8, dqk=128, dv=128,
                     kv_len=(128, 3000), lcap=3000, seed=2)
    d = DeviceProblem(p, layout=layout)
    d.decode(fused=fused)
    o, lse = _oracle(p)
    assert_close(f"gqa_g8 {layout}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"gqa_g8 {layout}", d.lse_out(), lse)


def test_empty_and_single_key_requests():
    p = make_problem(dtype="bf16", batch=4, lq=1, hq=8, hkv=2, dqk=128, dv=128,
                     kv_len=[0, 1, 129, 0], lcap=200, seed=3)
    d = DeviceProblem(p)
    d.decode()
    out = d.out()
    o, lse = _oracle(p)
    assert np.all(out[0] == 0) and np.all(out[3] == 0)
    assert np.all(np.isneginf(d.lse_out()[0]))
    # one visible key: O is that key's V row exactly (bf16 in, bf16 out)
    np.testing.assert_array_equal(out[1, 0], np.repeat(p.v[1][0], 4, axis=0))
    assert_close("empty/single", out, o, BF16_MAX, BF16_MEAN)
    assert_lse_close("empty/single", d.lse_out(), lse)


def test_fp32_output_and_bf16_output_is_its_rounding():
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[777, 1500], seed=4)
    d32 = DeviceProblem(p, o_dtype="f32")
    plan = d32.decode()
    d16 = DeviceProblem(p, o_dtype="bf16")
    d16.decode(plan=plan)
    o, _ = _oracle(p)
    assert_close("fp32 out", d32.out(), o, BF16_MAX, BF16_MEAN)
    assert torch.equal(d16.o, d32.o.to(torch.bfloat16))


def test_causal_multi_row_decode_bottom_right():
    # Two query rows per request (e.g. speculative decoding): row i sees keys
    # j <= i + L - 2.
    p = make_problem(dtype="bf16", batch=3, lq=2, hq=16, hkv=2, dqk=128, dv=128,
                     kv_len=[1, 300, 513], lcap=600, seed=5, causal=True)
    d = DeviceProblem(p)
    d.decode(s_request=3)
    o, lse = _oracle(p)
    assert_close("causal lq=2", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close("causal lq=2", d.lse_out(), lse)


def test_generic_kernel_bf16_head_dim_64():
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=12, hkv=3, dqk=64, dv=64,
                     kv_len=[190, 65], seed=6)
    d = DeviceProblem(p)
    plan = d.decode()
    assert plan.kernel == 0
    o, lse = _oracle(p)
    assert_close("generic d64", d.out(), o, BF16_MAX, BF16_MEAN)


@pytest.mark.parametrize("fused", [False, True])
def test_deterministic_bitwise(fused):
    # The single-launch merge always sums the splits in split order, whichever
    # split arrives last, so repeated calls agree bit for bit.
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[2048, 999], seed=7)
    d = DeviceProblem(p)
    plan = d.decode(fused=fused)
    first = d.o.clone()
    for _ in range(3):
        d.o.fill_(0)
        d.decode(plan=plan, fused=fused)
        assert torch.equal(first, d.o)


def test_fused_decode_reuses_workspace_and_leaves_counters_zero():
    # One problem (ragged, with a one-key request) twice through one workspace:
    # the arrival counters must be back at zero after every call.
    import reduction_attention_gqa_amd as ra
    p = make_problem(dtype="bf16", batch=4, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[4000, 300, 1, 2500], lcap=4096, seed=8)
    d = DeviceProblem(p)
    plan = ra.attn_decode_plan(d.problem(), 8, list(p.lens))
    assert plan.s_max > 1
    ws = ra.workspace(plan, "cuda")
    o, lse = _oracle(p)
    for _ in range(2):
        d.o.fill_(float("nan"))
        d.decode(plan=plan, ws=ws)
        assert int(ws[2].abs().sum()) == 0
        assert_close("fused reuse", d.out(), o, BF16_MAX, BF16_MEAN)
        assert_lse_close("fused reuse", d.lse_out(), lse)


_FULL = {}


def _full_oracle(name):
    """The workload and its whole fp64 oracle output, computed once per module."""
    if name not in _FULL:
        p = workload(name)
        t0 = time.perf_counter()
        o, lse = _oracle(p)
        print(f"[oracle] {name}: whole output in {time.perf_counter() - t0:.1f} s", flush=True)
        _FULL[name] = (p, o, lse)
    return _FULL[name]


@pytest.mark.parametrize("layout", ["head", "token"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["llama3_8b_gqa_decode", "ragged_decode_qwen3_32b"])
def test_full_size_decode_whole_output(name, fused, layout):
    # The full workload in the launch configuration the benchmark times
    # (planner-chosen s, attn_decode, head-major cache; token-major and the
    # two-launch form as well), every output element against the oracle.
    print(f"[case] {name} fused={fused} layout={layout}", flush=True)
    p, o, lse = _full_oracle(name)
    d = DeviceProblem(p, layout=layout)
    plan = d.decode(fused=fused)
    print(f"[plan] {name}: kernel={plan.kernel} s_max={plan.s_max} chunk={plan.chunk}", flush=True)
    assert_close(f"{name} whole output", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"{name} whole output", d.lse_out(), lse)


@pytest.mark.parametrize("layout", ["head", "token"])
@pytest.mark.parametrize("s", [2, 4, 8])
def test_full_size_llama_forced_splits(s, layout):
    # The Llama decode shape with the key axis split s ways (the planner takes
    # s = 1 here): the single-launch merge of every (request, KV head) at full
    # size, every output element against the oracle.
    print(f"[case] llama s={s} layout={layout}", flush=True)
    p, o, lse = _full_oracle("llama3_8b_gqa_decode")
    d = DeviceProblem(p, layout=layout)
    plan = d.decode(s_request=s)
    assert plan.s_max == s
    assert_close(f"llama s={s} {layout}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"llama s={s} {layout}", d.lse_out(), lse)


@pytest.mark.parametrize("fused", [False, True])
def test_device_lengths_beyond_the_plan_write_nan(fused):
    # The plan is made from host lengths that are shorter than the device's:
    # request 1 holds 2000 keys on the device but was planned with 1000, so
    # s_max * chunk (4 x 256) does not cover it.  Two launches: its rows come
    # out NaN instead of a silently truncated result and the other requests
    # are exact.  One launch: the runs of rounds per workgroup were cut from
    # the planned total, which the device's exceeds, so every workgroup writes
    # NaN for the rows it meets and no row holds a result.  The arrival
    # counters stay zero either way.
    import reduction_attention_gqa_amd as ra
    p = make_problem(dtype="bf16", batch=3, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[1000, 2000, 300], lcap=2048, seed=9)
    d = DeviceProblem(p)
    plan = ra.attn_decode_plan(d.problem(), 4, [1000, 1000, 300])
    assert plan.s_max * plan.chunk < 2000
    ws = ra.workspace(plan, "cuda")
    d.decode(plan=plan, ws=ws, fused=fused)
    out, lse = d.out(), d.lse_out()
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    if fused:
        assert np.isnan(out).all()
    else:
        o, lse_want = _oracle(p)
        keep = [0, 2]
        assert_close("beyond plan, other requests", out[keep], o[keep], BF16_MAX, BF16_MEAN)
        assert_lse_close("beyond plan, other requests", lse[keep], lse_want[keep])
    assert int(ws[2].abs().sum()) == 0


def test_more_work_items_than_planned_write_nan():
    # Host lengths [1000, 100, 300] plan 8 x (8 + 1 + 3) = 96 rounds of 128
    # keys; the device lengths [1000, 1000, 300] hold 152, so the runs of the
    # grid do not cover them.  Every workgroup writes NaN for the rows it meets
    # (and counts no arrival); rows no run reaches keep what O held (zero
    # here), so no row holds a result.
    import reduction_attention_gqa_amd as ra
    p = make_problem(dtype="bf16", batch=3, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                     kv_len=[1000, 1000, 300], lcap=1024, seed=10)
    d = DeviceProblem(p)
    plan = ra.attn_decode_plan(d.problem(), 4, [1000, 100, 300])
    assert plan.stream_rounds == 96 and plan.s_max * plan.chunk >= 1000
    ws = ra.workspace(plan, "cuda")
    d.o.fill_(0)
    d.decode(plan=plan, ws=ws, fused=True)
    out = d.out()
    assert np.isnan(out[0]).all() and np.isnan(out).any()
    assert np.all(np.isnan(out) | (out == 0))
    assert int(ws[2].abs().sum()) == 0


@pytest.mark.parametrize("layout", ["head", "token"])
def test_full_size_ragged_single_launch_bitwise_and_counters(layout):
    # The full ragged workload in one launch (the stream schedule: hundreds of
    # cut units whose pieces take their merge tickets as they start): repeated
    # calls agree bit for bit, and every arrival counter is back at zero.
    import reduction_attention_gqa_amd as ra
    p = workload("ragged_decode_qwen3_32b")
    print(f"[case] ragged_decode_qwen3_32b bitwise layout={layout}", flush=True)
    d = DeviceProblem(p, layout=layout)
    plan = ra.attn_decode_plan(d.problem(), 0, list(p.lens))
    assert plan.kernel == 1 and plan.s_max > 1 and plan.stream_pieces > 1
    ws = ra.workspace(plan, "cuda")
    d.decode(plan=plan, ws=ws)
    first, first_lse = d.o.clone(), d.lse.clone()
    assert int(ws[2].abs().sum()) == 0
    for _ in range(3):
        d.o.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        d.decode(plan=plan, ws=ws)
        assert torch.equal(first, d.o) and torch.equal(first_lse, d.lse)
        assert int(ws[2].abs().sum()) == 0
