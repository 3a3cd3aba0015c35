"""GPU parity of MLA-style decode (one latent KV head, V = K[..., :512]) against the oracle."""
import time

import numpy as np
import pytest

from gpu_helpers import BF16_MAX, BF16_MEAN, DeviceProblem, assert_close, assert_lse_close, v_rows
from oracle import attention
from synthetic.inputs import make_problem, workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("s", [0, 1, 3, 4, 6])
def test_mla_small(s):
    # s <= 4: the merge with every load issued ahead; more splits: the general merge.
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=128, hkv=1, dqk=576, dv=512,
                     kv_len=[300, 1000], lcap=1024, seed=41, mla=True)
    d = DeviceProblem(p)
    assert d.v.data_ptr() == d.k.data_ptr()
    plan = d.decode(s_request=s)
    o, lse = attention(p.q, p.k, v_rows(p), False, p.scale)
    assert_close(f"mla s={s} kernel={plan.kernel}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"mla s={s}", d.lse_out(), lse)


@pytest.mark.parametrize("fused", [True, False])
def test_mla_full_size_whole_output(fused):
    # The full MLA workload (B=64, 128 heads over one latent head, 8192 keys)
    # in the launch configuration the benchmark times; every output element
    # against the oracle.
    p = workload("mla_decode")
    print(f"[case] mla_decode whole output fused={fused}", flush=True)
    d = DeviceProblem(p)
    plan = d.decode(fused=fused)
    print(f"[plan] mla_decode: kernel={plan.kernel} s_max={plan.s_max} chunk={plan.chunk}",
          flush=True)
    t0 = time.perf_counter()
    o, lse = attention(p.q, p.k, v_rows(p), False, p.scale)
    print(f"[oracle] mla_decode: whole output in {time.perf_counter() - t0:.1f} s", flush=True)
    assert_close("mla whole output", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close("mla whole output", d.lse_out(), lse)


@pytest.mark.parametrize("s", [0, 2])
def test_mla_partial_row_groups_causal_two_queries(s):
    # 40 heads x 2 query rows = 80 rows: the last 16-row group is half empty;
    # causal bottom-right mask, a one-key request and ragged tails.
    p = make_problem(dtype="bf16", batch=3, lq=2, hq=40, hkv=1, dqk=576, dv=512,
                     kv_len=[1, 77, 645], lcap=704, seed=42, mla=True, causal=True)
    d = DeviceProblem(p)
    plan = d.decode(s_request=s)
    o, lse = attention(p.q, p.k, v_rows(p), True, p.scale)
    assert_close(f"mla causal lq=2 s={s} kernel={plan.kernel}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"mla causal lq=2 s={s}", d.lse_out(), lse)


def test_mla_single_launch_deterministic_empty_request_and_counters():
    # One launch (the last split of each request merges): repeated calls agree
    # bit for bit whichever split finishes last, an empty request gives O = 0
    # and LSE = -inf, and the arrival counters are zero after every call.
    import torch
    import reduction_attention_gqa_amd as ra
    p = make_problem(dtype="bf16", batch=3, lq=1, hq=128, hkv=1, dqk=576, dv=512,
                     kv_len=[2000, 513, 0], lcap=2048, seed=44, mla=True)
    d = DeviceProblem(p)
    plan = ra.attn_decode_plan(d.problem(), 4, list(p.lens))
    assert plan.kernel == 2 and plan.s_max == 4
    ws = ra.workspace(plan, "cuda")
    d.decode(plan=plan, ws=ws)
    first = d.o.clone()
    assert int(ws[2].abs().sum()) == 0
    o, lse = attention(p.q, p.k, v_rows(p), False, p.scale)
    assert_close("mla single launch", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close("mla single launch", d.lse_out(), lse)
    assert np.all(d.out()[2] == 0) and np.all(np.isneginf(d.lse_out()[2]))
    for _ in range(3):
        d.o.fill_(float("nan"))
        d.decode(plan=plan, ws=ws)
        assert torch.equal(first, d.o)
        assert int(ws[2].abs().sum()) == 0


def test_mla_device_length_beyond_the_plan_writes_nan():
    # Planned with 1000 keys for request 0 (4 splits of 256), which holds 2000
    # on the device: its rows are NaN, request 1 is exact, counters stay zero.
    import reduction_attention_gqa_amd as ra
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=128, hkv=1, dqk=576, dv=512,
                     kv_len=[2000, 700], lcap=2048, seed=45, mla=True)
    d = DeviceProblem(p)
    plan = ra.attn_decode_plan(d.problem(), 4, [1000, 700])
    assert plan.s_max * plan.chunk < 2000
    ws = ra.workspace(plan, "cuda")
    d.decode(plan=plan, ws=ws)
    out = d.out()
    assert np.isnan(out[0]).all() and np.isnan(d.lse_out()[0]).all()
    o, lse = attention(p.q, p.k, v_rows(p), False, p.scale)
    assert_close("mla beyond plan, request 1", out[1:], o[1:], BF16_MAX, BF16_MEAN)
    assert int(ws[2].abs().sum()) == 0


def test_mla_full_size_single_launch_bitwise_and_counters():
    # The full MLA workload in one launch (four splits per request, bf16
    # partials, the last split merging): repeated calls agree bit for bit,
    # and every arrival counter is back at zero.
    import torch
    import reduction_attention_gqa_amd as ra
    p = workload("mla_decode")
    print("[case] mla_decode bitwise", flush=True)
    d = DeviceProblem(p)
    plan = ra.attn_decode_plan(d.problem(), 0, list(p.lens))
    assert plan.kernel == 2 and plan.s_max == 4
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
