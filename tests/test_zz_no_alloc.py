"""attn_decode_noalloc (workspace in the library's device-resident scratch)
against attn_decode with a caller workspace, through the C ABI.

Two calls in a row through the shared scratch, the second smaller than the
first, each compared bit for bit with attn_decode on the same plan (same
kernels, so the same bits) and with the fp64 oracle at the bf16 bar; then an
MLA call (split + combine through the scratch) and a plan too large for the
scratch, which must be refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import reduction_attention_gqa_amd as ra
from gpu_helpers import BF16_MAX, BF16_MEAN, DeviceProblem, assert_close, assert_lse_close, v_rows
from oracle import attention
from synthetic.inputs import make_problem

pytestmark = pytest.mark.gpu


def _both(p, s_request=0):
    d = DeviceProblem(p)
    prob = d.problem()
    plan = ra.attn_decode_plan(prob, s_request, list(p.lens))
    ws = ra.workspace(plan, "cuda")
    ra.attn_decode(prob, plan, d.q, d.k, d.v, ws[0], ws[1], ws[2], d.o, d.lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = d.o.clone(), d.lse.clone()
    d.o.fill_(float("nan"))
    d.lse.fill_(float("nan"))
    ra.attn_decode_noalloc(prob, plan, d.q, d.k, d.v, d.o, d.lse)
    torch.cuda.synchronize()
    return d, plan, o_ref, lse_ref


def _check(name, p, s_request=0):
    print(f"[case] {name}", flush=True)
    d, plan, o_ref, lse_ref = _both(p, s_request)
    print(f"[plan] {name}: kernel={plan.kernel} s_max={plan.s_max} chunk={plan.chunk}", flush=True)
    assert torch.equal(d.o, o_ref), f"{name}: O differs from attn_decode"
    assert torch.equal(d.lse, lse_ref), f"{name}: LSE differs from attn_decode"
    o, lse = attention(p.q, p.k, v_rows(p), p.causal, p.scale)
    assert_close(name, d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(name, d.lse_out(), lse)
    return plan


def test_two_calls_in_a_row_second_smaller():
    big = make_problem(dtype="bf16", batch=6, lq=1, hq=64, hkv=8, dqk=128, dv=128,
                       kv_len=(128, 6000), lcap=6000, seed=61)
    plan = _check("noalloc call 1 (ragged, 6 requests)", big)
    assert plan.s_max > 1  # the single-launch merge runs through the scratch
    small = make_problem(dtype="bf16", batch=2, lq=1, hq=32, hkv=8, dqk=128, dv=128,
                         kv_len=[700, 65], lcap=704, seed=62)
    _check("noalloc call 2 (2 requests)", small, s_request=3)


def test_mla_through_the_scratch():
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=128, hkv=1, dqk=576, dv=512,
                     kv_len=[300, 1000], lcap=1024, seed=63, mla=True)
    _check("noalloc mla", p, s_request=3)


def test_plan_larger_than_the_scratch_is_refused():
    # 64 requests x 128 heads x 512 columns x 16 splits of fp32 partials is
    # 256 MiB, more than the scratch holds.
    q = torch.zeros((64, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 8192, 1, 576), dtype=torch.bfloat16, device="cuda")
    o = torch.full((64, 1, 128, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    prob = ra.make_problem(q, k, k[..., :512], o)
    plan = ra.attn_decode_plan(prob, 16)
    assert plan.ws_o_bytes > 96 << 20
    with pytest.raises(ra.AttnError) as e:
        ra.attn_decode_noalloc(prob, plan, q, k, k[..., :512], o)
    assert e.value.status == ra.ATTN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "a refused call wrote O"
