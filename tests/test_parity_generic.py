"""GPU parity of the vector-ALU (generic) attention kernel against the fp64
oracle, through the C ABI: every output-pairs-per-thread instantiation (value
head dims up to 64, 128, 256 and 512), staged and unstaged K/V tiles, and the
single-launch merge at split counts on both sides of the largest one it
tabulates in LDS (64; more splits take the one-partial-at-a-time path).

Tolerances: fp32 inputs, max abs 1e-5 and mean abs 1e-5 (as the other fp32
tests); bf16 inputs 1e-2 / 1e-3.  K/V rows past each request's
length hold NaN.
"""
import pytest
import torch

from gpu_helpers import BF16_MAX, BF16_MEAN, F32_MAX, F32_MEAN, DeviceProblem, assert_close, \
    assert_lse_close, v_rows
from oracle import attention
from synthetic.inputs import make_problem

pytestmark = pytest.mark.gpu


def _oracle(p):
    return attention(p.q, p.k, v_rows(p), p.causal, p.scale)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dqk,dv", [(40, 24), (64, 64), (96, 100), (40, 200), (96, 300), (64, 512)])
def test_generic_f32_head_dims(dqk, dv, fused):
    # 16 query rows per workgroup: G = 4 heads x 4 KV heads; lengths end mid-tile.
    p = make_problem(dtype="f32", batch=3, lq=1, hq=16, hkv=4, dqk=dqk, dv=dv,
                     kv_len=[1, 130, 700], lcap=704, seed=31)
    d = DeviceProblem(p)
    plan = d.decode(fused=fused)
    assert plan.kernel == 0
    o, lse = _oracle(p)
    name = f"generic f32 dqk={dqk} dv={dv} fused={fused} s_max={plan.s_max}"
    assert_close(name, d.out(), o, F32_MAX, F32_MEAN)
    assert_lse_close(name, d.lse_out(), lse, 1e-5)


@pytest.mark.parametrize("dqk,dv", [(40, 24), (96, 300)])
def test_generic_bf16_head_dims(dqk, dv):
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=8, hkv=2, dqk=dqk, dv=dv,
                     kv_len=[77, 300], lcap=320, seed=32)
    d = DeviceProblem(p, layout="head")
    plan = d.decode()
    assert plan.kernel == 0
    o, lse = _oracle(p)
    assert_close(f"generic bf16 dqk={dqk} dv={dv}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"generic bf16 dqk={dqk} dv={dv}", d.lse_out(), lse)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("s", [63, 64, 65, 130])
def test_generic_merge_split_counts(s, fused):
    # 64-key tiles: the longest request (64 s keys) gives s_max = s, one tile
    # per split; the shorter ones have fewer splits, the empty one none.
    p = make_problem(dtype="f32", batch=4, lq=1, hq=8, hkv=2, dqk=64, dv=64,
                     kv_len=[64 * s, 4000, 1, 0], lcap=64 * s, seed=33)
    d = DeviceProblem(p)
    plan = d.decode(s_request=s, fused=fused)
    assert plan.kernel == 0 and plan.s_max == s
    o, lse = _oracle(p)
    name = f"generic merge s={s} fused={fused}"
    assert_close(name, d.out(), o, F32_MAX, F32_MEAN)
    assert_lse_close(name, d.lse_out(), lse, 1e-5)


@pytest.mark.parametrize("s", [64, 65])
def test_generic_merge_deterministic_bitwise(s):
    # The merge sums the splits in split order whichever split comes last.
    p = make_problem(dtype="f32", batch=2, lq=1, hq=8, hkv=2, dqk=64, dv=64,
                     kv_len=[64 * s, 2900], lcap=64 * s, seed=34)
    d = DeviceProblem(p)
    plan = d.decode(s_request=s)
    first, first_lse = d.o.clone(), d.lse.clone()
    for _ in range(3):
        d.o.fill_(0)
        d.lse.fill_(0)
        d.decode(plan=plan)
        assert torch.equal(first, d.o)
        assert torch.equal(first_lse, d.lse)


def test_generic_planner_small_problem_one_tile_per_split():
    # 256 keys of 64-key tiles on a GPU the work does not fill: four splits.
    p = make_problem(dtype="f32", batch=1, lq=1, hq=8, hkv=2, dqk=64, dv=64, kv_len=256, seed=35)
    d = DeviceProblem(p)
    plan = d.decode()
    assert plan.s_max == 4 and plan.chunk == 64
    o, lse = _oracle(p)
    assert_close("generic one tile per split", d.out(), o, F32_MAX, F32_MEAN)
