"""GPU parity of RMSNorm followed by a MatMul against the fp64 oracle, through
the C ABI.

The kernel computes the rewritten graph (Cleave §1, Fig. 1: the Matmul on the
raw input with the rows' sums of squares beside it, the row scale applied
last), split over K (Cleave §2.2 "Split-K") when the plan says so, and from
256 tokens on (the prefill setting of Cleave §7.3) as a tiled MFMA GEMM; the
oracle is the definition (normalise, then multiply).  Tolerance derived from the
kernel's arithmetic (below) on the fp32 output, and the bf16 output must be
the round-to-nearest-even of the fp32 one.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, assert_close
import reduction_attention_gqa_amd as ra
from oracle import rmsnorm_matmul
from synthetic.inputs import make_rms_problem, rms_workload

pytestmark = pytest.mark.gpu

# Tolerance derived from the kernel's arithmetic.  Its MFMA operands are exact
# (bf16 inputs, and x g split into an exact bf16 high and low part, in both
# kernels), so every product is exact in fp32 and the
# only roundings are fp32 accumulation over K terms and the fp32 epilogue (the row scale from the fp32 sum of squares).
# With |Y| of order one and K <= 4096 the accumulated error is a random walk
# of about sqrt(K) fp32 roundings of the running sum, about 1e-6 (measured
# 5e-7 to 7e-7); the bar sits 100x above that and 100x below the error of a
# 1% scale mistake (an eps in the wrong place, a division by a padded K).
TOL_MAX, TOL_MEAN = 1e-4, 1e-5


def _dev(a, stride=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)
    if stride is None or stride == a.shape[-1]:
        return t
    wide = torch.full((a.shape[0], stride), float("nan"), dtype=torch.bfloat16, device=DEV)
    wide[:, : a.shape[1]] = t
    return wide[:, : a.shape[1]]


def _run(p, s_request=0, y_dtype=torch.float32, x_stride=None, w_stride=None, y_stride=None,
         tile_n=None):
    x, w = _dev(p.x, x_stride), _dev(p.w, w_stride)
    g = _dev(p.g[None, :])[0]
    y = torch.full((p.m, y_stride or p.n), float("nan"), dtype=y_dtype, device=DEV)[:, : p.n]
    prob = ra.make_rms_problem(x, g, w, y, eps=p.eps)
    plan = ra.rmsnorm_matmul_plan(prob, s_request)
    if tile_n is not None:  # a tile width of the caller's choosing
        assert plan.kernel == 0
        plan.tile_n = tile_n
        plan.grid[0] = -(-p.n // tile_n)
    ws = ra.rms_workspace(plan, DEV)
    ra.rmsnorm_matmul(prob, plan, x, g, w, y, ws)
    torch.cuda.synchronize()
    return y, plan


def _check(name, p, rows=None, **kw):
    """Y against the oracle (on the given rows only, when ``rows`` is set:
    the oracle's rows are independent), and bf16 Y == RNE(fp32 Y) everywhere."""
    rows = np.arange(p.m) if rows is None else np.asarray(rows)
    want = rmsnorm_matmul(p.x[rows], p.g, p.w, p.eps)
    y32, plan = _run(p, **kw)
    assert_close(f"{name} (kernel {plan.kernel}, s={plan.s})",
                 y32[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64), want,
                 TOL_MAX, TOL_MEAN)
    y16, _ = _run(p, y_dtype=torch.bfloat16, **kw)
    assert torch.equal(y16, y32.to(torch.bfloat16)), f"{name}: bf16 Y != RNE(fp32 Y)"
    return plan


@pytest.mark.parametrize("s", [0, 1, 2, 3, 8])
def test_tiny_split_counts(s):
    # n = 200 ends inside a 64-row tile; several splits over k = 256.
    p = rms_workload("tiny_rmsnorm_matmul")
    plan = _check(f"tiny s={s}", p, s_request=s)
    if s:
        assert plan.s == s


@pytest.mark.parametrize("s", [1, 4])
def test_ragged_tails(s):
    # m = 33 spans two 32-token tiles; k = 264 ends mid k-step; n = 70.
    p = make_rms_problem(m=33, k=264, n=70, seed=31)
    _check(f"tails s={s}", p, s_request=s)


def test_strided_rows():
    # X and W rows padded (NaN beyond k): only the first k columns may be read.
    p = make_rms_problem(m=7, k=512, n=130, seed=32)
    _check("strided", p, s_request=3, x_stride=520, w_stride=640)


def test_zero_and_tiny_rows():
    # A zero row gives Y = 0 (0 / sqrt(eps)); a tiny row is damped by eps.
    p = make_rms_problem(m=4, k=128, n=64, seed=33)
    p.x[1] = 0.0
    p.x[2] = (p.x[2] * np.float32(1e-3)).astype(np.float32)
    import synthetic.inputs as si
    p.x[2] = si.to_bf16_exact(p.x[2])
    y, _ = _run(p, s_request=2)
    assert torch.all(y[1] == 0)
    _check("zero/tiny rows", p, s_request=2)


def test_full_size_decode():
    # The Llama-3 8B decode shape (32 tokens, K = 4096, N = 14336) with the
    # planner's split; every output checked.
    p = rms_workload("llama3_8b_rmsnorm_matmul_decode")
    plan = _check("llama3_8b decode", p)
    # 56-row tiles on 256 workgroups: every tile boundary but every fourth
    # falls inside a 16-row MFMA block.
    assert plan.kernel == 0 and plan.s == 1 and plan.tile_n == 56 and plan.grid[0] == 256


def test_one_part_equals_many_parts():
    # The split and unsplit paths agree to fp32 rounding (different summation order).
    p = make_rms_problem(m=16, k=1024, n=256, seed=34)
    y1, _ = _run(p, s_request=1)
    y8, _ = _run(p, s_request=8)
    np.testing.assert_allclose(y1.cpu().numpy(), y8.cpu().numpy(), rtol=0, atol=2e-5)


def test_workspace_reused_across_calls():
    # One workspace serves call after call; each result matches the oracle.
    p = make_rms_problem(m=9, k=768, n=300, seed=35)
    want = rmsnorm_matmul(p.x, p.g, p.w, p.eps)
    x, w = _dev(p.x), _dev(p.w)
    g = _dev(p.g[None, :])[0]
    y = torch.empty((p.m, p.n), dtype=torch.float32, device=DEV)
    prob = ra.make_rms_problem(x, g, w, y, eps=p.eps)
    plan = ra.rmsnorm_matmul_plan(prob, 3)
    ws = ra.rms_workspace(plan, DEV)
    for call in range(3):
        y.fill_(float("nan"))
        ra.rmsnorm_matmul(prob, plan, x, g, w, y, ws)
        torch.cuda.synchronize()
        assert_close(f"reuse call {call}", y.cpu().numpy().astype(np.float64), want, TOL_MAX,
                     TOL_MEAN)


# The prefill setting (m >= 256 tokens, k a multiple of 64): the tiled GEMM.

def test_prefill_gemm_ragged_tiles():
    # m = 300 and n = 300 end inside the second 256-row / 256-column tile;
    # k = 320 is 5 steps of 64 columns, so the 2-stage ring ends mid-cycle.
    p = make_rms_problem(m=300, k=320, n=300, seed=36)
    plan = _check("prefill ragged", p)
    assert plan.kernel == 1 and plan.s == 1


def test_prefill_gemm_xcd_tile_order():
    # 8 column tiles: the grid is ordered XCD by XCD (column tiles x, x + 8, ..).
    p = make_rms_problem(m=512, k=256, n=8 * 256, seed=37)
    assert _check("prefill xcd order", p).kernel == 1


def test_prefill_gemm_strided_and_zero_rows():
    # Padded rows (NaN past k) and a zero row (Y = 0) through the GEMM path.
    p = make_rms_problem(m=260, k=320, n=96, seed=38)
    p.x[7] = 0.0
    y, plan = _run(p, x_stride=328, w_stride=352)
    assert plan.kernel == 1 and torch.all(y[7] == 0)
    _check("prefill strided", p, x_stride=328, w_stride=352)


def test_prefill_gemm_equals_split_kernel():
    # The two kernels compute the same exact products; only the fp32 summation
    # order differs.  The first 128 rows alone are planned on the streaming
    # kernel (m < 256).
    p = make_rms_problem(m=256, k=512, n=200, seed=39)
    y_gemm, plan = _run(p)
    half = dataclasses.replace(p, x=np.ascontiguousarray(p.x[:128]))
    y_half, plan_half = _run(half)
    assert plan.kernel == 1 and plan_half.kernel == 0
    np.testing.assert_allclose(y_gemm[:128].cpu().numpy(), y_half.cpu().numpy(), rtol=0, atol=2e-5)


def test_full_size_prefill_sampled_rows():
    # Llama-3 8B's projection at 4096 tokens (K = 4096, N = 14336), in the
    # launch configuration the benchmark times; every column of 96 rows: the
    # first and last row of each 256-row tile and 64 drawn rows.
    p = rms_workload("llama3_8b_rmsnorm_matmul_prefill")
    edges = [r for t in range(0, p.m, 256) for r in (t, t + 255)]
    drawn = np.random.default_rng(7).choice(p.m, 64, replace=False)
    rows = np.unique(np.concatenate([edges, drawn]))
    assert _check("llama3_8b prefill", p, rows=rows).kernel == 1


@pytest.mark.parametrize("m,k,n", [(256, 64, 1), (256, 64, 257), (257, 128, 3), (512, 192, 515)])
def test_prefill_gemm_edges(m, k, n):
    # One 64-column step (k = 64) and odd ones, exactly one row tile and one
    # row past it, a single output column and ragged column counts (odd n:
    # the bf16 output is written element by element at the tile's edge).
    p = make_rms_problem(m=m, k=k, n=n, seed=40 + m + n)
    assert _check(f"edges {m}x{k}x{n}", p).kernel == 1


def test_prefill_gemm_padded_output_rows():
    # Y with a row stride past n (NaN in the padding): the padding stays NaN.
    p = make_rms_problem(m=300, k=128, n=200, seed=49)
    y, plan = _run(p, y_stride=232)
    assert plan.kernel == 1
    full = y.as_strided((p.m, 232), (232, 1))
    assert torch.isnan(full[:, 200:]).all() and not torch.isnan(y).any()
    want = rmsnorm_matmul(p.x, p.g, p.w, p.eps)
    assert_close("padded y", y.cpu().numpy().astype(np.float64), want, TOL_MAX, TOL_MEAN)


@pytest.mark.parametrize("s", [1, 3])
@pytest.mark.parametrize("tile", [4, 20, 36, 56, 64])
def test_tile_widths(tile, s):
    # Workgroup tiles of 4 to 64 weight rows: tiles that end inside a 16-row
    # MFMA block, and n = 203 ending inside a tile and inside a quad of rows
    # (the rows past each tile belong to the next workgroup and must not be
    # written by this one).
    p = make_rms_problem(m=5, k=320, n=203, seed=41)
    plan = _check(f"tile {tile} s={s}", p, s_request=s, tile_n=tile)
    assert plan.tile_n == tile and plan.s == s

