"""GPU parity of SwiGLU against the fp64 oracle, through the C ABI.

The kernel streams both weight matrices in one loop over K (horizontal
fusion, Cleave §7.3), split over K when the plan says so (Cleave §2.2
"Split-K", parts added before the gate); from 256 tokens on (the prefill
setting of Cleave §7.3) both MatMuls run as one tiled MFMA GEMM whose
workgroups hold a gate and an up tile of the same columns.  Tolerance derived from the
kernel's arithmetic (below) on the fp32 output; the bf16 output must be the
round-to-nearest-even of the fp32 one.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, assert_close
import reduction_attention_gqa_amd as ra
from oracle import swiglu
from synthetic.inputs import make_swiglu_problem, swiglu_workload

pytestmark = pytest.mark.gpu

# Tolerance derived from the kernel's arithmetic.  Its MFMA operands are exact
# (bf16 inputs), so every product is exact in fp32 and the
# only roundings are fp32 accumulation over K terms and the fp32 epilogue (the gate).
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


def _run(p, s_request=0, y_dtype=torch.float32, strides=(None, None, None), y_stride=None,
         tile_n=None):
    x, wg, wu = _dev(p.x, strides[0]), _dev(p.w_gate, strides[1]), _dev(p.w_up, strides[2])
    y = torch.full((p.m, y_stride or p.n), float("nan"), dtype=y_dtype, device=DEV)[:, : p.n]
    prob = ra.make_swiglu_problem(x, wg, wu, y)
    cfg = ra.swiglu_plan(prob, s_request)
    if tile_n is not None:  # a tile width of the caller's choosing
        assert cfg.kernel == 0
        cfg.tile_n = tile_n
        cfg.grid[0] = -(-p.n // tile_n)
    ra.swiglu(prob, cfg, x, wg, wu, y, ra.swiglu_workspace(cfg, DEV))
    torch.cuda.synchronize()
    return y, cfg


def _check(name, p, rows=None, **kw):
    """H against the oracle (on the given rows only, when ``rows`` is set:
    the oracle's rows are independent), and bf16 H == RNE(fp32 H) everywhere."""
    rows = np.arange(p.m) if rows is None else np.asarray(rows)
    want = swiglu(p.x[rows], p.w_gate, p.w_up)
    y32, cfg = _run(p, **kw)
    assert_close(f"{name} (kernel {cfg.kernel}, s={cfg.s})",
                 y32[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64), want,
                 TOL_MAX, TOL_MEAN)
    y16, _ = _run(p, y_dtype=torch.bfloat16, **kw)
    assert torch.equal(y16, y32.to(torch.bfloat16)), f"{name}: bf16 H != RNE(fp32 H)"
    return cfg


@pytest.mark.parametrize("s", [0, 1, 2, 3, 8])
def test_tiny_split_counts(s):
    cfg = _check(f"tiny s={s}", swiglu_workload("tiny_swiglu"), s_request=s)
    if s:
        assert cfg.s == s


@pytest.mark.parametrize("s", [1, 4])
def test_ragged_tails(s):
    # m = 33 spans two token tiles; k = 264 ends mid k-step; n = 70 mid tile.
    _check(f"tails s={s}", make_swiglu_problem(m=33, k=264, n=70, seed=41), s_request=s)


def test_strided_rows():
    _check("strided", make_swiglu_problem(m=7, k=512, n=130, seed=42), s_request=3,
           strides=(520, 640, 576))


def test_full_size_decode():
    # Llama-3 8B's MLP at 32 tokens: K = 4096, N = 14336; every output checked,
    # with the planner's 56-column tiles on 256 workgroups.
    cfg = _check("llama3_8b decode", swiglu_workload("llama3_8b_swiglu_decode"))
    assert cfg.kernel == 0 and cfg.s == 1 and cfg.tile_n == 56 and cfg.grid[0] == 256


def test_one_part_equals_many_parts():
    p = make_swiglu_problem(m=16, k=1024, n=256, seed=43)
    y1, _ = _run(p, s_request=1)
    y8, _ = _run(p, s_request=8)
    np.testing.assert_allclose(y1.cpu().numpy(), y8.cpu().numpy(), rtol=0, atol=5e-5)


# The prefill setting (m >= 256 tokens, k a multiple of 64): the tiled GEMM.

def test_prefill_gemm_ragged_tiles():
    # m = 300 ends inside the second 256-row tile, n = 200 inside the second
    # 128-column tile; k = 320 is 5 steps of 64 columns, so the 2-stage ring
    # ends mid-cycle.
    cfg = _check("prefill ragged", make_swiglu_problem(m=300, k=320, n=200, seed=44))
    assert cfg.kernel == 1 and cfg.s == 1


def test_prefill_gemm_xcd_tile_order():
    # 16 column tiles of 128: the grid is ordered XCD by XCD.
    assert _check("prefill xcd order", make_swiglu_problem(m=512, k=256, n=16 * 128,
                                                           seed=45)).kernel == 1


def test_prefill_gemm_strided_rows():
    _check("prefill strided", make_swiglu_problem(m=270, k=320, n=150, seed=46),
           strides=(328, 352, 336))


def test_prefill_gemm_equals_split_kernel():
    # Same exact products as the streaming kernel; fp32 summation order differs.
    p = make_swiglu_problem(m=256, k=512, n=200, seed=47)
    y_gemm, cfg = _run(p)
    half = dataclasses.replace(p, x=np.ascontiguousarray(p.x[:128]))
    y_half, cfg_half = _run(half)
    assert cfg.kernel == 1 and cfg_half.kernel == 0
    np.testing.assert_allclose(y_gemm[:128].cpu().numpy(), y_half.cpu().numpy(), rtol=0, atol=5e-5)


def test_full_size_prefill_sampled_rows():
    # Llama-3 8B's MLP at 4096 tokens (K = 4096, N = 14336), in the launch
    # configuration the benchmark times; every column of the first and last
    # row of each 256-row tile and of 64 drawn rows.
    p = swiglu_workload("llama3_8b_swiglu_prefill")
    edges = [r for t in range(0, p.m, 256) for r in (t, t + 255)]
    drawn = np.random.default_rng(8).choice(p.m, 64, replace=False)
    rows = np.unique(np.concatenate([edges, drawn]))
    assert _check("llama3_8b prefill", p, rows=rows).kernel == 1


@pytest.mark.parametrize("m,k,n", [(256, 64, 1), (256, 64, 129), (257, 128, 3), (512, 192, 259)])
def test_prefill_gemm_edges(m, k, n):
    # One 64-column step and odd step counts, exactly one row tile and one row
    # past it, a single output column and ragged column counts.
    cfg = _check(f"edges {m}x{k}x{n}", make_swiglu_problem(m=m, k=k, n=n, seed=50 + m + n))
    assert cfg.kernel == 1


def test_prefill_gemm_padded_output_rows():
    p = make_swiglu_problem(m=300, k=128, n=200, seed=59)
    y, cfg = _run(p, y_stride=232)
    assert cfg.kernel == 1
    full = y.as_strided((p.m, 232), (232, 1))
    assert torch.isnan(full[:, 200:]).all() and not torch.isnan(y).any()
    assert_close("padded y", y.cpu().numpy().astype(np.float64), swiglu(p.x, p.w_gate, p.w_up),
                 TOL_MAX, TOL_MEAN)


@pytest.mark.parametrize("s", [1, 3])
@pytest.mark.parametrize("tile", [4, 20, 36, 56, 64])
def test_tile_widths(tile, s):
    # Workgroup tiles of 4 to 64 output columns: tiles that end inside a
    # 16-row MFMA block, and n = 203 ending inside a tile and inside a quad of
    # columns (columns past each tile belong to the next workgroup).
    p = make_swiglu_problem(m=5, k=320, n=203, seed=42)
    cfg = _check(f"tile {tile} s={s}", p, s_request=s, tile_n=tile)
    assert cfg.tile_n == tile and cfg.s == s

