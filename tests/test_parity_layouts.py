"""GPU parity of the paged and packed (variable-length) layouts against the
fp64 oracle, through the C ABI.

The oracle computes on each request's logical key rows; the layouts only
change where the kernels find those rows (a shuffled page pool, packed key
rows, packed ragged query rows).  Pool and packed rows that no request owns
hold NaN, so a read of a row that should not be read poisons the output, and
packed output rows that no request owns must stay NaN (never written).

Tolerances as for the plain layouts: bf16 max abs 1e-2, mean abs 1e-3; fp32
1e-5.
"""
import numpy as np
import pytest

from gpu_helpers import (BF16_MAX, BF16_MEAN, F32_MAX, F32_MEAN, PackedDeviceProblem,
                         PagedDeviceProblem, assert_close, assert_lse_close, v_rows)
from oracle import attention
from synthetic.inputs import make_problem

pytestmark = pytest.mark.gpu

LLAMA = dict(hq=32, hkv=8, dqk=128, dv=128)


def _oracle(p):
    return attention(p.q, p.k, v_rows(p), p.causal, p.scale)


def _oracle_ragged(p, q_lens):
    """Per request: its first q_lens[b] query rows as a request of their own
    (bottom-right causal alignment uses that request's own row count)."""
    vr = v_rows(p)
    outs, lses = [], []
    for b, n in enumerate(q_lens):
        if n == 0:
            continue
        o, lse = attention(p.q[b:b + 1, :n], [p.k[b]], [vr[b]], p.causal, p.scale)
        outs.append(o[0])
        lses.append(lse[0])
    return np.concatenate(outs), np.concatenate(lses)


def _tol(p):
    return (BF16_MAX, BF16_MEAN) if p.dtype == "bf16" else (F32_MAX, F32_MEAN)


# ------------------------------------------------------------ paged decode

@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("ps", [1, 16, 64, 256])
def test_paged_gqa_decode(ps, layout, fused):
    # Llama-3-8B heads; lengths that end mid-page and mid-tile, an empty and a
    # one-key request; the MFMA kernel gathers rows through the page table.
    p = make_problem(dtype="bf16", batch=4, lq=1, kv_len=[1000, 1, 0, 2311], lcap=2400,
                     seed=11, **LLAMA)
    d = PagedDeviceProblem(p, ps, layout=layout, seed=ps)
    plan = d.decode(fused=fused)
    assert plan.kernel == 1
    o, lse = _oracle(p)
    name = f"paged ps={ps} {layout} fused={fused} (s_max {plan.s_max})"
    assert_close(name, d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(name, d.lse_out(), lse)


@pytest.mark.parametrize("s", [1, 3, 1000])
def test_paged_gqa_decode_split_counts(s):
    p = make_problem(dtype="bf16", batch=3, lq=1, kv_len=[3000, 129, 2047], lcap=3000,
                     seed=12, hq=64, hkv=8, dqk=128, dv=128)
    d = PagedDeviceProblem(p, 16, seed=5)
    plan = d.decode(s_request=s)
    o, lse = _oracle(p)
    name = f"paged ps=16 s={s} (s_max {plan.s_max})"
    assert_close(name, d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(name, d.lse_out(), lse)


def test_paged_one_key_pages_split_at_the_page_id_bound():
    # One key per page: a split holds at most 8320 keys (its page ids must fit
    # in LDS), so a 9000-key request takes two splits even when one is asked for.
    p = make_problem(dtype="bf16", batch=2, lq=1, kv_len=[9000, 300], seed=13, **LLAMA)
    d = PagedDeviceProblem(p, 1, layout="head", seed=6)
    plan = d.decode(s_request=1)
    assert plan.kernel == 1 and plan.s_max == 2
    o, lse = _oracle(p)
    assert_close("paged ps=1 long", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close("paged ps=1 long", d.lse_out(), lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_non_power_of_two_pages_run_generic(dtype):
    p = make_problem(dtype=dtype, batch=3, lq=1, kv_len=[50, 0, 200], lcap=240, seed=14,
                     hq=8, hkv=2, dqk=128, dv=128)
    d = PagedDeviceProblem(p, 24, seed=7)
    plan = d.decode()
    assert plan.kernel == 0
    o, lse = _oracle(p)
    mx, mean = _tol(p)
    assert_close(f"paged ps=24 {dtype}", d.out(), o, mx, mean)
    assert_lse_close(f"paged ps=24 {dtype}", d.lse_out(), lse, 1e-3 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("fused", [False, True])
def test_paged_causal_query_rows(fused):
    # Four query rows per request over G = 4 (16 MFMA rows), bottom-right causal;
    # the 2-key request leaves rows 0 and 1 with no visible key.
    p = make_problem(dtype="bf16", batch=3, lq=4, kv_len=[2, 700, 63], lcap=720, seed=15,
                     causal=True, hq=16, hkv=4, dqk=128, dv=128)
    d = PagedDeviceProblem(p, 32, seed=8)
    plan = d.decode(s_request=2, fused=fused)
    assert plan.kernel == 1
    o, lse = _oracle(p)
    out = d.out()
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(d.lse_out()[0, :2]))
    assert_close(f"paged causal fused={fused}", out, o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"paged causal fused={fused}", d.lse_out(), lse)


@pytest.mark.parametrize("ps,s", [(1, 0), (1, 3), (64, 0), (48, 0)])
def test_paged_mla_decode(ps, s):
    # MLA (one latent KV head, V = first 512 columns of K); power-of-two pages
    # run on the MLA kernel, 48-key pages on the generic one.
    p = make_problem(dtype="bf16", batch=3, lq=1, hq=16, hkv=1, dqk=576, dv=512,
                     kv_len=[300, 77, 1031], lcap=1040, seed=16, mla=True)
    d = PagedDeviceProblem(p, ps, seed=9, layout="head" if ps == 1 else "token")
    plan = d.decode(s_request=s)
    assert plan.kernel == (0 if ps == 48 else 2)
    o, lse = _oracle(p)
    name = f"paged mla ps={ps} s={s} (s_max {plan.s_max})"
    assert_close(name, d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(name, d.lse_out(), lse)


def test_paged_mla_one_key_pages_split_at_the_page_id_bound():
    # One key per page: an MLA split holds at most 4064 keys.
    p = make_problem(dtype="bf16", batch=1, lq=2, hq=16, hkv=1, dqk=576, dv=512,
                     kv_len=[5000], seed=22, mla=True, causal=True)
    d = PagedDeviceProblem(p, 1, seed=23)
    plan = d.decode(s_request=1)
    assert plan.kernel == 2 and plan.s_max == 2
    o, lse = _oracle(p)
    assert_close("paged mla ps=1 long", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close("paged mla ps=1 long", d.lse_out(), lse)


@pytest.mark.parametrize("s", [0, 2])
def test_packed_key_mla_decode(s):
    p = make_problem(dtype="bf16", batch=3, lq=1, hq=16, hkv=1, dqk=576, dv=512,
                     kv_len=[300, 0, 1031], lcap=1040, seed=24, mla=True)
    d = PackedDeviceProblem(p)
    plan = d.decode(s_request=s)
    assert plan.kernel == 2
    o, lse = _oracle(p)
    assert_close(f"packed mla s={s}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"packed mla s={s}", d.lse_out(), lse)


# ------------------------------------------------------ packed-key decode

@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("s", [0, 3])
def test_packed_key_decode(s, fused):
    p = make_problem(dtype="bf16", batch=4, lq=1, kv_len=[0, 5, 1000, 130], lcap=1024,
                     seed=17, **LLAMA)
    d = PackedDeviceProblem(p)
    plan = d.decode(s_request=s, fused=fused)
    assert plan.kernel == 1
    o, lse = _oracle(p)
    name = f"packed keys s={s} fused={fused}"
    assert_close(name, d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(name, d.lse_out(), lse)


# --------------------------------------------------------- ragged prefill

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,dqk", [("bf16", 128), ("f32", 64)])
def test_ragged_prefill_packed(dtype, dqk, causal):
    # Packed queries and keys; one request without queries, one with more
    # queries than keys (causal: its first rows see nothing).
    q_lens = [5, 0, 64, 33]
    p = make_problem(dtype=dtype, batch=4, lq=64, kv_len=[5, 7, 200, 16], lcap=200,
                     seed=18, causal=causal, hq=8, hkv=2, dqk=dqk, dv=dqk)
    d = PackedDeviceProblem(p, q_lens=q_lens)
    d.prefill()
    o, lse = _oracle_ragged(p, q_lens)
    out = d.out()
    got_lse = d.lse_out()
    tq = d.tq
    assert np.isnan(out[tq:]).all() and np.isnan(got_lse[tq:]).all()  # rows no request owns
    mx, mean = _tol(p)
    name = f"ragged prefill {dtype} causal={causal}"
    assert_close(name, out[:tq], o, mx, mean)
    assert_lse_close(name, got_lse[:tq], lse, 1e-3 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("ps", [1, 2, 16, 128, 24])
def test_paged_prefill(ps):
    # Prefill over a paged cache (a prefix already cached): 96 new rows per
    # request, bottom-right causal against up to 700 keys.
    p = make_problem(dtype="bf16", batch=3, lq=96, kv_len=[96, 700, 301], lcap=704,
                     seed=19, causal=True, **LLAMA)
    d = PagedDeviceProblem(p, ps, seed=10)
    d.prefill()
    o, lse = _oracle(p)
    assert_close(f"paged prefill ps={ps}", d.out(), o, BF16_MAX, BF16_MEAN)
    assert_lse_close(f"paged prefill ps={ps}", d.lse_out(), lse)


@pytest.mark.parametrize("kv", ["packed", "paged16", "paged1"])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_prefill_several_row_tiles(causal, kv):
    # Packed queries over G = 4: 100 and 257 query rows span two and five
    # 256-row tiles; one request has no query and one a single query row.
    q_lens = [100, 0, 257, 1]
    p = make_problem(dtype="bf16", batch=4, lq=257, kv_len=[300, 10, 257, 1000], lcap=1024,
                     seed=20, causal=causal, **LLAMA)
    if kv == "packed":
        d = PackedDeviceProblem(p, q_lens=q_lens)
    else:
        d = PagedDeviceProblem(p, int(kv[5:]), q_lens=q_lens, seed=21)
    d.prefill()
    o, lse = _oracle_ragged(p, q_lens)
    out, got_lse, tq = d.out(), d.lse_out(), d.tq
    assert np.isnan(out[tq:]).all() and np.isnan(got_lse[tq:]).all()
    name = f"ragged prefill {kv} causal={causal}"
    assert_close(name, out[:tq], o, BF16_MAX, BF16_MEAN)
    assert_lse_close(name, got_lse[:tq], lse)
