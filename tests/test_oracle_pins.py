"""Pins for the fp64 oracle: values fixed by the mathematics, not by the oracle.

Each check below compares ``oracle.attention`` with something it does not
compute itself: the pure-Python brute force, torch's float64 CPU attention,
closed forms (all-zero Q, a dominant key, one or two visible keys) and exact
invariants of softmax attention (Cleave §2.2 "FlashAttention", Fig. 2).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, attention_rows, brute_attention
from synthetic.inputs import make_problem, workload


def _rand_case(rng, causal, g, hkv, lq, lens, d, dv):
    bsz = len(lens)
    hq = g * hkv
    q = rng.standard_normal((bsz, lq, hq, d))
    k = [rng.standard_normal((n, hkv, d)) for n in lens]
    v = [rng.standard_normal((n, hkv, dv)) for n in lens]
    return q, k, v


BRUTE_CASES = [
    # causal, G, Hkv, Lq, lens, D, Dv
    (False, 1, 1, 1, [5], 3, 2),
    (False, 2, 2, 2, [7, 3], 4, 3),
    (True, 4, 1, 3, [7, 3], 4, 3),
    (True, 2, 2, 3, [3, 1], 2, 2),
    (True, 1, 2, 3, [2, 5], 3, 1),      # Lq > L_b for request 0: empty causal rows
    (False, 4, 1, 1, [1, 6], 4, 3),
    (True, 2, 1, 2, [0, 4], 3, 2),      # an empty request
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_matches_brute_force(case):
    causal, g, hkv, lq, lens, d, dv = case
    rng = np.random.default_rng(100 + BRUTE_CASES.index(case))
    q, k, v = _rand_case(rng, causal, g, hkv, lq, lens, d, dv)
    scale = 0.7
    o, lse = attention(q, k, v, causal, scale)
    bo, bl = brute_attention(q.tolist(), [x.tolist() for x in k], [x.tolist() for x in v],
                             causal, scale, dv)
    bo = np.array(bo, dtype=np.float64).reshape(o.shape)
    bl = np.array(bl, dtype=np.float64)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-13)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-13)


def _torch_sdpa(q, k, v, causal, scale):
    """torch float64 CPU attention with KV heads repeated and a bottom-right mask."""
    bsz, lq, hq, _ = q.shape
    outs = []
    for b in range(bsz):
        kb, vb = k[b], v[b]
        n, hkv = kb.shape[0], kb.shape[1]
        g = hq // hkv
        qt = torch.tensor(q[b], dtype=torch.float64).permute(1, 0, 2)          # [Hq, Lq, D]
        kt = torch.tensor(kb, dtype=torch.float64).permute(1, 0, 2).repeat_interleave(g, 0)
        vt = torch.tensor(vb, dtype=torch.float64).permute(1, 0, 2).repeat_interleave(g, 0)
        mask = None
        if causal:
            i = torch.arange(lq)[:, None]
            j = torch.arange(n)[None, :]
            mask = j <= i + (n - lq)
        ob = torch.nn.functional.scaled_dot_product_attention(
            qt[None], kt[None], vt[None], attn_mask=mask, scale=scale)[0]
        outs.append(ob.permute(1, 0, 2).numpy())
    return np.stack(outs)


def test_matches_torch_sdpa_tiny_gqa_decode():
    p = workload("tiny_gqa_decode_f32")
    o, _ = attention(p.q, p.k, p.v, p.causal, p.scale)
    ref = _torch_sdpa(p.q.astype(np.float64), [x.astype(np.float64) for x in p.k],
                      [x.astype(np.float64) for x in p.v], False, p.scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,lq,n", [(True, 64, 64), (True, 17, 50), (False, 5, 300)])
def test_matches_torch_sdpa_gqa_slices(causal, lq, n):
    p = make_problem(dtype="bf16", batch=2, lq=lq, hq=8, hkv=2, dqk=128, dv=128,
                     kv_len=n, seed=3, causal=causal)
    o, _ = attention(p.q, p.k, p.v, p.causal, p.scale)
    ref = _torch_sdpa(p.q.astype(np.float64), [x.astype(np.float64) for x in p.k],
                      [x.astype(np.float64) for x in p.v], causal, p.scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    rng = np.random.default_rng(1)
    lq, n, hkv, g = 6, 9, 2, 3
    q = np.zeros((1, lq, hkv * g, 5))
    k = [rng.standard_normal((n, hkv, 5))]
    v = [rng.standard_normal((n, hkv, 4))]
    o, lse = attention(q, k, v, causal, 0.3)
    for i in range(lq):
        last = i + n - lq if causal else n - 1
        for h in range(hkv * g):
            want = v[0][: last + 1, h // g, :].mean(axis=0)
            np.testing.assert_allclose(o[0, i, h], want, rtol=0, atol=1e-14)
            assert abs(lse[0, i, h] - math.log(last + 1)) <= 1e-14


def test_dominant_key_closed_form():
    # Q = beta e0, K_jstar = e0, every other key has K[..., 0] = 0:
    # O = (e^{tau beta} V_jstar + sum_{j != jstar} V_j) / (e^{tau beta} + n - 1).
    rng = np.random.default_rng(2)
    n, d, dv, jstar, tau = 11, 6, 5, 4, 0.5
    for beta in (3.0, 100.0):
        k = rng.standard_normal((n, 1, d))
        k[:, 0, 0] = 0.0
        k[jstar, 0, :] = 0.0
        k[jstar, 0, 0] = 1.0
        v = rng.standard_normal((n, 1, dv))
        q = np.zeros((1, 1, 1, d))
        q[0, 0, 0, 0] = beta
        o, _ = attention(q, [k], [v], False, tau)
        big = math.exp(tau * beta) if tau * beta < 700 else None
        if big is not None:
            want = (big * v[jstar, 0] + (v[:, 0].sum(axis=0) - v[jstar, 0])) / (big + n - 1)
        else:
            want = v[jstar, 0]
        np.testing.assert_allclose(o[0, 0, 0], want, rtol=0, atol=1e-13)
    # tau*beta = 50: the output is the dominant row to within e^-50 * n.
    assert np.max(np.abs(o[0, 0, 0] - v[jstar, 0])) < 1e-12


def test_single_visible_key_is_exact():
    rng = np.random.default_rng(4)
    # causal row 0 of a square prefill sees only key 0; a request of length 1 too.
    q = rng.standard_normal((1, 4, 2, 8))
    k = [rng.standard_normal((4, 1, 8))]
    v = [rng.standard_normal((4, 1, 3))]
    o, lse = attention(q, k, v, True, 0.25)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], v[0][0, 0])
        s0 = 0.25 * float(np.dot(q[0, 0, h], k[0][0, 0]))
        assert abs(lse[0, 0, h] - s0) <= 4 * np.finfo(float).eps * max(1.0, abs(s0))
    o1, lse1 = attention(q[:, :1], [k[0][:1]], [v[0][:1]], False, 0.25)
    assert np.array_equal(o1[0, 0, 0], v[0][0, 0])


def test_two_keys_sigmoid_form():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 1, 7))
    k = [rng.standard_normal((2, 1, 7))]
    v = [rng.standard_normal((2, 1, 4))]
    tau = 0.9
    o, _ = attention(q, k, v, False, tau)
    s0 = tau * float(q[0, 0, 0] @ k[0][0, 0])
    s1 = tau * float(q[0, 0, 0] @ k[0][1, 0])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    want = sig(s0 - s1) * v[0][0, 0] + sig(s1 - s0) * v[0][1, 0]
    np.testing.assert_allclose(o[0, 0, 0], want, rtol=0, atol=1e-14)


def _small(seed, causal=False, lens=(13, 9), lq=3, g=2, hkv=2, d=8, dv=5):
    rng = np.random.default_rng(seed)
    return _rand_case(rng, causal, g, hkv, lq, list(lens), d, dv)


def test_invariant_key_value_permutation():
    q, k, v = _small(6)
    o, lse = attention(q, k, v, False, 0.4)
    perm = [np.random.default_rng(7).permutation(x.shape[0]) for x in k]
    o2, lse2 = attention(q, [k[b][perm[b]] for b in range(2)], [v[b][perm[b]] for b in range(2)],
                         False, 0.4)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_invariant_key_shift(causal):
    # Adding u to every key of KV head kvh leaves O unchanged and shifts LSE by tau q.u.
    q, k, v = _small(8, causal)
    tau = 0.35
    o, lse = attention(q, k, v, causal, tau)
    u = np.random.default_rng(9).standard_normal(k[0].shape[1:])      # [Hkv, D]
    o2, lse2 = attention(q, [x + u[None] for x in k], v, causal, tau)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    g = q.shape[2] // k[0].shape[1]
    shift = tau * np.einsum("bihd,hd->bih", q, np.repeat(u, g, axis=0))
    fin = np.isfinite(lse)
    np.testing.assert_allclose((lse2 - lse)[fin], shift[fin], rtol=0, atol=1e-12)


def test_invariant_linear_in_values_and_scale_transfer():
    q, k, v = _small(10, True)
    w = [x * 0 + np.random.default_rng(11 + i).standard_normal(x.shape) for i, x in enumerate(v)]
    a, c = 1.7, -0.6
    o1, _ = attention(q, k, v, True, 0.5)
    o2, _ = attention(q, k, w, True, 0.5)
    o3, _ = attention(q, k, [a * x + c * y for x, y in zip(v, w)], True, 0.5)
    np.testing.assert_allclose(o3, a * o1 + c * o2, rtol=0, atol=1e-12)
    o4, lse4 = attention(2.5 * q, k, v, True, 0.5 / 2.5)
    _, lse1 = attention(q, k, v, True, 0.5)
    np.testing.assert_allclose(o4, o1, rtol=0, atol=1e-12)
    fin = np.isfinite(lse1)
    np.testing.assert_allclose(lse4[fin], lse1[fin], rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    q, k, v = _small(12, True, g=4, hkv=2)
    o, lse = attention(q, k, v, True, 0.3)
    k_rep = [np.repeat(x, 4, axis=1) for x in k]          # head h reads h // G
    v_rep = [np.repeat(x, 4, axis=1) for x in v]
    o2, lse2 = attention(q, k_rep, v_rep, True, 0.3)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=0, atol=1e-13)


def test_mla_value_alias_equals_copy():
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=16, hkv=1, dqk=40, dv=32, kv_len=(3, 50),
                     seed=13, mla=True)
    v_view = [p.v_rows(b) for b in range(p.batch)]
    assert all(np.shares_memory(v_view[b], p.k[b]) for b in range(p.batch))
    o, _ = attention(p.q, p.k, v_view, False, p.scale)
    o2, _ = attention(p.q, p.k, [np.array(x, copy=True) for x in v_view], False, p.scale)
    assert np.array_equal(o, o2)
    np.testing.assert_allclose(p.scale, 1 / math.sqrt(40))


def test_rows_mode_equals_full_mode():
    p = make_problem(dtype="bf16", batch=2, lq=20, hq=4, hkv=2, dqk=16, dv=16,
                     kv_len=[20, 33], seed=14, causal=True)
    o, lse = attention(p.q, p.k, p.v, True, p.scale)
    rows = [(0, 0, 0), (0, 19, 3), (1, 5, 1), (1, 19, 2)]
    ro, rl = attention_rows(p.q, p.k, p.v, True, p.scale, rows)
    for r, (b, i, h) in enumerate(rows):
        np.testing.assert_allclose(ro[r], o[b, i, h], rtol=0, atol=1e-14)
        assert abs(rl[r] - lse[b, i, h]) <= 1e-14


def test_rejects_non_divisible_heads():
    q = np.zeros((1, 1, 3, 4))
    with pytest.raises(ValueError):
        attention(q, [np.zeros((2, 2, 4))], [np.zeros((2, 2, 4))], False, 1.0)
