"""Pins of the MatMul+MatMul oracle (CPU only).

Checked against things other than itself: the pure-Python brute force (an
independent writing with exactly rounded sums), closed forms (a zero query
gives zero; a query that matches one key and is orthogonal to the others
picks that key's value row scaled by tau * beta), invariants (linear in V and
in tau; GQA equals MHA with each KV head repeated for its group; permuting
keys and values together changes nothing without a mask), and the error
bounds from both sides: a simulated bf16-intermediate kernel stays inside
them, and on constructed inputs a CPU model of the kernel's arithmetic
reaches most of each of their terms, so a bound made looser fails as surely
as one made tighter.  Planted mistakes in a copy of the oracle (in the
definition and in the bounds) must each fail a pin.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import brute_matmul_matmul, error_bounds, matmul_matmul, matmul_matmul_rows

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "matmul_matmul.py")

CASES = [  # (causal, G, Hkv, Lq, lens, d, dv)
    (False, 2, 2, 3, [5, 2], 4, 3),
    (True, 2, 2, 3, [5, 2], 4, 3),
    (True, 1, 1, 4, [4, 1], 3, 2),
    (False, 4, 1, 2, [6, 0], 3, 2),
    (True, 1, 2, 5, [3], 2, 2),      # causal with Lq > L_b: early rows see no key
]


def _case(seed, causal, g, hkv, lq, lens, d, dv):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((len(lens), lq, g * hkv, d))
    k = [rng.standard_normal((n, hkv, d)) for n in lens]
    v = [rng.standard_normal((n, hkv, dv)) for n in lens]
    return q, k, v


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("scale", [None, 0.7])
def test_definition_matches_brute_force(ci, scale):
    causal, g, hkv, lq, lens, d, dv = CASES[ci]
    q, k, v = _case(10 + ci, *CASES[ci])
    tau = 1.0 / math.sqrt(d) if scale is None else scale
    want = np.array(brute_matmul_matmul(q.tolist(), [x.tolist() for x in k],
                                        [x.tolist() for x in v], causal, tau, dv))
    got = matmul_matmul(q, k, v, causal, scale)
    np.testing.assert_allclose(got, want.reshape(got.shape), rtol=0, atol=1e-12)


def test_rows_match_full():
    causal, g, hkv, lq, lens, d, dv = CASES[1]
    q, k, v = _case(3, *CASES[1])
    full = matmul_matmul(q, k, v, causal, 0.5)
    rows = [(0, 2, 3), (1, 0, 1), (1, 2, 0), (0, 0, 2)]
    got = matmul_matmul_rows(q, k, v, causal, 0.5, rows)
    for r, (b, i, h) in enumerate(rows):
        np.testing.assert_allclose(got[r], full[b, i, h], rtol=0, atol=1e-14)


def test_zero_query_gives_zero():
    q, k, v = _case(4, *CASES[0])
    out = matmul_matmul(np.zeros_like(q), k, v, False)
    assert np.all(out == 0.0)


def test_one_matching_key_selects_its_value_row():
    # Q = beta e0, K_j* = e0, every other key has K[..., 0] = 0: T_ij = tau beta
    # at j* and 0 elsewhere, so O = tau beta V_j*.
    rng = np.random.default_rng(5)
    n, d, dv, beta, tau, jstar = 9, 6, 4, 3.0, 0.25, 4
    kb = rng.standard_normal((n, 1, d))
    kb[:, 0, 0] = 0.0
    kb[jstar, 0, :] = 0.0
    kb[jstar, 0, 0] = 1.0
    vb = rng.standard_normal((n, 1, dv))
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = beta
    out = matmul_matmul(q, [kb], [vb], False, tau)
    np.testing.assert_allclose(out[0, 0, 0], tau * beta * vb[jstar, 0], rtol=0, atol=1e-14)


def test_linear_in_values_and_scale():
    q, k, v = _case(6, *CASES[0])
    base = matmul_matmul(q, k, v, False, 0.5)
    v2 = [3.0 * x for x in v]
    np.testing.assert_allclose(matmul_matmul(q, k, v2, False, 0.5), 3.0 * base, rtol=1e-13,
                               atol=1e-13)
    np.testing.assert_allclose(matmul_matmul(q, k, v, False, 1.5), 3.0 * base, rtol=1e-13,
                               atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    causal, g, hkv, lq, lens, d, dv = CASES[1]
    q, k, v = _case(7, *CASES[1])
    k_rep = [np.repeat(x, g, axis=1) for x in k]   # KV head j serves query heads j*G .. j*G+G-1
    v_rep = [np.repeat(x, g, axis=1) for x in v]
    np.testing.assert_allclose(matmul_matmul(q, k, v, causal), matmul_matmul(q, k_rep, v_rep, causal),
                               rtol=0, atol=1e-14)


def test_key_permutation_invariance_without_mask():
    q, k, v = _case(8, *CASES[0])
    perm = [np.random.default_rng(9).permutation(x.shape[0]) for x in k]
    kp = [x[p] for x, p in zip(k, perm)]
    vp = [x[p] for x, p in zip(v, perm)]
    np.testing.assert_allclose(matmul_matmul(q, kp, vp, False), matmul_matmul(q, k, v, False),
                               rtol=0, atol=1e-12)


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float32).numpy().astype(np.float64)


def test_error_bounds_hold_for_a_simulated_bf16_intermediate():
    # A CPU model of the kernel's arithmetic: T in fp32, rounded to bf16, T V in
    # fp32.  Its difference from the exact O must stay within ``worst`` and its
    # mean within the mean of ``rms``.
    rng = np.random.default_rng(11)
    lq, n, d, dv, tau = 16, 200, 32, 8, 1.0 / math.sqrt(32)
    q = _bf16(rng.standard_normal((1, lq, 1, d)))
    kb = _bf16(rng.standard_normal((n, 1, d)))
    vb = _bf16(rng.standard_normal((n, 1, dv)))
    exact = matmul_matmul(q, [kb], [vb], False, tau)
    t32 = (q[0, :, 0, :].astype(np.float32) @ kb[:, 0, :].astype(np.float32).T) * np.float32(tau)
    sim = (_bf16(t32).astype(np.float32) @ vb[:, 0, :].astype(np.float32)).astype(np.float64)
    err = np.abs(sim - exact[0, :, 0, :])
    worst, rms = error_bounds(q, [kb], [vb], False, tau)
    assert np.all(err <= worst[0, :, 0, :])
    assert err.mean() <= rms.mean()
    # and the bound is not vacuous: dropping one key's term breaks it somewhere
    t_drop = _bf16(t32)
    t_drop[:, 17] = 0.0
    sim_drop = t_drop @ vb[:, 0, :]
    assert np.any(np.abs(sim_drop - exact[0, :, 0, :]) > worst[0, :, 0, :])


MUTANTS = {
    "scale_dropped": ("t = scale * np.matmul(", "t = np.matmul("),
    "mask_ignored": ("return np.where(vis, t, 0.0)", "return t"),
    "gqa_modulo_heads": ("kb_all[:, h // g, :], vis, scale)   # first MatMul",
                         "kb_all[:, h % hkv, :], vis, scale)   # first MatMul"),
    "values_reversed": ("o[b, :, h, :] = np.matmul(t, vb_all[:, h // g, :])",
                        "o[b, :, h, :] = np.matmul(t, vb_all[::-1, h // g, :])"),
    "first_product_transposed": ("np.asarray(kb, dtype=np.float64).T)",
                                 "np.asarray(kb, dtype=np.float64)[::-1].T)"),
}


def _load_mutant(name):
    src = open(SRC_PATH).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = src.replace("from .attention import visible_mask",
                      "from oracle.attention import visible_mask")
    mod = types.ModuleType(f"oracle_mm_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_brute_force(name):
    mod = _load_mutant(name)
    caught = False
    for ci, case in enumerate(CASES):
        causal, g, hkv, lq, lens, d, dv = case
        q, k, v = _case(20 + ci, *case)
        want = np.array(brute_matmul_matmul(q.tolist(), [x.tolist() for x in k],
                                            [x.tolist() for x in v], causal, 0.6, dv))
        got = mod.matmul_matmul(q, k, v, causal, 0.6)
        if not np.allclose(got, want.reshape(got.shape), rtol=0, atol=1e-9):
            caught = True
            break
    assert caught, f"mutant {name} passed every pin"


# --------------------------------------------------------------------------
# The bounds pinned from the other side: constructed inputs on which a CPU
# model of the kernel's arithmetic reaches most of each term of ``worst``, so
# that a bound made looser (a larger unit roundoff, a doubled fp32 term) fails
# as surely as one made tighter.

F32 = np.float32


def _kernel_model(q, kb, vb, tau):
    """One (request, head) as the kernel computes it: each intermediate entry
    an fp32 sum of exact bf16 products taken in key-dimension order, times tau
    in fp32, rounded to bf16; then fp32 sums of T V in key order.  q [Lq, d],
    kb [n, d], vb [n, dv] hold bf16 values.  Returns O (float64) and the fp32
    intermediate before its bf16 rounding."""
    lq, d = q.shape
    n, dv = vb.shape
    t = np.zeros((lq, n), dtype=np.float32)
    for i in range(lq):
        for j in range(n):
            acc = F32(0.0)
            for x in range(d):
                acc = F32(acc + F32(q[i, x]) * F32(kb[j, x]))
            t[i, j] = F32(F32(tau) * acc)
    t32 = t.copy()
    t = _bf16(t).astype(np.float32)
    o = np.zeros((lq, dv))
    for i in range(lq):
        for c in range(dv):
            acc = F32(0.0)
            for j in range(n):
                acc = F32(acc + t[i, j] * F32(vb[j, c]))
            o[i, c] = float(acc)
    return o, t32


def _tight_cases():
    """(name, q [Lq, d], k [n, d], v [n, dv], tau, rounds_intermediate, min ratio)."""
    cases = []
    # bf16 rounding of the intermediate: every entry 1 + 2^-8 - 2^-16 (exact in
    # fp32) rounds down to 1, an error of 0.996 u |T| per entry, all of one sign.
    n = 64
    q = np.array([[1.0, 1.0]])
    k = np.tile([1.0, 2.0 ** -8 * (1 - 2.0 ** -8)], (n, 1))
    cases.append(("bf16 intermediate", q, k, np.ones((n, 1)), 1.0, True, 0.9))
    # fp32 accumulation of the second product: a running sum of 1 that each of
    # 999 addends of 2^-24 (1 + 2^-7) pushes up by almost one unit roundoff.
    n = 1000
    v = np.full((n, 1), 2.0 ** -24 * (1 + 2.0 ** -7))
    v[0, 0] = 1.0
    cases.append(("fp32 second product", np.ones((1, 1)), np.ones((n, 1)), v, 1.0, False, 0.9))
    # fp32 sum of the first product with cancellation: 1, then 126 addends that
    # each round the sum up, then -1; the error is relative to A = tau |Q||K|^T
    # (about 2), not to the small |T| that is left.
    q = np.concatenate([[1.0], np.full(126, 2.0 ** -24 * (1 + 2.0 ** -7)), [-1.0]])[None, :]
    cases.append(("fp32 first product", q, np.ones((1, 128)), np.ones((1, 1)), 1.0, False, 0.45))
    return cases


def _bound_failures(bounds_fn):
    """Each constructed case where ``bounds_fn`` is violated or is too loose."""
    fails = []
    for name, q, k, v, tau, rounds, min_ratio in _tight_cases():
        assert np.array_equal(_bf16(q), q) and np.array_equal(_bf16(k), k)
        assert np.array_equal(_bf16(v), v)
        got, t32 = _kernel_model(q, k, v, tau)
        if not rounds:
            # the bound without the bf16 term needs every fp32 intermediate
            # to be a bf16 value already
            assert np.array_equal(_bf16(t32), t32.astype(np.float64))
        exact = matmul_matmul(q[None, :, None, :], [k[:, None, :]], [v[:, None, :]], False,
                              tau)[0, :, 0, :]
        worst, _ = bounds_fn(q[None, :, None, :], [k[:, None, :]], [v[:, None, :]], False, tau,
                             rounds_intermediate=rounds)
        worst = worst[0, :, 0, :]
        err = np.abs(got - exact)
        ratio = float(np.max(err / worst))
        if np.any(err > worst):
            fails.append(f"{name}: error above the bound (ratio {ratio:.3f})")
        elif ratio < min_ratio:
            fails.append(f"{name}: bound too loose (ratio {ratio:.3f} < {min_ratio})")
    return fails


def test_error_bounds_are_reached_on_constructed_inputs():
    assert _bound_failures(error_bounds) == []


def _rms_ratio(bounds_fn):
    """Mean error of the modelled kernel over the mean of the RMS bound, on
    normal data.  Rounding errors are uniform within at most u |T|, and the
    mean of |a sum of them| is about 0.8 of its RMS, so the ratio sits at a
    fixed fraction (about 0.6) of one: a doubled RMS bound is caught as well
    as a halved one."""
    rng = np.random.default_rng(5)
    lq, n, d, dv, tau = 24, 160, 16, 6, 1.0 / math.sqrt(16)
    q = _bf16(rng.standard_normal((lq, d)))
    k = _bf16(rng.standard_normal((n, d)))
    v = _bf16(rng.standard_normal((n, dv)))
    got, _ = _kernel_model(q, k, v, tau)
    exact = matmul_matmul(q[None, :, None, :], [k[:, None, :]], [v[:, None, :]], False,
                          tau)[0, :, 0, :]
    _, rms = bounds_fn(q[None, :, None, :], [k[:, None, :]], [v[:, None, :]], False, tau)
    return float(np.abs(got - exact).mean() / rms.mean())


RMS_RANGE = (0.35, 1.0)


def test_rms_bound_is_near_the_typical_error():
    assert RMS_RANGE[0] <= _rms_ratio(error_bounds) <= RMS_RANGE[1]


BOUND_MUTANTS = {
    "bf16_unit_roundoff_doubled": ("BF16_UNIT_ROUNDOFF = 2.0 ** -8", "BF16_UNIT_ROUNDOFF = 2.0 ** -7"),
    "bf16_unit_roundoff_halved": ("BF16_UNIT_ROUNDOFF = 2.0 ** -8", "BF16_UNIT_ROUNDOFF = 2.0 ** -9"),
    "second_product_term_doubled": ("worst[b, :, h, :] = ((u + n * e * (1 + u) ** 2)",
                                    "worst[b, :, h, :] = ((u + 2 * n * e * (1 + u) ** 2)"),
    "second_product_term_dropped": ("worst[b, :, h, :] = ((u + n * e * (1 + u) ** 2)",
                                    "worst[b, :, h, :] = ((u + 0 * n * e * (1 + u) ** 2)"),
    "first_product_term_doubled": ("+ (dqk + 1) * e * (1 + u) * (1 + n * e)",
                                   "+ 2 * (dqk + 1) * e * (1 + u) * (1 + n * e)"),
    "first_product_term_dropped": ("+ (dqk + 1) * e * (1 + u) * (1 + n * e)",
                                   "+ 0 * (dqk + 1) * e * (1 + u) * (1 + n * e)"),
    "rms_doubled": ("rms[b, :, h, :] = (u / math.sqrt(3.0) + n * e)",
                    "rms[b, :, h, :] = 2 * (u / math.sqrt(3.0) + n * e)"),
    "rms_halved": ("rms[b, :, h, :] = (u / math.sqrt(3.0) + n * e)",
                   "rms[b, :, h, :] = 0.5 * (u / math.sqrt(3.0) + n * e)"),
}


@pytest.mark.parametrize("name", sorted(BOUND_MUTANTS))
def test_planted_mistake_in_the_bounds_is_caught(name):
    src = open(SRC_PATH).read()
    old, new = BOUND_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = src.replace("from .attention import visible_mask",
                      "from oracle.attention import visible_mask")
    mod = types.ModuleType(f"oracle_mm_bound_mutant_{name}")
    exec(compile(src.replace(old, new), f"<bound mutant {name}>", "exec"), mod.__dict__)
    rms_ok = RMS_RANGE[0] <= _rms_ratio(mod.error_bounds) <= RMS_RANGE[1]
    assert _bound_failures(mod.error_bounds) or not rms_ok, f"bound mutant {name} passed every pin"
