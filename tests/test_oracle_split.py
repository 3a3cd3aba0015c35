"""Pins for the oracle's split mode (Cleave §2.2 "Split-K", Fig. 3; §4, Fig. 5(b)).

The Split-K identity says the s partial reductions over contiguous parts sum
to the full reduction, whatever the partition.  For attention the partials are
a per-split row sum and a per-split value-product [s, S_Q, D]; the combine
reduces both over s and divides.  These tests check the oracle's split mode
against its unsplit mode (random, non-dividing, empty and oversized
partitions), and its log-sum-exp combine against the pages' own form, written
here directly from the scores.
"""
import math

import numpy as np
import pytest

from oracle import attention, attention_split, combine, split_partials
from synthetic.inputs import make_problem


def _random_bounds(rng, n, s):
    cuts = np.sort(rng.integers(0, n + 1, size=s - 1)) if s > 1 else np.array([], dtype=int)
    return [0] + [int(c) for c in cuts] + [n]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("s", [1, 2, 3, 7, 16])
def test_split_equals_unsplit_random_partitions(causal, s):
    p = make_problem(dtype="f32", batch=3, lq=4, hq=6, hkv=2, dqk=8, dv=5,
                     kv_len=[11, 4, 9], seed=20 + s, causal=causal)
    rng = np.random.default_rng(s)
    bounds = [_random_bounds(rng, int(n), s) for n in p.lens]
    o, lse = attention(p.q, p.k, p.v, causal, p.scale)
    o2, lse2 = attention_split(p.q, p.k, p.v, causal, p.scale, bounds)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lse2))
    np.testing.assert_allclose(lse2[fin], lse[fin], rtol=0, atol=1e-13)


def test_split_with_more_splits_than_keys_and_empty_splits():
    p = make_problem(dtype="f32", batch=2, lq=1, hq=4, hkv=1, dqk=4, dv=3,
                     kv_len=[3, 2], seed=30)
    bounds = [[0, 0, 1, 1, 3, 3, 3], [0, 1, 1, 1, 2, 2, 2]]
    po, pl = split_partials(p.q, p.k, p.v, False, p.scale, bounds)
    assert po.shape == (6, 2, 1, 4, 3)
    assert np.all(np.isneginf(pl[0, 0])) and np.all(po[0, 0] == 0)   # request 0: [0, 0)
    assert np.all(np.isneginf(pl[5])) and np.all(po[5] == 0)         # both: empty tail
    o, lse = attention(p.q, p.k, p.v, False, p.scale)
    o2, lse2 = combine(po, pl)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def test_even_split_matches_cleave_split_shape():
    # Split(A:[m, k], dim=1) -> [s, m, k/s] (Cleave §4): with k = 256 and s = 4 the
    # partial value-product has shape [s, S_Q, D] and every part has k/s = 64 keys.
    p = make_problem(dtype="f32", batch=1, lq=1, hq=8, hkv=2, dqk=64, dv=64, kv_len=256, seed=0)
    bounds = [[0, 64, 128, 192, 256]]
    po, pl = split_partials(p.q, p.k, p.v, False, p.scale, bounds)
    assert po.shape == (4, 1, 1, 8, 64) and pl.shape == (4, 1, 1, 8)
    o, _ = attention(p.q, p.k, p.v, False, p.scale)
    np.testing.assert_allclose(combine(po, pl)[0], o, rtol=0, atol=1e-13)


def test_lse_combine_equals_rowsum_valueproduct_form():
    # Cleave §4: each split emits an unnormalised row sum l_j = sum exp(S - c) and a
    # value-product U_j = sum exp(S - c) V, for one common reference c; the combine
    # sums both over s and divides.  Compute that form straight from the scores.
    rng = np.random.default_rng(40)
    n, d, dv, s = 37, 6, 4, 5
    q = rng.standard_normal(d)
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, dv))
    tau = 0.6
    scores = tau * (k @ q)
    c = 0.0
    bounds = [0, 3, 10, 10, 30, 37]
    l_parts = [math.fsum(math.exp(x - c) for x in scores[a:b]) for a, b in zip(bounds, bounds[1:])]
    u_parts = [np.array([math.fsum(math.exp(scores[j] - c) * v[j, t] for j in range(a, b))
                         for t in range(dv)]) for a, b in zip(bounds, bounds[1:])]
    want = sum(u_parts) / sum(l_parts)
    po, pl = split_partials(q[None, None, None, :], [k[:, None, :]], [v[:, None, :]], False, tau,
                            [bounds])
    o, lse = combine(po, pl)
    np.testing.assert_allclose(o[0, 0, 0], want, rtol=0, atol=1e-13)
    assert abs(lse[0, 0, 0] - (c + math.log(sum(l_parts)))) <= 1e-13


def test_combine_all_empty_rows():
    po = np.zeros((3, 1, 1, 2, 4))
    pl = np.full((3, 1, 1, 2), -np.inf)
    o, lse = combine(po, pl)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_combine_is_order_independent_and_extreme_lse_safe():
    rng = np.random.default_rng(41)
    po = rng.standard_normal((4, 2, 1, 3, 5))
    pl = rng.standard_normal((4, 2, 1, 3)) * 300.0      # would overflow a naive exp
    o, lse = combine(po, pl)
    perm = [2, 0, 3, 1]
    o2, lse2 = combine(po[perm], pl[perm])
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(o))


def test_split_rejects_bad_bounds():
    p = make_problem(dtype="f32", batch=1, lq=1, hq=2, hkv=1, dqk=4, dv=3, kv_len=5, seed=1)
    for bad in ([0, 3, 2, 5], [1, 5], [0, 4]):
        with pytest.raises(ValueError):
            split_partials(p.q, p.k, p.v, False, p.scale, [bad])
