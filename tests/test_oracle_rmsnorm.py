"""Pins of the RMSNorm + MatMul oracle (CPU only).

The oracle is checked against things other than itself: the pure-Python brute
force (an independent writing of the definition with exactly rounded sums),
closed forms (identity weights give the normalised rows, whose mean square is
known; a constant row normalises to +-1; without eps the result does not
depend on the input's scale), and the Split-K identity of the rewritten graph
(Cleave §1 / Fig. 1 and §2.2 "Split-K") against the same brute force.  Planted
mistakes in a copy of the oracle must each fail one of these pins.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import (RMS_EPS, brute_rmsnorm_matmul, rmsnorm_matmul, rmsnorm_matmul_split)

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "rmsnorm_matmul.py")


def _tiny(seed, m=3, k=7, n=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((m, k)), 1.0 + 0.3 * rng.standard_normal(k),
            rng.standard_normal((n, k)))


def _bounds(k):
    return [[0, k], [0, 3, k], [0, 1, 1, 4, k], [0, 0, k - 1, k]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_definition_matches_brute_force(seed):
    x, g, w = _tiny(seed)
    want = np.array(brute_rmsnorm_matmul(x.tolist(), g.tolist(), w.tolist(), RMS_EPS))
    np.testing.assert_allclose(rmsnorm_matmul(x, g, w), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_split_rewrite_matches_brute_force(seed):
    # The rewritten graph (Matmul on the raw input, sums of squares alongside,
    # row scale last), split over K in several ways, equals the definition.
    x, g, w = _tiny(seed, m=4, k=9, n=6)
    want = np.array(brute_rmsnorm_matmul(x.tolist(), g.tolist(), w.tolist(), RMS_EPS))
    for b in _bounds(9):
        np.testing.assert_allclose(rmsnorm_matmul_split(x, g, w, b), want, rtol=0, atol=1e-12)


def test_identity_weights_give_normalised_rows():
    # W = I, g = 1: Y = x / sqrt(ms + eps), so mean(Y^2) = ms / (ms + eps) per row.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 16)) * np.array([[0.01], [1.0], [30.0], [1e-3]])
    y = rmsnorm_matmul(x, np.ones(16), np.eye(16))
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + RMS_EPS), rtol=1e-12)


def test_constant_row_normalises_to_its_sign():
    # A row of equal entries c has rms |c| (eps = 0): it normalises to sign(c),
    # so Y = sign(c) * (W g)^T.
    rng = np.random.default_rng(6)
    g = 1.0 + 0.5 * rng.standard_normal(8)
    w = rng.standard_normal((5, 8))
    x = np.array([[2.5] * 8, [-0.125] * 8])
    y = rmsnorm_matmul(x, g, w, eps=0.0)
    np.testing.assert_allclose(y[0], w @ g, rtol=1e-13)
    np.testing.assert_allclose(y[1], -(w @ g), rtol=1e-13)


def test_scale_invariance_without_eps():
    x, g, w = _tiny(7, m=3, k=11, n=4)
    np.testing.assert_allclose(rmsnorm_matmul(37.0 * x, g, w, eps=0.0),
                               rmsnorm_matmul(x, g, w, eps=0.0), rtol=1e-12)
    # With eps the scale matters: a tiny row is damped, not normalised.
    small = rmsnorm_matmul(1e-4 * x, g, w)
    assert np.all(np.abs(small) < 0.05 * np.abs(rmsnorm_matmul(x, g, w)).max())


def test_shapes_are_checked():
    x, g, w = _tiny(8)
    with pytest.raises(ValueError):
        rmsnorm_matmul(x, g[:-1], w)
    with pytest.raises(ValueError):
        rmsnorm_matmul_split(x, g, w, [0, 2, 1, x.shape[1]])


# ---------------------------------------------------------------- mutants

MUTANTS = {
    "eps_dropped": ("np.sqrt(mean_sq + eps)", "np.sqrt(mean_sq)"),
    "sum_not_mean": ("mean_sq = np.mean(x * x, axis=1, keepdims=True)",
                     "mean_sq = np.sum(x * x, axis=1, keepdims=True)"),
    "sqrt_dropped": ("x / np.sqrt(mean_sq + eps) * g[None, :]", "x / (mean_sq + eps) * g[None, :]"),
    "gain_dropped": ("x / np.sqrt(mean_sq + eps) * g[None, :]", "x / np.sqrt(mean_sq + eps)"),
    "mean_over_rows": ("mean_sq = np.mean(x * x, axis=1, keepdims=True)",
                       "mean_sq = np.mean(x * x, axis=0, keepdims=True)"),
    "weights_not_transposed": ("return np.matmul(rmsnorm(x, g, eps), w.T)",
                               "return np.matmul(rmsnorm(x, g, eps), w[:, ::-1].T)"),
    "partial_gain_dropped": ("xg = x * g[None, :]", "xg = x"),
    "partial_range_shifted": ("u.append(np.matmul(xg[:, lo:hi], w[:, lo:hi].T))",
                              "u.append(np.matmul(xg[:, lo:hi], w[:, lo + 1:hi + 1].T))"),
    "ssq_not_squared": ("ssq.append(np.sum(x[:, lo:hi] ** 2, axis=1))",
                        "ssq.append(np.sum(np.abs(x[:, lo:hi]), axis=1))"),
    "combine_divides_by_parts": ("return u / np.sqrt(ssq / k + eps)[:, None]",
                                 "return u / np.sqrt(ssq / len(ssq_parts) + eps)[:, None]"),
    "combine_scale_dropped": ("return u / np.sqrt(ssq / k + eps)[:, None]", "return u"),
}


def _load(name=None):
    src = open(SRC_PATH).read()
    if name is not None:
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        src = src.replace(old, new)
    mod = types.ModuleType(f"rms_oracle_{name}")
    exec(compile(src, f"<rms {name}>", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    try:
        for seed in (11, 12):
            x, g, w = _tiny(seed, m=3, k=8, n=4)
            want = np.array(brute_rmsnorm_matmul(x.tolist(), g.tolist(), w.tolist(), RMS_EPS))
            if not np.allclose(mod.rmsnorm_matmul(x, g, w), want, rtol=0, atol=1e-12):
                return False
            for b in _bounds(8):
                if not np.allclose(mod.rmsnorm_matmul_split(x, g, w, b), want, rtol=0,
                                   atol=1e-12):
                    return False
    except (ValueError, IndexError, AssertionError, FloatingPointError):
        return False
    return True


def test_unmutated_copy_passes_pins():
    assert _pins_pass(_load())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_load(name)), f"pins did not catch mutant {name}"


def test_brute_force_is_the_textbook_formula():
    # One hand-computed case: x = [3, 4], g = [1, 2], eps = 0: rms = sqrt(12.5).
    y = brute_rmsnorm_matmul([[3.0, 4.0]], [1.0, 2.0], [[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]], 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(y[0], [3 / r, 8 / r, 11 / r], rtol=1e-15)
