"""Pins of the SwiGLU oracle (CPU only).

Checked against things other than itself: the pure-Python brute force (an
independent writing with exactly rounded sums), closed forms (silu(0) = 0;
silu(z) - silu(-z) = z; silu(z) -> z for large z and -> 0 for very negative
z; a zero gate weight or a zero up weight gives zero), and the Split-K
identity (Cleave §2.2 "Split-K": parts of both MatMuls added before the gate)
against the same brute force.  Planted mistakes must each fail a pin.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import brute_swiglu, silu, swiglu, swiglu_split

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "swiglu.py")


def _tiny(seed, m=3, k=7, n=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((m, k)), rng.standard_normal((n, k)), rng.standard_normal((n, k)))


def _bounds(k):
    return [[0, k], [0, 3, k], [0, 1, 1, 4, k], [0, 0, k - 1, k]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_definition_matches_brute_force(seed):
    x, wg, wu = _tiny(seed)
    want = np.array(brute_swiglu(x.tolist(), wg.tolist(), wu.tolist()))
    np.testing.assert_allclose(swiglu(x, wg, wu), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [3, 4])
def test_split_matches_brute_force(seed):
    x, wg, wu = _tiny(seed, m=4, k=9, n=6)
    want = np.array(brute_swiglu(x.tolist(), wg.tolist(), wu.tolist()))
    for b in _bounds(9):
        np.testing.assert_allclose(swiglu_split(x, wg, wu, b), want, rtol=0, atol=1e-12)


def test_silu_closed_forms():
    z = np.array([-800.0, -30.0, -1.5, 0.0, 0.25, 2.0, 40.0, 700.0])
    s = silu(z)
    assert s[3] == 0.0
    np.testing.assert_allclose(s - silu(-z), z, rtol=1e-15, atol=1e-300)
    assert abs(s[-1] - 700.0) < 1e-12 and abs(s[0]) < 1e-300      # no overflow at the tails
    np.testing.assert_allclose(s[4], 0.25 / (1 + math.exp(-0.25)), rtol=1e-15)
    np.testing.assert_allclose(s[2], -1.5 / (1 + math.exp(1.5)), rtol=1e-15)


def test_zero_weights_give_zero():
    x, wg, wu = _tiny(5)
    assert np.all(swiglu(x, np.zeros_like(wg), wu) == 0)
    assert np.all(swiglu(x, wg, np.zeros_like(wu)) == 0)
    assert np.all(swiglu(np.zeros_like(x), wg, wu) == 0)


def test_gate_passes_large_positive_and_blocks_large_negative():
    # One input column; gate weight +-c with c large: silu(c x) ~ c x or ~0.
    x = np.array([[2.0]])
    wu = np.array([[3.0], [3.0]])
    wg = np.array([[50.0], [-50.0]])
    h = swiglu(x, wg, wu)
    np.testing.assert_allclose(h[0, 0], 100.0 * 6.0, rtol=1e-12)
    assert abs(h[0, 1]) < 1e-40


def test_shapes_are_checked():
    x, wg, wu = _tiny(6)
    with pytest.raises(ValueError):
        swiglu(x, wg, wu[:, :-1])
    with pytest.raises(ValueError):
        swiglu_split(x, wg, wu, [0, 4, 2, x.shape[1]])


MUTANTS = {
    "sigmoid_sign": ("sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))",
                     "sig = np.where(z >= 0, e / (1.0 + e), 1.0 / (1.0 + e))"),
    "gate_not_multiplied": ("return z * sig", "return sig"),
    "gate_on_up": ("return silu(np.matmul(x, wg.T)) * np.matmul(x, wu.T)",
                   "return np.matmul(x, wg.T) * silu(np.matmul(x, wu.T))"),
    "weights_swapped_in_parts": ("u.append(np.matmul(x[:, lo:hi], wu[:, lo:hi].T))",
                                 "u.append(np.matmul(x[:, lo:hi], wg[:, lo:hi].T))"),
    "part_range_shifted": ("g.append(np.matmul(x[:, lo:hi], wg[:, lo:hi].T))",
                           "g.append(np.matmul(x[:, lo:hi], wg[:, lo + 1:hi + 1].T))"),
    "gate_per_part": ("return silu(np.sum(g_parts, axis=0)) * np.sum(u_parts, axis=0)",
                      "return np.sum(silu(g_parts) * u_parts, axis=0)"),
    "up_untransposed": ("return silu(np.matmul(x, wg.T)) * np.matmul(x, wu.T)",
                        "return silu(np.matmul(x, wg.T)) * np.matmul(x, wu[::-1].T)"),
}


def _load(name=None):
    src = open(SRC_PATH).read()
    if name is not None:
        old, new = MUTANTS[name]
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        src = src.replace(old, new)
    mod = types.ModuleType(f"swiglu_oracle_{name}")
    exec(compile(src, f"<swiglu {name}>", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    try:
        for seed in (11, 12):
            x, wg, wu = _tiny(seed, m=3, k=8, n=4)
            want = np.array(brute_swiglu(x.tolist(), wg.tolist(), wu.tolist()))
            if not np.allclose(mod.swiglu(x, wg, wu), want, rtol=0, atol=1e-12):
                return False
            for b in _bounds(8):
                if not np.allclose(mod.swiglu_split(x, wg, wu, b), want, rtol=0, atol=1e-12):
                    return False
    except (ValueError, IndexError, AssertionError, FloatingPointError):
        return False
    return True


def test_unmutated_copy_passes_pins():
    assert _pins_pass(_load())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_load(name)), f"pins did not catch mutant {name}"
