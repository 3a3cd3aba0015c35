"""Planted mistakes in a copy of the oracle must be caught by its pins.

Each mutant is the oracle's source with one plausible slip (a dropped term, a
wrong sign or index, a misaligned mask, a missing normalisation) planted by
text substitution, loaded as a throw-away module on the CPU.  The pins used
here are the independent ones: the pure-Python brute force for the unsplit
result and LSE, and the split/combine identity checked against the same brute
force.  A mutant that no pin notices would mean the pins are too weak.
"""
import os
import types

import numpy as np
import pytest

from oracle import brute_attention

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")

MUTANTS = {
    "scale_dropped": ("s = scale * np.matmul(qg, kb.T)", "s = np.matmul(qg, kb.T)"),
    "gqa_interleaved_heads": ("heads = slice(kvh * g, (kvh + 1) * g)",
                              "heads = slice(kvh, hq, hkv)"),
    "causal_top_left": ("vis = vis & (j <= i + (n_keys - lq))", "vis = vis & (j <= i)"),
    "causal_off_by_one": ("vis = vis & (j <= i + (n_keys - lq))",
                          "vis = vis & (j < i + (n_keys - lq))"),
    "lse_without_log": ("m + np.log(safe_l)", "m + safe_l"),
    "lse_without_max": ("m + np.log(safe_l)", "np.log(safe_l)"),
    "division_dropped": ("p = e / safe_l[:, :, None]", "p = e"),
    "split_range_exclusive_lo": ("vis = (j >= lo) & (j < hi)", "vis = (j > lo) & (j < hi)"),
    "combine_weight_sign": ("np.exp(np.where(finite, lse_parts, 0.0) - m[None])",
                            "np.exp(m[None] - np.where(finite, lse_parts, 0.0))"),
    "combine_unweighted": ("o = (w[..., None] * o_parts).sum(axis=0) / safe[..., None]",
                           "o = o_parts.sum(axis=0) / o_parts.shape[0]"),
    "combine_lse_dropped_max": ("lse = np.where(any_f, m + np.log(safe), -np.inf)",
                                "lse = np.where(any_f, np.log(safe), -np.inf)"),
    "transposed_value_product": ("o = np.matmul(p, vb)",
                                 "o = np.matmul(p, vb[::-1])"),
}


def _load_mutant(name):
    src = open(SRC_PATH).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _cases():
    rng = np.random.default_rng(77)
    out = []
    for causal, g, hkv, lq, lens, d, dv in [(True, 2, 2, 3, [5, 2], 4, 3),
                                            (False, 2, 2, 1, [6, 4], 3, 2),
                                            (True, 1, 1, 4, [4], 3, 2)]:
        q = rng.standard_normal((len(lens), lq, g * hkv, d))
        k = [rng.standard_normal((n, hkv, d)) for n in lens]
        v = [rng.standard_normal((n, hkv, dv)) for n in lens]
        out.append((causal, q, k, v, dv, lens))
    return out


def _pins_pass(mod):
    """True if every pin holds for ``mod``; a raised error counts as a failure."""
    tau = 0.8
    try:
        for causal, q, k, v, dv, lens in _cases():
            bo, bl = brute_attention(q.tolist(), [x.tolist() for x in k],
                                     [x.tolist() for x in v], causal, tau, dv)
            bo = np.array(bo).reshape(q.shape[:3] + (dv,))
            bl = np.array(bl)
            o, lse = mod.attention(q, k, v, causal, tau)
            if not np.allclose(o, bo, rtol=0, atol=1e-12):
                return False
            if not np.array_equal(np.isfinite(lse), np.isfinite(bl)):
                return False
            fin = np.isfinite(bl)
            if not np.allclose(lse[fin], bl[fin], rtol=0, atol=1e-12):
                return False
            bounds = [[0, min(1, n), n // 2 if n > 1 else n, n] for n in lens]
            bounds = [[0] + sorted(b[1:-1]) + [b[-1]] for b in bounds]
            o2, lse2 = mod.attention_split(q, k, v, causal, tau, bounds)
            if not np.allclose(o2, bo, rtol=0, atol=1e-12):
                return False
            if not np.allclose(lse2[fin], bl[fin], rtol=0, atol=1e-12):
                return False
    except (AssertionError, ValueError, IndexError, FloatingPointError):
        return False
    return True


def test_unmutated_copy_passes_pins():
    src = open(SRC_PATH).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "<copy>", "exec"), mod.__dict__)
    assert _pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_load_mutant(name)), f"pins did not catch mutant {name}"
