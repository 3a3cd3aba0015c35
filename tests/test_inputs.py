"""The seeded input generator: determinism, bf16 exactness, lengths, draw order."""
import math

import numpy as np
import pytest

from synthetic.inputs import WORKLOADS, make_problem, padded, to_bf16_exact, workload


def test_seeded_and_deterministic():
    a = make_problem(dtype="bf16", batch=2, lq=3, hq=4, hkv=2, dqk=8, dv=8, kv_len=(4, 40), seed=5)
    b = make_problem(dtype="bf16", batch=2, lq=3, hq=4, hkv=2, dqk=8, dv=8, kv_len=(4, 40), seed=5)
    c = make_problem(dtype="bf16", batch=2, lq=3, hq=4, hkv=2, dqk=8, dv=8, kv_len=(4, 40), seed=6)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.lens, b.lens)
    assert all(np.array_equal(x, y) for x, y in zip(a.k, b.k))
    assert not np.array_equal(a.q, c.q)


def test_bf16_values_are_exact_bf16():
    p = make_problem(dtype="bf16", batch=1, lq=2, hq=2, hkv=1, dqk=16, dv=16, kv_len=9, seed=1)
    bits = p.q.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    assert np.array_equal(to_bf16_exact(p.q), p.q)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert list(to_bf16_exact(x)) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7]


def test_log_uniform_lengths_range_and_spread():
    p = make_problem(dtype="bf16", batch=2000, lq=1, hq=1, hkv=1, dqk=1, dv=1,
                     kv_len=(128, 32768), lcap=32768, seed=0)
    assert p.lens.min() >= 128 and p.lens.max() <= 32768
    logs = np.log(p.lens)
    # log-uniform: the mean of ln L is (ln 128 + ln 32768) / 2 to within sampling error.
    assert abs(logs.mean() - (math.log(128) + math.log(32768)) / 2) < 0.15


def test_draw_order_lengths_then_q_then_k_then_v():
    p = make_problem(dtype="f32", batch=2, lq=1, hq=2, hkv=1, dqk=3, dv=2, kv_len=[2, 1], seed=9)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 1, 2, 3), dtype=np.float32)
    k0 = rng.standard_normal((2, 1, 3), dtype=np.float32)
    k1 = rng.standard_normal((1, 1, 3), dtype=np.float32)
    v0 = rng.standard_normal((2, 1, 2), dtype=np.float32)
    assert np.array_equal(p.q, q) and np.array_equal(p.k[0], k0)
    assert np.array_equal(p.k[1], k1) and np.array_equal(p.v[0], v0)


def test_padding_is_nan_past_valid_rows():
    p = make_problem(dtype="bf16", batch=2, lq=1, hq=2, hkv=1, dqk=4, dv=4, kv_len=[3, 5],
                     lcap=8, seed=2)
    k = padded(p.k, p.lcap)
    assert k.shape == (2, 8, 1, 4)
    assert np.all(np.isnan(k[0, 3:])) and not np.any(np.isnan(k[0, :3]))
    assert np.all(np.isnan(k[1, 5:]))
    kz = padded(p.k, p.lcap, pad=0.0)
    assert np.all(kz[0, 3:] == 0)


def test_workload_table_shapes():
    assert set(WORKLOADS) == {"tiny_gqa_decode_f32", "llama3_8b_gqa_decode", "gqa_causal_prefill",
                              "ragged_decode_qwen3_32b", "mla_decode"}
    p = workload("tiny_gqa_decode_f32")
    assert p.q.shape == (1, 1, 8, 64) and p.k[0].shape == (256, 2, 64) and p.s == 4
    assert p.dtype == "f32" and abs(p.scale - 1 / 8) < 1e-15


def test_rejects_length_over_capacity():
    with pytest.raises(ValueError):
        make_problem(dtype="f32", batch=1, lq=1, hq=1, hkv=1, dqk=2, dv=2, kv_len=[9], lcap=8)
