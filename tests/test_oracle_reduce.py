"""Pins of the oracle's reduce-scatter arithmetic.

What fixes the expected values:
* the data-parallel identity of "4.1 数据并行详解" section 2 (the mean of
  the N local mean gradients equals the global-batch gradient), checked
  exactly with rational arithmetic on dyadic data where every float
  operation is exact;
* the micro-batch rule of "Infra: Data Parallel" (Naive DP section): n
  equal micro-batches with each loss divided by n give the full-batch
  gradient, again exact on dyadic data;
* the textbook error bound of recursive summation (Higham, Accuracy and
  Stability of Numerical Algorithms, eq. 4.4) on random data, against
  the exact rational result;
* cases whose answer is fixed by IEEE-754 alone (summation order, signed
  zero, overflow, inf - inf);
* the all-reduce = reduce-scatter + all-gather identity of "4.1 数据并行详解"
  section 5.1.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import gen

U32 = 2.0 ** -24


def _bf16_exact(values):
    """bf16 patterns of float32 values that are exactly representable in bf16."""
    x = np.asarray(values, dtype=np.float32)
    h = gen.bf16_bits_trunc(x)
    assert np.array_equal(oracle.bf16_to_f32(h), x), "value not representable in bf16"
    return h


def _frac(x):
    return Fraction(float(x))


@pytest.mark.parametrize("world", [1, 2, 4, 8, 16, 64])
def test_data_parallel_mean_equals_global_batch_gradient(world):
    b, S = 4, 257
    r = np.random.default_rng(world)
    # per-sample gradients: integers in [-8, 8] times 2^-4 (dyadic, tiny)
    per_sample = r.integers(-8, 9, size=(world, b, S)) / 16.0
    local = per_sample.mean(axis=1)             # each rank's local mean, exact
    grads = [_bf16_exact(local[q]) for q in range(world)]
    acc = oracle.reduce(grads, np.float32(1.0 / world))
    for i in range(0, S, 16):
        exact = sum(Fraction(int(round(v * 16)), 16) for v in per_sample[:, :, i].reshape(-1)) / (world * b)
        assert _frac(acc[i]) == exact


def test_micro_batches_each_divided_by_n_give_full_batch_gradient():
    world, n, b, S = 8, 4, 2, 129
    r = np.random.default_rng(7)
    per_sample = r.integers(-8, 9, size=(n, world, b, S)) / 16.0
    acc = np.full(S, np.nan, dtype=np.float32)
    scale = np.float32(1.0 / (world * n))
    for m in range(n):
        grads = [_bf16_exact(per_sample[m, q].mean(axis=0)) for q in range(world)]
        oracle.reduce(grads, scale, acc, accumulate=m > 0)
    for i in range(S):
        exact = sum(Fraction(int(round(v * 16)), 16) for v in per_sample[..., i].reshape(-1)) / (n * world * b)
        assert _frac(acc[i]) == exact


def test_summation_runs_in_ascending_rank_order():
    # 2^24 + 1 rounds back to 2^24 (tie to even): the order of the terms decides.
    big, one = 2.0 ** 24, 1.0
    acc = oracle.reduce([_bf16_exact([big]), _bf16_exact([one]), _bf16_exact([one])], 1.0)
    assert acc[0] == np.float32(big)
    acc = oracle.reduce([_bf16_exact([one]), _bf16_exact([one]), _bf16_exact([big])], 1.0)
    assert acc[0] == np.float32(big + 2)


def test_sum_starts_from_rank_zero_value():
    neg_zero = np.array([0x8000], dtype=np.uint16)
    acc = oracle.reduce([neg_zero] * 5, np.float32(0.2))
    assert acc.view(np.uint32)[0] == 0x80000000  # -0 stays -0
    acc = oracle.reduce([neg_zero, np.array([0], np.uint16)], np.float32(0.5))
    assert acc.view(np.uint32)[0] == 0  # -0 + +0 = +0


@pytest.mark.parametrize("world", [2, 8, 16, 64])
def test_equal_gradients_average_to_themselves(world):
    g = gen.bf16_normal(300, 1e-3, 3, gen.STREAM_GRAD, world)
    acc = oracle.reduce([g] * world, np.float32(1.0 / world))
    np.testing.assert_array_equal(acc, oracle.bf16_to_f32(g))


def test_single_rank_is_a_widening_copy():
    g = gen.bf16_normal(1000, 1.0, 4, gen.STREAM_GRAD)
    np.testing.assert_array_equal(oracle.reduce([g], 1.0), oracle.bf16_to_f32(g))


@pytest.mark.parametrize("world,n", [(3, 1), (8, 1), (16, 4), (64, 1), (5, 3)])
def test_error_within_recursive_summation_bound(world, n):
    S = 64
    acc = np.zeros(S, dtype=np.float32)
    scale = np.float32(1.0 / (world * n))
    exact = [Fraction(0)] * S
    bound = [0.0] * S
    gamma = (world - 1) * U32 / (1 - (world - 1) * U32)
    for m in range(n):
        grads = [gen.bf16_normal(S, 1.0, 11, gen.STREAM_GRAD, 0, m, q) for q in range(world)]
        oracle.reduce(grads, scale, acc, accumulate=m > 0)
        vals = np.stack([oracle.bf16_to_f32(g) for g in grads])
        for i in range(S):
            s = sum(_frac(v) for v in vals[:, i])
            abs_sum = float(np.abs(vals[:, i].astype(np.float64)).sum())
            y = s * _frac(scale)
            # sum error, then one rounding for the scale, one for the accumulate
            e = float(scale) * (gamma * abs_sum * (1 + U32)) + U32 * (abs(float(y)) + float(scale) * gamma * abs_sum)
            exact[i] = exact[i] + y if m > 0 else y
            bound[i] = (bound[i] + e if m > 0 else e) + (U32 * abs(float(acc[i])) if m > 0 else 0.0)
    for i in range(S):
        assert abs(float(_frac(acc[i]) - exact[i])) <= bound[i] * 1.0000001


def test_matches_independent_float32_loop():
    world, S = 7, 500
    grads = [gen.bf16_normal(S, 1e-3, 5, gen.STREAM_GRAD, q) for q in range(world)]
    acc0 = gen.normal_f32(S, 1e-4, 5, gen.STREAM_EXP_AVG)
    scale = np.float32(1.0 / 28)
    got = oracle.reduce(grads, scale, acc0.copy(), accumulate=True)
    vals = [oracle.bf16_to_f32(g) for g in grads]
    s = vals[0].copy()
    for q in range(1, world):
        s = (s + vals[q]).astype(np.float32)
    want = (acc0 + (s * scale).astype(np.float32)).astype(np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_overflow_and_nonfinite_set_the_flag():
    fin = _bf16_exact([1.0, -2.0, 0.5])
    assert oracle.found_inf(oracle.reduce([fin, fin], 0.5)) == 0
    pinf, ninf, nan = np.uint16(0x7F80), np.uint16(0xFF80), np.uint16(0x7FC0)
    a = fin.copy()
    a[1] = pinf
    acc = oracle.reduce([a, fin], 0.5)
    assert np.isposinf(acc[1]) and oracle.found_inf(acc) == 1
    b = fin.copy()
    b[1] = ninf
    acc = oracle.reduce([a, b], 0.5)
    assert np.isnan(acc[1]) and oracle.found_inf(acc) == 1
    c = fin.copy()
    c[2] = nan
    assert oracle.found_inf(oracle.reduce([fin, c], 0.5)) == 1
    big = np.array([0x7F7F], dtype=np.uint16)  # largest finite bf16, about 3.39e38
    acc = oracle.reduce([big, big], 0.5)
    assert np.isposinf(acc[0]) and oracle.found_inf(acc) == 1  # the fp32 sum overflows first


def test_nonfinite_survives_later_micro_batches():
    fin = _bf16_exact([1.0, 1.0])
    a = fin.copy()
    a[0] = np.uint16(0x7F80)
    acc = oracle.reduce([a, fin], 0.25)
    oracle.reduce([fin, fin], 0.25, acc, accumulate=True)
    assert oracle.found_inf(acc) == 1


def test_sq_norm_exact_on_dyadic_and_bounded_on_random():
    vals = (np.arange(-50, 51) / 64.0).astype(np.float32)
    exact = sum(_frac(v) ** 2 for v in vals)
    assert Fraction(oracle.sq_norm(vals)) == exact
    x = gen.normal_f32(5000, 1e-3, 9, gen.STREAM_GRAD)
    exact = sum(_frac(v) ** 2 for v in x)
    err = abs(Fraction(oracle.sq_norm(x)) - exact)
    assert float(err) <= 5000 * 2.0 ** -53 * float(exact)


@pytest.mark.parametrize("world", [2, 3, 8])
def test_allreduce_equals_reduce_scatter_then_allgather(world):
    S = 37
    full = [gen.bf16_normal(world * S, 1.0, 13, gen.STREAM_GRAD, q) for q in range(world)]
    whole = oracle.reduce(full, np.float32(1.0 / world))
    pieces = [oracle.reduce([g[r * S:(r + 1) * S].copy() for g in full], np.float32(1.0 / world))
              for r in range(world)]
    np.testing.assert_array_equal(np.concatenate(pieces).view(np.uint32), whole.view(np.uint32))
