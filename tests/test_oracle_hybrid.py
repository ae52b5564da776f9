"""Pins of the oracle's hybrid-sharding reduce ("PyTorch FSDP ..." section
3.3, sharding factor F; "4.1 数据并行详解", HYBRID_SHARD row and tip: a
reduce-scatter inside each group of F ranks, an all-reduce across the W/F
groups).

* F = W (full sharding) and F = 1 (replication) are the flat rank order, so
  they equal the flat reduce bit for bit.
* On dyadic data every operation is exact: the result is the exact mean
  over all W ranks, which is also the mean of the group means.
* A case where the two-level order and the flat order round differently
  pins the grouping itself (and that groups are consecutive ranks).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _bf16(vals):
    x = np.asarray(vals, np.float32)
    h = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(h), x)
    return h


def _random_rows(world, S, seed):
    r = np.random.default_rng(seed)
    x = r.normal(0, 1e-2, size=(world, S)).astype(np.float32)
    return [(x[q].view(np.uint32) >> 16).astype(np.uint16) for q in range(world)]


@pytest.mark.parametrize("world,S", [(8, 257), (16, 64), (2, 9), (1, 5)])
def test_extreme_factors_are_the_flat_order(world, S):
    rows = _random_rows(world, S, world)
    flat = oracle.reduce(rows, np.float32(1.0 / world))
    for group in (world, 1):
        assert np.array_equal(oracle.reduce_hybrid(rows, group, np.float32(1.0 / world)), flat)


@pytest.mark.parametrize("world,group,n_micro", [(16, 8, 1), (8, 2, 4), (64, 8, 2), (12, 4, 1)])
def test_dyadic_data_gives_the_exact_mean(world, group, n_micro):
    """Gradients k * 2^-6, |k| <= 64: every partial sum fits fp32 exactly;
    with W n a power of two the scale is exact too (W = 12 only checks
    the sum, scaled by 1)."""
    r = np.random.default_rng(world + group)
    S = 33
    k = r.integers(-64, 65, size=(n_micro, world, S))
    exact_scale = (world * n_micro) & (world * n_micro - 1) == 0
    scale = np.float32(1.0 / (world * n_micro)) if exact_scale else np.float32(1.0)
    div = world * n_micro if exact_scale else 1
    acc = np.zeros(S, np.float32)
    for m in range(n_micro):
        rows = [_bf16(k[m, q] * 2.0 ** -6) for q in range(world)]
        oracle.reduce_hybrid(rows, group, scale, acc, accumulate=m > 0)
    want = [Fraction(int(k[:, :, i].sum()), 64 * div) for i in range(S)]
    assert [Fraction(float(v)) for v in acc] == want
    # mean of the group means
    G = world // group
    means = [Fraction(int(k[:, g * group:(g + 1) * group, i].sum()), 64 * group * n_micro)
             for g in range(G) for i in range(S)]
    if exact_scale:
        for i in range(S):
            assert Fraction(float(acc[i])) == sum(means[g * S + i] for g in range(G)) / G


def test_two_level_order_is_pinned():
    """W = 4, F = 2, values 2^24, 1, 1, 1: the flat order adds each 1 to 2^24
    and rounds back to 2^24 (ties to even); the two-level order first forms
    the group sums 2^24 and 2, whose sum 2^24 + 2 is exact."""
    rows = [_bf16([2.0 ** 24]), _bf16([1.0]), _bf16([1.0]), _bf16([1.0])]
    assert oracle.reduce(rows, np.float32(1.0))[0] == 2.0 ** 24
    assert oracle.reduce_hybrid(rows, 2, np.float32(1.0))[0] == 2.0 ** 24 + 2
    # groups are consecutive ranks: pairing rank 0 with rank 2 would give 2^24 + 2 too,
    # so also check a case that separates the two pairings
    rows = [_bf16([2.0 ** 24]), _bf16([1.0]), _bf16([-(2.0 ** 24)]), _bf16([1.0])]
    # consecutive groups: (2^24 + 1) -> 2^24, (-2^24 + 1) exact; total 1
    assert oracle.reduce_hybrid(rows, 2, np.float32(1.0))[0] == 1.0
    # flat: 2^24 + 1 -> 2^24, - 2^24 -> 0, + 1 -> 1 (the same here); strided
    # groups (0, 2), (1, 3) would give 0 + 2 = 2
    assert oracle.reduce(rows, np.float32(1.0))[0] == 1.0


def test_overflow_in_one_group():
    rows = [np.full(4, 0x7F7F, np.uint16) for _ in range(4)]   # largest finite bf16
    acc = oracle.reduce_hybrid(rows, 2, np.float32(0.25))
    assert oracle.found_inf(acc) == 1


def test_signed_zero_survives_both_levels():
    """All gradients -0: each group sum starts from its first rank's value and
    the total from the first group's sum, so the result is -0, as in the flat
    order."""
    rows = [np.full(3, 0x8000, np.uint16) for _ in range(8)]
    acc = oracle.reduce_hybrid(rows, 4, np.float32(1 / 8))
    assert np.all(acc == 0) and np.all(np.signbit(acc))
