"""Pins of the oracle's steps on either side of the reduce.

* Local accumulation without communication ("Infra: Data Parallel",
  section "Naive Data Parallelism", gradient-accumulation paragraph; "PyTorch
  FSDP ..." section 3.4): on dyadic data, where every operation is exact,
  accumulating n micro-batches locally, rounding once to bf16 and reducing
  with 1/(N n) must give the exact rational mean, and the same result as
  accumulating with communication; the fixed micro-batch order, the bf16
  rounding of the exchanged row and the propagation of inf are pinned by
  values worked out from the formats.
* The consumers of the overflow flag and of the gradient norm ("PyTorch FSDP
  ..." section 3.5, sharded gradient scaler; clipping is not on the pages):
  the loss-scale trajectory of the dynamic scaling rule for given overflow
  sequences, the unscale factor for power-of-two scales, the clipped norm as
  measured by numpy, and AdamW's use of the factor on the gradient.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads.configs import AdamW

HP = AdamW()


def _bf16_exact(vals):
    """bf16 patterns of values that bf16 represents exactly (checked)."""
    x = np.asarray(vals, np.float32)
    h = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f32(h), x), "value not exact in bf16"
    return h


# ------------------------------------------------------------------ no_sync
@pytest.mark.parametrize("world,n_micro,S", [(2, 4, 37), (4, 2, 64), (8, 4, 129), (1, 2, 5)])
def test_local_accumulation_gives_the_exact_mean(world, n_micro, S):
    """Dyadic gradients k * 2^-6 with |k| <= 64: the local sums of up to 4
    micro-batches need at most 8 significant bits, so the bf16 row is exact,
    and with N n a power of two the reduce is exact too."""
    r = np.random.default_rng(world * 100 + n_micro)
    k = r.integers(-64, 65, size=(n_micro, world, S))
    g = [[_bf16_exact(k[m, q] * 2.0 ** -6) for q in range(world)] for m in range(n_micro)]
    rows = []
    for q in range(world):
        local = None
        for m in range(n_micro - 1):
            local = oracle.local_accumulate(g[m][q], local, accumulate=m > 0)
        rows.append(oracle.local_finish(g[-1][q], local, accumulate=n_micro > 1))
    scale = np.float32(1.0 / (world * n_micro))
    got = oracle.reduce(rows, scale)
    want = [Fraction(int(k[:, :, i].sum()), 64 * world * n_micro) for i in range(S)]
    assert [Fraction(float(v)) for v in got] == want
    # the same as accumulating with communication, micro-batch by micro-batch
    acc = np.zeros(S, np.float32)
    for m in range(n_micro):
        oracle.reduce(g[m], scale, acc, accumulate=m > 0)
    assert np.array_equal(acc, got)


def test_one_micro_batch_passes_the_gradient_through():
    """n = 1: the exchanged row is the gradient itself, bit for bit, including
    -0, subnormals, infinities and NaN (which stays a NaN)."""
    h = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0xFF80, 0x7F80, 0x3F80, 0xC2F7], np.uint16)
    assert np.array_equal(oracle.local_finish(h), h)
    nan = oracle.local_finish(np.array([0x7FC1], np.uint16))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_exchanged_row_rounds_to_nearest_even():
    """bf16 keeps 8 significant bits: at 1.0 the spacing is 2^-7.  A local sum
    of 1 + 2^-8 is halfway and goes to the even neighbour 1.0; 1 + 3 * 2^-8
    goes to 1 + 2^-6; just above halfway goes up; the sign is symmetric."""
    local = np.array([1.0, 1.0, 1.0 + 2.0 ** -16, -1.0, 1.0], np.float32)
    add = np.array([2.0 ** -8, 3 * 2.0 ** -8, 2.0 ** -8, -(3 * 2.0 ** -8), 2.0 ** -9], np.float32)
    g = _bf16_exact(add)
    got = oracle.bf16_to_f32(oracle.local_finish(g, local, accumulate=True))
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -6), 1.0]


def test_micro_batches_are_added_in_order_in_fp32():
    """2^24 + 1 is not an fp32 value (it rounds to the even 2^24), so the sum
    2^24, 1, -2^24 in that order is 0, while any order that adds the two large
    terms first gives 1."""
    seq = [_bf16_exact([2.0 ** 24]), _bf16_exact([1.0]), _bf16_exact([-(2.0 ** 24)])]
    local = oracle.local_accumulate(seq[0])
    local = oracle.local_accumulate(seq[1], local, accumulate=True)
    out = oracle.local_finish(seq[2], local, accumulate=True)
    assert oracle.bf16_to_f32(out)[0] == 0.0
    local = oracle.local_accumulate(seq[0])
    local = oracle.local_accumulate(seq[2], local, accumulate=True)
    out = oracle.local_finish(seq[1], local, accumulate=True)
    assert oracle.bf16_to_f32(out)[0] == 1.0


def test_local_overflow_reaches_the_flag():
    """An inf in one micro-batch of one rank survives the local sum and the
    bf16 row, and the reduce's overflow check sees it; two finite maxima
    overflow fp32 only in the rank sum."""
    world, S = 4, 8
    g = [[np.zeros(S, np.uint16) for _ in range(world)] for _ in range(2)]
    g[0][2][5] = 0x7F80
    rows = [oracle.local_finish(g[1][q], oracle.local_accumulate(g[0][q]), accumulate=True)
            for q in range(world)]
    assert rows[2][5] == 0x7F80
    acc = oracle.reduce(rows, np.float32(1 / 8))
    assert oracle.found_inf(acc) == 1
    big = [np.full(S, 0x7F7F, np.uint16) for _ in range(2)]          # largest finite bf16
    rows = [oracle.local_finish(b) for b in big]
    assert oracle.found_inf(oracle.reduce(rows, np.float32(0.25))) == 1


# ------------------------------------------------------------------ scaler and clipping
def test_loss_scale_trajectory():
    """Dynamic loss scaling with growth interval 3: the scale doubles after
    every 3 clean steps in a row and halves on an overflow, which also
    restarts the count."""
    flags = [0, 0, 0, 0, 1, 0, 0, 1, 0, 0, 0, 0, 0, 0]
    want = [65536, 65536, 131072, 131072, 65536, 65536, 65536, 32768, 32768, 32768, 65536, 65536,
            65536, 131072]
    scale, clean, got = 65536.0, 0, []
    for f in flags:
        scale, clean = oracle.scaler_update(f, scale, clean, growth_interval=3)
        got.append(scale)
    assert got == want


def test_loss_scale_default_interval():
    scale, clean = 2.0 ** 16, 0
    for _ in range(1999):
        scale, clean = oracle.scaler_update(0, scale, clean)
    assert (scale, clean) == (2.0 ** 16, 1999)
    assert oracle.scaler_update(0, scale, clean) == (2.0 ** 17, 0)
    assert oracle.scaler_update(1, scale, clean) == (2.0 ** 15, 0)


@pytest.mark.parametrize("k", [0, 3, 16, 24])
def test_unscale_is_exact_for_power_of_two_scales(k):
    assert oracle.grad_coef(123.0, 2.0 ** k, 0.0) == 2.0 ** -k


@pytest.mark.parametrize("seed", range(6))
def test_clipped_norm(seed):
    """Multiplying the loss-scaled gradient by the factor gives an unscaled
    gradient whose norm (numpy's) is min(||g||, ~max_norm): unchanged below
    max_norm, max_norm * ||g|| / (||g|| + 1e-6) above it."""
    r = np.random.default_rng(seed)
    L = float(2.0 ** r.integers(0, 20))
    g = r.normal(0, 10.0 ** r.uniform(-3, 1), size=1000)
    scaled = (g * L).astype(np.float32)
    sq = float(np.sum(scaled.astype(np.float64) ** 2))
    true_norm = float(np.linalg.norm(scaled.astype(np.float64))) / L
    for max_norm in (0.5 * true_norm, 2.0 * true_norm):
        c = oracle.grad_coef(sq, L, max_norm)
        norm = float(np.linalg.norm(scaled.astype(np.float64) * c))
        if true_norm > max_norm:
            assert norm == pytest.approx(max_norm * true_norm / (true_norm + 1e-6), rel=1e-12)
            assert norm < max_norm
        else:
            assert norm == pytest.approx(true_norm, rel=1e-12)


def test_no_clipping_when_max_norm_is_zero():
    assert oracle.grad_coef(1e30, 1.0, 0.0) == 1.0
    assert oracle.grad_coef(0.0, 1.0, 1.0) == 1.0


def test_adamw_applies_the_factor_to_the_gradient():
    """AdamW of a gradient scaled by a power of two with the inverse factor is
    AdamW of the gradient itself, bit for bit; a factor of 0 leaves only the
    decoupled decay, theta (1 - lr wd), with fresh moments staying 0."""
    r = np.random.default_rng(3)
    S = 257
    g = r.normal(0, 1e-3, S).astype(np.float32)
    th = r.normal(0, 0.02, S).astype(np.float32)
    kw = dict(lr=HP.lr, beta1=HP.beta1, beta2=HP.beta2, eps=HP.eps, weight_decay=HP.weight_decay, step=1)
    a = [th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)]
    oracle.adamw(g, *a, **kw)
    b = [th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)]
    oracle.adamw((g * np.float32(1024.0)).astype(np.float32), *b, coef=1.0 / 1024.0, **kw)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    z = [th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)]
    oracle.adamw(g, *z, coef=0.0, **kw)
    assert np.array_equal(z[0], (th.astype(np.float64) * (1.0 - HP.lr * HP.weight_decay)).astype(np.float32))
    assert not z[1].any() and not z[2].any()
    with_one = [th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)]
    oracle.adamw(g, *with_one, coef=1.0, **kw)
    for x, y in zip(a, with_one):
        assert np.array_equal(x, y)
    assert math.isfinite(float(z[0][0]))
