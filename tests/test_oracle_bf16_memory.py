"""Pins of the oracle's bf16 rounding, unshard copy and model-state memory model.

* bf16 rounding is checked against torch's CPU float32 -> bfloat16
  conversion (a library round-to-nearest-even) over every sign, exponent
  and upper mantissa with each class of dropped bits (below, at and above
  one half, both parities); the full 2^32 sweep runs with FP_SLOW_TESTS=1.
* unshard is checked against numpy concatenation.
* the memory model is checked against the numbers "4.1 数据并行详解"
  prints for a 7B model on 8 GPUs (sections 4.3, 6.1, 7) and against the
  per-GPU formulas of the ZeRO figure in "Infra: Data Parallel".
"""

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden
from workloads import gen


def _torch_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _same_or_both_nan(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    nan_a = (a & 0x7F80 == 0x7F80) & (a & 0x007F != 0)
    nan_b = (b & 0x7F80 == 0x7F80) & (b & 0x007F != 0)
    return (a == b) | (nan_a & nan_b)


def test_bf16_rounding_every_upper_half_and_rounding_class():
    upper = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lowers = [0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF]
    lowers += [int(x) for x in gen.rng(0, 99).integers(0, 1 << 16, size=8)]
    for lo in lowers:
        x = (upper | np.uint32(lo)).view(np.float32)
        got = oracle.f32_to_bf16(x)
        assert np.all(_same_or_both_nan(got, _torch_bf16(x))), hex(lo)
    # NaN in, NaN out (quiet), sign kept
    nans = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0xFFFFFFFF], dtype=np.uint32).view(np.float32)
    h = oracle.f32_to_bf16(nans)
    assert np.all((h & 0x7F80) == 0x7F80) and np.all(h & 0x0040)
    np.testing.assert_array_equal(h >> 15, np.array([0, 1, 0, 1], np.uint16))


@pytest.mark.slow
def test_bf16_rounding_exhaustive():
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        x = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        assert np.all(_same_or_both_nan(oracle.f32_to_bf16(x), _torch_bf16(x))), start


def test_bf16_widening_round_trip():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    back = oracle.f32_to_bf16(oracle.bf16_to_f32(h))
    assert np.all(_same_or_both_nan(back, h))
    np.testing.assert_array_equal(oracle.bf16_to_f32(h).view(np.uint32), h.astype(np.uint32) << 16)


@pytest.mark.parametrize("world,S", [(1, 5), (2, 12), (3, 7), (8, 33), (64, 3)])
def test_unshard_is_concatenation_in_rank_order(world, S):
    shards = [gen.bf16_normal(S, 1.0, 6, gen.STREAM_SHARD, q) for q in range(world)]
    full = oracle.unshard(shards)
    np.testing.assert_array_equal(full, np.concatenate(shards))
    for q in range(world):
        np.testing.assert_array_equal(full[q * S:(q + 1) * S], shards[q])


def test_memory_model_7b_on_8_gpus():
    g = load_golden("zero_memory_7b_n8.json")
    psi, n, k = g["psi"], g["world"], g["k"]
    gb = lambda stage: oracle.state_bytes(psi, n, k, stage) / 1e9  # noqa: E731
    assert gb(0) == pytest.approx(g["ddp_gb"], rel=1e-12)
    assert abs(gb(2) - g["zero2_gb_approx"]) <= g["zero2_gb_tolerance"]
    assert gb(3) == pytest.approx(g["zero3_gb"], rel=1e-12)
    assert oracle.state_bytes(psi, 1, k, 0) / psi == g["bytes_per_param_replicated"]
    assert k * psi / oracle.state_bytes(psi, n, k, 0) == pytest.approx(g["optimizer_share_of_total"])


def test_memory_model_structure():
    psi, k = 1e9, 12
    for n in (2, 4, 8, 64):
        vals = [oracle.state_bytes(psi, n, k, s) for s in range(4)]
        assert vals[0] > vals[1] > vals[2] > vals[3]          # each stage shards more
        # stage 3 shards everything; stage 0 nothing
        assert vals[3] * n == pytest.approx(vals[0])
    for s in range(4):  # one GPU: nothing to shard
        assert oracle.state_bytes(psi, 1, k, s) == pytest.approx(16 * psi)
    assert oracle.state_bytes(psi, 8, k, 7) == -1.0
