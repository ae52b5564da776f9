"""Pins of the oracle's N -> N' reshard of a flat buffer ("Infra: Data
Parallel", section "Checkpoint：让各张卡保存自己的分片": a sharded checkpoint
can be loaded into a different number of ranks).

* A hand-worked case (10 elements, 4 -> 3 ranks).
* Resharding the shards of the pack oracle's FlatParameter for N ranks gives
  the pack oracle's shards for N' ranks (pack is pinned against numpy).
* N -> N' -> N is the identity; N' = N is the identity; a per-rank call is
  the slice of the all-ranks call.
* The old shards' padding is never read (it may hold anything), and bit
  patterns (NaN payloads, -0) survive, for 2- and 4-byte elements.
"""

import math

import numpy as np
import pytest

import oracle


def _shards(flat, world):
    S = flat.size // world
    return [flat[q * S:(q + 1) * S].copy() for q in range(world)]


def test_hand_worked_case():
    flat = np.concatenate([np.arange(1, 11, dtype=np.float32), np.full(2, 7.0, np.float32)])  # padding garbage
    old = _shards(flat, 4)                                   # S = 3
    got = oracle.reshard(old, 10, 3)                         # S' = 4, P' = 12
    assert got.tolist() == [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 0, 0]
    assert oracle.reshard(old, 10, 3, new_rank=2).tolist() == [9, 10, 0, 0]
    assert oracle.reshard(old, 10, 1).tolist() == list(range(1, 11))


@pytest.mark.parametrize("seed", range(12))
def test_reshard_matches_pack_for_the_new_world(seed):
    r = np.random.default_rng(seed)
    shapes = [tuple(int(d) for d in r.integers(1, 9, size=int(r.integers(0, 3)))) for _ in range(int(r.integers(1, 8)))]
    dtype = np.float32 if seed % 2 else np.uint16
    tensors = [r.integers(0, 2 ** 16, size=math.prod(s)).astype(dtype).reshape(s) for s in shapes]
    T = sum(math.prod(s) for s in shapes)
    N, N2 = int(r.choice([1, 2, 3, 8, 64])), int(r.choice([1, 2, 5, 8, 16]))
    old = _shards(oracle.pack(tensors, N), N)
    assert np.array_equal(oracle.reshard(old, T, N2).view(np.uint8), oracle.pack(tensors, N2).view(np.uint8))
    for q in sorted({0, N2 - 1, int(r.integers(0, N2))}):
        S2 = -(-T // N2)
        assert np.array_equal(oracle.reshard(old, T, N2, new_rank=q),
                              oracle.reshard(old, T, N2)[q * S2:(q + 1) * S2])


@pytest.mark.parametrize("N,N2", [(8, 3), (3, 8), (64, 1), (1, 64), (16, 16), (7, 5)])
def test_round_trip_and_identity(N, N2):
    r = np.random.default_rng(N * 100 + N2)
    T = 1000 + N * N2
    P = -(-T // N) * N
    flat = np.zeros(P, np.uint32).view(np.float32)
    flat.view(np.uint32)[:T] = r.integers(0, 2 ** 32, size=T, dtype=np.uint64).astype(np.uint32)
    flat.view(np.uint32)[0] = 0x7FC12345                     # NaN payload
    flat.view(np.uint32)[1] = 0x80000000                     # -0
    old = _shards(flat, N)
    mid = _shards(oracle.reshard(old, T, N2), N2)
    back = oracle.reshard(mid, T, N)
    assert np.array_equal(back.view(np.uint32), flat.view(np.uint32))
    same = oracle.reshard(old, T, N)
    assert np.array_equal(same.view(np.uint32), flat.view(np.uint32))


def test_old_padding_is_not_read():
    T, N = 10, 4
    flat = np.concatenate([np.arange(T, dtype=np.uint16), np.full(2, 0xBEEF, np.uint16)])
    for N2 in (3, 6, 12):
        out = oracle.reshard(_shards(flat, N), T, N2)
        assert not np.any(out[T:])
        assert np.array_equal(out[:T], flat[:T])
