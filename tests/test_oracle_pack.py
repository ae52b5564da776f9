"""Pins of the oracle's FlatParameter packing, geometry and views.

What fixes the expected values:
* the FSDP1 worked example of "Infra: Data Parallel" (golden fixture);
* numpy's concatenate / pad (a library routine) for brute force on tiny
  shapes;
* bit patterns that must survive a copy (NaN payloads, -0, subnormals);
* the view coverage property: over all ranks, every tensor element is
  seen exactly once, and reading a fragment from the shard returns the
  tensor's own elements.
"""

import math

import numpy as np
import pytest

import oracle
from conftest import load_golden
from workloads import CONFIGS, gen


def test_fsdp1_worked_example_shards():
    g = load_golden("fsdp1_three_4x2_two_ranks.json")
    names = g["names"]
    numel = [math.prod(s) for s in g["shapes"]]
    total, padded, shard = oracle.geometry(numel, g["world"])
    assert (total, shard) == (g["total"], g["shard"])
    assert padded == total  # 24 splits evenly over 2 ranks, no padding
    # distinct values so every element names its tensor and position
    tensors = [(np.arange(n, dtype=np.float32) + 100 * (i + 1)).reshape(s)
               for i, (n, s) in enumerate(zip(numel, g["shapes"]))]
    flat = oracle.pack(tensors, g["world"])
    for rank, pieces in g["shard_contents"].items():
        r = int(rank)
        expect = np.concatenate([tensors[names.index(nm)].reshape(-1)[a:b] for nm, a, b in pieces])
        np.testing.assert_array_equal(flat[r * shard:(r + 1) * shard], expect)


def test_fsdp1_worked_example_views():
    g = load_golden("fsdp1_three_4x2_two_ranks.json")
    names = g["names"]
    numel = [math.prod(s) for s in g["shapes"]]
    for rank, pieces in g["shard_contents"].items():
        bo, ln, to = oracle.views(numel, g["world"], int(rank))
        held = {nm: (a, b) for nm, a, b in pieces}
        for i, nm in enumerate(names):
            if nm in g["empty_views"][rank]:
                assert ln[i] == 0
            else:
                a, b = held[nm]
                assert (to[i], to[i] + ln[i]) == (a, b)
        # fragments laid end to end tile the shard in tensor order
        nonempty = [(bo[i], ln[i]) for i in range(len(names)) if ln[i] > 0]
        pos = 0
        for off, n in nonempty:
            assert off == pos
            pos += n
        assert pos == g["shard"]


@pytest.mark.parametrize("seed", range(40))
def test_pack_brute_force_against_concatenate(seed):
    r = np.random.default_rng(seed)
    world = int(r.choice([1, 2, 3, 4, 5, 7, 8, 16, 64]))
    n_t = int(r.integers(1, 9))
    shapes = [tuple(int(d) for d in r.integers(1, 6, size=int(r.integers(1, 4)))) for _ in range(n_t)]
    dtype = np.float32 if seed % 2 == 0 else np.uint16
    tensors = []
    for i, s in enumerate(shapes):
        x = gen.normal_f32(math.prod(s), 1.0, seed, gen.STREAM_TENSOR, i)
        tensors.append((x if dtype == np.float32 else gen.bf16_bits_trunc(x)).reshape(s))
    flat = oracle.pack(tensors, world)
    cat = np.concatenate([t.reshape(-1) for t in tensors])
    pad = (-cat.size) % world
    expect = np.pad(cat, (0, pad))
    assert flat.dtype == expect.dtype
    np.testing.assert_array_equal(flat.view(np.uint8), expect.view(np.uint8))
    t, p, s = oracle.geometry([x.size for x in tensors], world)
    assert (t, p, s) == (cat.size, cat.size + pad, (cat.size + pad) // world)
    assert 0 <= p - t < world


def test_pack_preserves_bit_patterns():
    pats = np.array([0x7FC00001, 0xFFC12345, 0x7F800001, 0x80000000, 0x00000001,
                     0x807FFFFF, 0x7F800000, 0xFF800000, 0x3F800000], dtype=np.uint32)
    a = pats.view(np.float32)
    b = np.array([1.0, 2.0], dtype=np.float32)
    flat = oracle.pack([a, b], 4)
    assert flat.size == 12
    np.testing.assert_array_equal(flat.view(np.uint32)[:9], pats)
    np.testing.assert_array_equal(flat.view(np.uint32)[11:], np.zeros(1, np.uint32))


@pytest.mark.parametrize("seed", range(25))
def test_views_cover_every_element_once(seed):
    r = np.random.default_rng(100 + seed)
    world = int(r.choice([1, 2, 3, 5, 8, 13]))
    numel = [int(x) for x in r.integers(1, 30, size=int(r.integers(1, 10)))]
    tensors = [np.arange(n, dtype=np.float32) + 1000 * (i + 1) for i, n in enumerate(numel)]
    flat = oracle.pack(tensors, world)
    _, _, S = oracle.geometry(numel, world)
    seen = [np.zeros(n, dtype=np.int32) for n in numel]
    for q in range(world):
        shard = flat[q * S:(q + 1) * S]
        bo, ln, to = oracle.views(numel, world, q)
        for i in range(len(numel)):
            if ln[i] == 0:
                continue
            np.testing.assert_array_equal(shard[bo[i]:bo[i] + ln[i]], tensors[i][to[i]:to[i] + ln[i]])
            seen[i][to[i]:to[i] + ln[i]] += 1
    for s in seen:
        np.testing.assert_array_equal(s, np.ones_like(s))
    bo, ln, to = oracle.views(numel, world, -1)
    for i in range(len(numel)):
        np.testing.assert_array_equal(flat[bo[i]:bo[i] + ln[i]], tensors[i])


@pytest.mark.parametrize("seed", range(10))
def test_locate_against_searchsorted(seed):
    r = np.random.default_rng(seed)
    numel = r.integers(1, 50, size=int(r.integers(1, 30)))
    world = int(r.integers(1, 9))
    _, p, _ = oracle.geometry(numel, world)
    pos = np.sort(r.integers(0, p, size=200))
    tensor, offset = oracle.locate_sorted(numel, pos)
    starts = np.concatenate([[0], np.cumsum(numel)])
    idx = np.searchsorted(starts, pos, side="right") - 1
    pad = idx >= len(numel)
    np.testing.assert_array_equal(tensor[~pad], idx[~pad])
    np.testing.assert_array_equal(offset[~pad], pos[~pad] - starts[idx[~pad]])
    assert np.all(tensor[pad] == -1)


def test_layer_unit_d1024_shard_boundaries():
    """Rank 1 and rank 7 of the eight-rank d=1024 layer unit.

    S = 12,596,224 / 8 = 1,574,528.  Rank 1 starts inside the qkv weight
    (3072 x 1024 = 3,145,728 elements), takes its rest, the qkv bias and the
    first 256 elements of the attention output weight; rank 7 ends with the
    second MLP weight's tail, its bias and the four LayerNorm vectors.
    """
    cfg = CONFIGS["c2_layer_d1024_nd8"]
    numel = [math.prod(s) for s in cfg.shapes]
    t, p, S = oracle.geometry(numel, 8)
    assert (t, p, S) == (12_596_224, 12_596_224, 1_574_528)
    bo, ln, to = oracle.views(numel, 8, 1)
    got = [(cfg.names[i], int(to[i]), int(to[i] + ln[i])) for i in range(len(numel)) if ln[i]]
    assert got == [("qkv.weight", 1_574_528, 3_145_728), ("qkv.bias", 0, 3072), ("out.weight", 0, 256)]
    bo, ln, to = oracle.views(numel, 8, 7)
    got = [(cfg.names[i], int(to[i]), int(to[i] + ln[i])) for i in range(len(numel)) if ln[i]]
    assert got == [("ff2.weight", 4_194_304 - 1_569_408, 4_194_304), ("ff2.bias", 0, 1024),
                   ("ln1.weight", 0, 1024), ("ln1.bias", 0, 1024),
                   ("ln2.weight", 0, 1024), ("ln2.bias", 0, 1024)]


def test_ragged_10k_geometry():
    cfg = CONFIGS["c5_ragged10k_nd64"]
    numel = [s[0] for s in cfg.shapes]
    t, p, S = oracle.geometry(numel, 64)
    assert t == 2_728_745_331
    assert p == 2_728_745_344 and S == 42_636_646
    bo, ln, to = oracle.views(numel, 64, 63)
    # the last rank holds the 13 padding elements after the last tensor's tail
    assert int(bo[-1] + ln[-1]) == S - 13
