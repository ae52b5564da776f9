"""Pins of the oracle's per-parameter dim-0 sharding (the FSDP2 layout).

What fixes the expected values:
* the FSDP2 figure and the (8, 4) example of "Infra: Data Parallel"
  (golden fixture: which rows each rank keeps, local shapes, elements per
  rank);
* torch.chunk along dim 0 (a library routine) for uneven splits, with each
  rank's chunk zero-padded to the common chunk size -- the reading taken
  where the pages show only even splits;
* the round trip: gathering every rank's buffer and unpacking returns the
  parameters bit for bit (NaN payloads and -0 included);
* the contrast the figure draws with FSDP1: the flat split cuts through W2,
  the per-parameter split cuts every weight.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden
from workloads import gen


def _distinct(shapes, dtype=np.float32):
    return [(np.arange(math.prod(s), dtype=np.float32) + 1000 * (i + 1)).astype(dtype).reshape(s)
            for i, s in enumerate(shapes)]


@pytest.mark.parametrize("k", [0, 1])
def test_page_examples(k):
    ex = load_golden("fsdp2_dim0_examples.json")["examples"][k]
    shapes = [tuple(s) for s in ex["shapes"]]
    world = ex["world"]
    c, r, off, S = oracle.shard0_geometry(shapes, world)
    assert S == ex["elements_per_rank"]
    for ci, ri in zip(c, r):
        assert (ci, ri) == tuple(ex["local_shape"])       # local (rows, row length)
    ws = _distinct(shapes)
    for q, (a, b) in ex["rows_of_rank"].items():
        buf = oracle.shard0_pack(ws, world, int(q))
        expect = np.concatenate([w[a:b].reshape(-1) for w in ws])
        np.testing.assert_array_equal(buf, expect)


def test_contrast_with_the_flat_split():
    ex = load_golden("fsdp2_dim0_examples.json")["examples"][0]
    shapes = [tuple(s) for s in ex["shapes"]]
    ws = _distinct(shapes)
    flat = oracle.pack(ws, 2)
    per_param = oracle.shard0_pack(ws, 2, 0)
    # FSDP1 rank 0: W1 whole + half of W2; FSDP2 rank 0: two rows of each weight
    np.testing.assert_array_equal(flat[:12], np.concatenate([ws[0].reshape(-1), ws[1].reshape(-1)[:4]]))
    np.testing.assert_array_equal(per_param, np.concatenate([w[:2].reshape(-1) for w in ws]))
    assert not np.array_equal(flat[:12], per_param)


def _torch_chunk_buffer(ws, world, q):
    """Rank q's buffer from torch.chunk along dim 0, each chunk padded with
    zero rows to the common chunk size ceil(d0 / world)."""
    parts = []
    for w in ws:
        t = torch.from_numpy(np.ascontiguousarray(w)) if w.ndim else torch.from_numpy(w.reshape(1))
        d0 = t.shape[0]
        rowlen = math.prod(t.shape[1:]) if t.dim() > 1 else 1
        c = -(-d0 // world)
        chunks = torch.chunk(t, world, dim=0) if d0 else ()
        piece = chunks[q].reshape(-1).numpy() if q < len(chunks) else np.zeros(0, w.dtype)
        pad = np.zeros(c * rowlen - piece.size, dtype=w.dtype)
        parts.append(np.concatenate([piece, pad]))
    return np.concatenate(parts) if parts else np.zeros(0)


@pytest.mark.parametrize("seed", range(30))
def test_uneven_splits_against_torch_chunk(seed):
    r = np.random.default_rng(7000 + seed)
    world = int(r.choice([1, 2, 3, 4, 7, 8, 16]))
    shapes = []
    for _ in range(int(r.integers(1, 8))):
        nd = int(r.integers(0, 4))
        shapes.append(tuple(int(x) for x in r.integers(0 if nd > 1 else 1, 12, size=nd)))
    ws = [gen.normal_f32(math.prod(s), 1.0, seed, gen.STREAM_TENSOR, i).reshape(s) for i, s in enumerate(shapes)]
    _, _, _, S = oracle.shard0_geometry(shapes, world)
    for q in range(world):
        buf = oracle.shard0_pack(ws, world, q)
        assert buf.size == S
        np.testing.assert_array_equal(buf.view(np.uint32), _torch_chunk_buffer(ws, world, q).view(np.uint32))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_round_trip_bitwise(seed, dtype):
    r = np.random.default_rng(7100 + seed)
    world = int(r.choice([1, 2, 3, 5, 8, 64]))
    shapes = [tuple(int(x) for x in r.integers(1, 9, size=int(r.integers(0, 4)))) for _ in range(6)]
    ws = []
    for i, s in enumerate(shapes):
        x = gen.normal_f32(math.prod(s), 1.0, seed, gen.STREAM_TENSOR, i)
        x[0] = np.float32("nan")
        x.view(np.uint32)[-1] = 0x80000000       # -0
        ws.append((x if dtype == np.float32 else gen.bf16_bits_trunc(x)).reshape(s))
    full = np.concatenate([oracle.shard0_pack(ws, world, q) for q in range(world)])
    back = oracle.shard0_unpack(full, shapes, world)
    for a, b in zip(back, ws):
        assert a.shape == b.shape
        assert a.tobytes() == np.ascontiguousarray(b).tobytes()


def test_padding_rows_are_zero_and_sizes_equal():
    shapes = [(5, 3), (2,), (), (9, 1, 2)]
    world = 4
    c, r, off, S = oracle.shard0_geometry(shapes, world)
    assert list(c) == [2, 1, 1, 3] and list(r) == [3, 1, 1, 2]
    assert list(off) == [0, 6, 7, 8] and S == 14
    ws = [np.full(s, 7.0, dtype=np.float32) for s in shapes]
    for q in range(world):
        buf = oracle.shard0_pack(ws, world, q)
        real = [min(max(d0 - q * ci, 0), ci) for d0, ci in zip([5, 2, 1, 9], c)]
        for i in range(len(shapes)):
            seg = buf[off[i]:off[i] + c[i] * r[i]]
            assert np.all(seg[:real[i] * r[i]] == 7.0) and np.all(seg[real[i] * r[i]:] == 0.0)
