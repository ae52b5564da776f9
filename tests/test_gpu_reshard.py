"""GPU parity of fp_reshard (a flat buffer cut into N shards recut into N'
shards, "Infra: Data Parallel", section "Checkpoint：让各张卡保存自己的分片") against the
oracle: byte equality, for bf16 and fp32 elements, every new rank at once
and one rank at a time, odd element offsets, destinations pre-filled with
garbage (the zeros past T must be written), old ranks that hold only
padding passed as NULL, a round trip N -> N' -> N, and the d=12288 layer's
bf16 parameters at full size (8 -> 16 and 8 -> 3 ranks).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import dev, say, to_dev, to_host
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu


def _same(a, b):
    a = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    b = np.ascontiguousarray(b).reshape(-1).view(np.uint8)
    return a.shape == b.shape and bool(np.array_equal(a, b))


def _tdtype(dtype):
    return torch.float32 if dtype == np.float32 else torch.int16


def _at(h, offset, dtype):
    buf = torch.zeros(h.size + offset + 8, dtype=_tdtype(dtype), device=dev())
    v = buf[offset:offset + h.size]
    if h.size:
        v.copy_(to_dev(h))
    return v


def _old_shards(T, N, dtype, seed, garbage_padding=True):
    """Host shards of a flat buffer of T random words (NaN / -0 included),
    padding filled with garbage that must never be read."""
    S = -(-T // N)
    r = np.random.default_rng(seed)
    bits = 32 if dtype == np.float32 else 16
    flat = r.integers(0, 2 ** bits, size=N * S, dtype=np.uint64).astype(np.uint32 if bits == 32 else np.uint16)
    if T:
        flat[0] = 0x7FC12345 if bits == 32 else 0x7FC1
    if garbage_padding:
        flat[T:] = 0xBEEF
    flat = flat.view(dtype)
    return [flat[q * S:(q + 1) * S].copy() for q in range(N)]


@pytest.mark.parametrize("T,N,N2", [(1000, 8, 3), (1000, 3, 8), (100_003, 64, 1), (100_003, 1, 64),
                                    (65_536, 16, 16), (777, 7, 5), (5, 8, 3), (0, 4, 2), (3 * 2048 + 5, 2, 128)])
@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_reshard_matches_oracle(fp, T, N, N2, dtype):
    say(f"reshard T={T} N={N} N'={N2} dtype={np.dtype(dtype).name}")
    old = _old_shards(T, N, dtype, T + N * 7 + N2)
    plan = fp.ReshardPlan(T, N, N2)
    S2 = plan.shard_new
    d_old = [(_at(o, q % 4, dtype) if q * plan.shard_old < T else None) for q, o in enumerate(old)]
    garbage = -7 if dtype == np.uint16 else float("nan")
    dst = torch.full((N2 * S2 + 3,), garbage, dtype=_tdtype(dtype), device=dev())[1:1 + N2 * S2]
    plan.reshard(d_old, dst)
    torch.cuda.synchronize()
    want = oracle.reshard(old, T, N2)
    assert _same(to_host(dst), want)
    for q in sorted({0, N2 - 1, N2 // 2}):
        one = torch.full((S2 + 2,), garbage, dtype=_tdtype(dtype), device=dev())[2 - q % 2:2 - q % 2 + S2]
        plan.reshard(d_old, one, rank=q)
        torch.cuda.synchronize()
        assert _same(to_host(one), want[q * S2:(q + 1) * S2]), f"new rank {q}"


@pytest.mark.parametrize("N,N2", [(8, 3), (5, 64)])
def test_reshard_round_trip(fp, N, N2):
    T = 50_001
    say(f"reshard round trip {N} -> {N2} -> {N}")
    old = _old_shards(T, N, np.float32, 3, garbage_padding=False)
    for q in range(N):                                  # proper zero padding
        lo = q * old[0].size
        old[q][max(0, T - lo):] = 0
    fwd = fp.ReshardPlan(T, N, N2)
    mid = fwd.reshard([to_dev(o) for o in old])
    S2 = fwd.shard_new
    back = fp.ReshardPlan(T, N2, N).reshard([mid[q * S2:(q + 1) * S2] for q in range(N2)])
    torch.cuda.synchronize()
    assert _same(to_host(back), np.concatenate(old))


@pytest.mark.parametrize("N2", [16, 3])
def test_reshard_layer_parameters_full_size(fp, N2):
    """The d=12288 layer's bf16 FlatParameter (1.81G elements) cut for 8 ranks
    recut for N' ranks, compared in full with the oracle."""
    cfg = CONFIGS["c4_layer_d12288_nd8"]
    T = sum(math.prod(s) for s in cfg.shapes)
    N = cfg.world
    say(f"reshard full size T={T} 8 -> {N2}")
    plan = fp.ReshardPlan(T, N, N2)
    S = plan.shard_old
    flat = torch.zeros(N * S, dtype=torch.int16, device=dev())
    flat[:T] = gen.torch_bf16_normal(T, 0.02, 3, (gen.STREAM_MASTER,), dev())
    out = plan.reshard([flat[q * S:(q + 1) * S] for q in range(N)])
    torch.cuda.synchronize()
    host = to_host(flat)
    del flat
    got = to_host(out)
    del out
    want = oracle.reshard([host[q * S:(q + 1) * S] for q in range(N)], T, N2)
    assert _same(got, want)


@pytest.mark.parametrize("N2", [128, 32])
def test_reshard_ragged_10k_fp32_full_size(fp, N2):
    """The 10k-tensor FlatParameter's fp32 state (2.73G elements, as the bench
    times it) cut for 64 ranks recut for 128 and for 32, every new rank's
    shard in one call, compared in full with the oracle."""
    cfg = CONFIGS["c5_ragged10k_nd64"]
    T = sum(math.prod(s) for s in cfg.shapes)
    N = cfg.world
    say(f"reshard full size fp32 T={T} {N} -> {N2}")
    plan = fp.ReshardPlan(T, N, N2)
    S = plan.shard_old
    flat = torch.zeros(N * S, dtype=torch.float32, device=dev())
    flat[:T] = gen.torch_normal_f32(T, 0.02, 4, (gen.STREAM_MASTER,), dev())
    out = plan.reshard([flat[q * S:(q + 1) * S] for q in range(N)])
    torch.cuda.synchronize()
    host = to_host(flat)
    del flat
    got = to_host(out)
    del out
    want = oracle.reshard([host[q * S:(q + 1) * S] for q in range(N)], T, N2)
    assert _same(got, want)
    plan.close()
