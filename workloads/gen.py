"""Seeded random draws for the synthetic workloads.

Host draws use numpy's PCG64 keyed by SeedSequence(seed, spawn_key=key);
device draws (for the multi-GB workloads) use torch's Philox generator
seeded from the same SeedSequence.  The key names what is drawn:

    key = (stream, unit, micro, rank)

so that every buffer of every unit, micro-batch and rank is reproducible
on its own.  Gradients are bf16: the fp32 draw with its low 16 bits
dropped (round toward zero).  That is input preparation only -- the
method's own fp32 -> bf16 rounding is not implemented here.
"""

from __future__ import annotations

import numpy as np

STREAM_MASTER = 0      # fp32 master weights (the packed FlatParameter)
STREAM_GRAD = 1        # per-rank bf16 gradients
STREAM_SHARD = 2       # other ranks' bf16 parameter shards
STREAM_EXP_AVG = 3     # first moment when a test starts mid-run
STREAM_EXP_AVG_SQ = 4  # second moment when a test starts mid-run
STREAM_INF = 5         # positions of injected non-finite gradients
STREAM_TENSOR = 6      # per-tensor source values for pack tests


def seed_sequence(seed: int, *key: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))


def rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_sequence(seed, *key)))


def normal_f32(n: int, sigma: float, seed: int, *key: int) -> np.ndarray:
    """n float32 draws from N(0, sigma), sigma read as standard deviation."""
    x = rng(seed, *key).standard_normal(int(n), dtype=np.float32)
    return x * np.float32(sigma)


def bf16_bits_trunc(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of each float32 (truncation), as uint16 bf16 patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_normal(n: int, sigma: float, seed: int, *key: int) -> np.ndarray:
    return bf16_bits_trunc(normal_f32(n, sigma, seed, *key))


def positions(n: int, fraction: float, seed: int, *key: int) -> np.ndarray:
    """Sorted distinct indices in [0, n): round(fraction * n) of them, at least 1."""
    k = max(1, int(round(fraction * n)))
    k = min(k, n)
    return np.sort(rng(seed, *key).choice(n, size=k, replace=False))


# ----------------------------------------------------------------------------
# Device draws for workloads too large to build on the host.
# ----------------------------------------------------------------------------

def torch_seed(seed: int, *key: int) -> int:
    state = seed_sequence(seed, *key).generate_state(2, np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & ((1 << 63) - 1)


def torch_normal_f32(n: int, sigma: float, seed: int, key, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, *key))
    x = torch.randn(int(n), generator=g, device=device, dtype=torch.float32)
    return x.mul_(float(sigma))


def torch_bf16_bits_trunc(x):
    """Device counterpart of bf16_bits_trunc: int16 tensor of bf16 patterns."""
    import torch
    return torch.bitwise_right_shift(x.view(torch.int32), 16).to(torch.int16)


def torch_bf16_normal(n: int, sigma: float, seed: int, key, device):
    return torch_bf16_bits_trunc(torch_normal_f32(n, sigma, seed, key, device))
