"""GPU parity of the hybrid-sharding reduce (fp_reduce_shard_hybrid) against
the oracle: bitwise fp32 results (non-finite by class) and the same overflow
flag, the norm within 1e-12 rel.  "PyTorch FSDP ..." section 3.3 (sharding
factor F); "4.1 数据并行详解", HYBRID_SHARD.  Cases: a value pattern whose
two-level sum differs from the flat one (so the order itself is checked),
W / F from 8 / 1 to 128 / 16 and 12 / 4, ragged sizes with odd offsets,
accumulation over micro-batches, injected inf.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import assert_f32_bitexact, dev, say, to_dev, to_host
from workloads import gen

pytestmark = pytest.mark.gpu


def _rows(host_rows, offset):
    out = []
    for h in host_rows:
        buf = torch.zeros(h.size + offset + 8, dtype=torch.int16, device=dev())
        v = buf[offset:offset + h.size]
        v.copy_(to_dev(h))
        out.append(v)
    return out


@pytest.mark.parametrize("S", [16, 19, 4 * 2048 + 1])
def test_two_level_order_on_gpu(fp, S):
    """Ranks 2^24, 1, 1, 1 in groups of 2: the two-level sum is 2^24 + 2, the
    flat sum 2^24 (each +1 rounds back to the even 2^24)."""
    say(f"hybrid order S={S}")
    vals = [0x4B80, 0x3F80, 0x3F80, 0x3F80]           # bf16 of 2^24, 1, 1, 1
    rows = [np.full(S, v, np.uint16) for v in vals]
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    fp.reduce_shard_hybrid([to_dev(r) for r in rows], acc, group=2, scale=1.0)
    flat = torch.zeros(S, dtype=torch.float32, device=dev())
    fp.reduce_shard([to_dev(r) for r in rows], flat, scale=1.0)
    torch.cuda.synchronize()
    assert np.all(to_host(acc) == 2.0 ** 24 + 2)
    assert np.all(to_host(flat) == 2.0 ** 24)
    assert_f32_bitexact(to_host(acc), oracle.reduce_hybrid(rows, 2, np.float32(1.0)))


@pytest.mark.parametrize("world,group,S,n_micro,offset", [
    (16, 8, 100_003, 2, 1), (8, 2, 4099, 4, 0), (64, 8, 20_001, 1, 3), (128, 16, 5003, 1, 2),
    (12, 4, 777, 2, 1), (8, 8, 3001, 1, 0), (8, 1, 3001, 1, 0), (4, 2, 3, 1, 1)])
def test_hybrid_reduce_matches_oracle(fp, world, group, S, n_micro, offset):
    say(f"hybrid reduce W={world} F={group} S={S} n={n_micro} offset={offset}")
    seed = world * 1000 + group
    scale = np.float32(1.0 / (world * n_micro))
    micro = [[gen.bf16_normal(S, 1e-2, seed, gen.STREAM_GRAD, m, q) for q in range(world)]
             for m in range(n_micro)]
    if S > 10:
        micro[-1][world - 1][S // 3] = 0x7F80                # +inf in the last group
    acc_o = np.zeros(S, np.float32)
    for m in range(n_micro):
        oracle.reduce_hybrid(micro[m], group, scale, acc_o, accumulate=m > 0)
    flag_o = oracle.found_inf(acc_o)
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    ws = fp.new_workspace(dev(), S)
    for m in range(n_micro):
        fp.reduce_shard_hybrid(_rows(micro[m], offset), acc, group=group, scale=float(scale),
                               accumulate=m > 0, found_inf=flag, sq_norm=sq if m == n_micro - 1 else None,
                               workspace=ws)
    torch.cuda.synchronize()
    assert_f32_bitexact(to_host(acc), acc_o, "hybrid reduce")
    assert int(flag.item()) == flag_o
    if not flag_o:
        want = oracle.sq_norm(acc_o)
        assert abs(float(sq.item()) - want) <= 1e-12 * want


def test_hybrid_reduce_layer_d12288_full_size(fp):
    """The d=12288 layer's slice for F = 8 (226.5M elements) reduced over
    W = 16 ranks in two groups, compared with the oracle at 2^14 sampled
    positions, with the overflow flag and the norm's determinism."""
    from workloads import CONFIGS
    import math as _m
    cfg = CONFIGS["c4_layer_d12288_nd8"]
    F, W = cfg.world, 2 * cfg.world
    S = fp.Plan(cfg.shapes, F).shard
    say(f"hybrid full size S={S} W={W} F={F}")
    rows = gen.torch_bf16_normal(W * S, 1e-3, 5, (gen.STREAM_GRAD,), dev()).view(W, S)
    idx = torch.from_numpy(np.sort(np.random.default_rng(4).choice(S, 1 << 14, replace=False))).to(dev())
    acc = torch.empty(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(2, dtype=torch.float64, device=dev())
    ws = fp.new_workspace(dev(), S)
    fp.reduce_shard_hybrid(rows, acc, group=F, scale=1.0 / W, found_inf=flag, sq_norm=sq[0:1], workspace=ws)
    fp.reduce_shard_hybrid(rows, acc, group=F, scale=1.0 / W, found_inf=flag, sq_norm=sq[1:2], workspace=ws)
    torch.cuda.synchronize()
    picked = [a for a in rows.index_select(1, idx).cpu().numpy().view(np.uint16)]
    want = oracle.reduce_hybrid(picked, F, np.float32(1.0 / W))
    assert_f32_bitexact(acc.index_select(0, idx).cpu().numpy(), want, "hybrid reduce, sampled")
    assert int(flag.item()) == 0
    assert float(sq[0].item()) == float(sq[1].item()) and _m.isfinite(float(sq[0].item()))


@pytest.mark.parametrize("layout", ["line-aligned rows", "packed rows"])
def test_hybrid_ragged_10k_full_size(fp, layout):
    """The 10k-tensor group's slice for F = 64 (42.6M elements) reduced over
    W = 128 ranks in two groups, with each rank's row on a cache line (as the
    bench lays them out) and packed back to back (rows 4-byte aligned, the
    unaligned loads), against the oracle at 2^14 sampled positions."""
    from workloads import CONFIGS
    cfg = CONFIGS["c5_ragged10k_nd64"]
    F, W = cfg.world, 2 * cfg.world
    S = -(-sum(math.prod(s) for s in cfg.shapes) // F)
    Sp = -(-S // 64) * 64 if layout == "line-aligned rows" else S
    say(f"hybrid full size S={S} W={W} F={F} {layout}")
    rows = gen.torch_bf16_normal(W * Sp, 1e-3, 6, (gen.STREAM_GRAD,), dev()).view(W, Sp)[:, :S]
    idx = torch.from_numpy(np.sort(np.random.default_rng(5).choice(S, 1 << 14, replace=False))).to(dev())
    acc = torch.empty(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    fp.reduce_shard_hybrid(rows, acc, group=F, scale=1.0 / W, found_inf=flag)
    torch.cuda.synchronize()
    picked = [a for a in rows.index_select(1, idx).cpu().numpy().view(np.uint16)]
    want = oracle.reduce_hybrid(picked, F, np.float32(1.0 / W))
    assert_f32_bitexact(acc.index_select(0, idx).cpu().numpy(), want, "hybrid reduce, sampled")
    assert int(flag.item()) == 0
