"""GPU parity on the five workloads at their full sizes.

* d=1024 layer unit, N_d=8 (1.57M-element shard): the whole shard compared
  with the oracle for three consecutive steps, on both step paths.
* 611M-parameter model in 25 MiB buckets, N_d=16, 4 micro-batches: every
  bucket reduced and updated on the GPU; the oracle recomputes 2^14 sampled
  elements per bucket from the same inputs; full-size properties (other
  shards copied bit for bit, own shard = bf16 of the new master).
* d=12288 layer unit, N_d=8 (226.5M-element shard): the fp32 pack of its 12
  tensors checked tensor by tensor; sampled oracle parity of the step
  plus the same properties and the gradient norm against an fp64 sum.
* 10k ragged tensors (2.73G elements), N_d=64: the pack checked tensor by
  tensor against its source and at sampled positions by the oracle's
  locator; the step with 0.01% injected +inf must skip (state untouched
  bit for bit), and without the infs matches the oracle at sampled elements.
Inputs are drawn on the device from seeded generators (workloads.gen); the
oracle receives the same input values gathered at the sampled positions.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (assert_bf16_equal, assert_bf16_within_1ulp, assert_f32_bitexact,
                        assert_f32_close, dev, hp_kwargs, say, to_dev, to_host, norm_rel_tol)
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu


def _bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _gather_rows(rows, idx):
    """rows: [N, S] int16 device tensor; idx: device int64 -> list of N host uint16 arrays."""
    g = rows.index_select(1, idx)
    return [a for a in _bf16_host(g)]


def _samples(n, k, seed, *key):
    k = min(k, n)
    return np.sort(gen.rng(seed, *key).choice(n, size=k, replace=False)).astype(np.int64)


def _torch_cast(t):
    return t.to(torch.bfloat16).view(torch.int16)


def _others_equal(full, others, rank, S):
    """full equals `others` outside the own shard [rank*S, (rank+1)*S)."""
    lo, hi = rank * S, (rank + 1) * S
    return torch.equal(full[:lo], others[:lo]) and torch.equal(full[hi:], others[hi:])


# ------------------------------------------------------------------ d=1024 unit
@pytest.mark.parametrize("flags", [0, 4])
@pytest.mark.parametrize("rank", [1, 7])
def test_layer_d1024_full_shard_three_steps(fp, rank, flags):
    cfg = CONFIGS["c2_layer_d1024_nd8"]
    world, hp = cfg.world, cfg.hp
    plan = fp.Plan(cfg.shapes, world)
    S = plan.shard
    say(f"d1024 unit rank={rank} flags={flags} S={S}")
    master = gen.normal_f32(S, cfg.master_sigma, cfg.seed, gen.STREAM_MASTER, 0, 0, rank)
    th_o, m_o, v_o = master.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    d_th, d_m, d_v = to_dev(master), torch.zeros(S, device=dev()), torch.zeros(S, device=dev())
    acc = torch.zeros(S, device=dev())
    ws = fp.new_workspace(dev(), S)
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    for t in (1, 2, 3):
        grads = [gen.bf16_normal(S, cfg.grad_sigma, cfg.seed, gen.STREAM_GRAD, t, 0, q) for q in range(world)]
        others = [gen.bf16_normal(S, cfg.master_sigma, cfg.seed, gen.STREAM_SHARD, t, 0, q) for q in range(world)]
        acc_o = np.zeros(S, np.float32)
        full_o, flag_o, norm_o = oracle.shard_step([grads], acc_o, th_o, m_o, v_o, others, rank,
                                                   hp=hp, step=t)
        flag = torch.zeros(1, dtype=torch.int32, device=dev())
        shards = [None if q == rank else to_dev(o) for q, o in enumerate(others)]
        fp.shard_step(to_dev(np.stack(grads)), acc, d_th, d_m, d_v, shards, full, rank,
                      scale=1.0 / world, step=t, found_inf=flag, sq_norm=sq, workspace=ws, flags=flags,
                      **hp_kwargs(hp))
        torch.cuda.synchronize()
        assert int(flag.item()) == flag_o == 0
        assert_f32_close(to_host(d_th), th_o, f"master t={t}")
        assert_f32_close(to_host(d_m), m_o, f"exp_avg t={t}")
        assert_f32_close(to_host(d_v), v_o, f"exp_avg_sq t={t}")
        fh = to_host(full)
        own = slice(rank * S, (rank + 1) * S)
        assert_bf16_within_1ulp(fh[own], full_o[own], "own shard")
        mask = np.ones(world * S, bool)
        mask[own] = False
        assert_bf16_equal(fh[mask], full_o[mask], "other shards")
        assert float(sq.item()) == pytest.approx(norm_o, rel=norm_rel_tol(S))
    assert fp.workspace_timeouts(ws) == 0


def test_layer_d1024_pack_and_views(fp):
    cfg = CONFIGS["c2_layer_d1024_nd8"]
    say("d1024 unit pack")
    host = [gen.normal_f32(math.prod(s), cfg.master_sigma, cfg.seed, gen.STREAM_TENSOR, i).reshape(s)
            for i, s in enumerate(cfg.shapes)]
    plan = fp.Plan(cfg.shapes, cfg.world)
    flat = plan.pack([to_dev(h) for h in host])
    torch.cuda.synchronize()
    want = oracle.pack(host, cfg.world)
    assert np.array_equal(to_host(flat).view(np.uint32), want.view(np.uint32))
    S = plan.shard
    numel = [math.prod(s) for s in cfg.shapes]
    for q in (1, 7):
        bo, ln, to = oracle.views(numel, cfg.world, q)
        for i, v in enumerate(plan.views(flat[q * S:(q + 1) * S], q)):
            assert v.numel() == ln[i]
            if ln[i]:
                assert v.data_ptr() == flat.data_ptr() + 4 * (q * S + bo[i])


# ------------------------------------------------------------------ 611M buckets
def test_611m_buckets_four_micro_batches(fp):
    cfg = CONFIGS["c3_611m_buckets_nd16"]
    world, n, hp, rank = cfg.world, cfg.n_micro, cfg.hp, cfg.ranks[0]
    sizes = cfg.units()
    shards = [T // world for T in sizes]
    say(f"611M buckets: {len(sizes)} buckets, shards {shards[0]} / {shards[-1]}, N={world}, n={n}")
    scale = np.float32(1.0 / (world * n))
    offs = np.concatenate([[0], np.cumsum(shards)])
    total = int(offs[-1])
    th = gen.torch_normal_f32(total, cfg.master_sigma, cfg.seed, (gen.STREAM_MASTER,), dev())
    m = gen.torch_normal_f32(total, 1e-4, cfg.seed, (gen.STREAM_EXP_AVG,), dev())
    v = gen.torch_normal_f32(total, 1e-3, cfg.seed, (gen.STREAM_EXP_AVG_SQ,), dev()).square_()
    th0, m0, v0 = th.clone(), m.clone(), v.clone()
    acc = torch.zeros(total, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    samples = [torch.from_numpy(_samples(S, 1 << 14, cfg.seed, 7, b)).to(dev()) for b, S in enumerate(shards)]
    sampled = [[None] * n for _ in sizes]
    for mi in range(n):
        for b, S in enumerate(shards):
            g = gen.torch_bf16_normal(world * S, cfg.grad_sigma, cfg.seed, (gen.STREAM_GRAD, b, mi), dev())
            g = g.view(world, S)
            fp.reduce_shard(g, acc[offs[b]:offs[b + 1]], scale=float(scale), accumulate=mi > 0, found_inf=flag)
            sampled[b][mi] = _gather_rows(g, samples[b])
            del g
    step = 5
    for b, S in enumerate(shards):
        sl = slice(int(offs[b]), int(offs[b + 1]))
        full = torch.zeros(world * S, dtype=torch.int16, device=dev())
        fp.adamw_shard(acc[sl], th[sl], m[sl], v[sl], step=step, found_inf=flag,
                       param_bf16=full[rank * S:(rank + 1) * S], **hp_kwargs(hp))
        others = gen.torch_bf16_normal(world * S, cfg.master_sigma, cfg.seed, (gen.STREAM_SHARD, b), dev())
        fp.unshard([None if q == rank else others[q * S:(q + 1) * S] for q in range(world)], full)
        torch.cuda.synchronize()
        assert _others_equal(full, others, rank, S), f"bucket {b}: other shards"
        assert torch.equal(full[rank * S:(rank + 1) * S], _torch_cast(th[sl])), f"bucket {b}: own shard cast"
        del others
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    # oracle on the sampled elements of every bucket
    for b, S in enumerate(shards):
        idx = samples[b] + int(offs[b])
        acc_o = np.zeros(idx.numel(), np.float32)
        for mi in range(n):
            oracle.reduce(sampled[b][mi], scale, acc_o, accumulate=mi > 0)
        assert_f32_bitexact(to_host(acc.index_select(0, idx)), acc_o, f"bucket {b} acc")
        th_o, m_o, v_o = (to_host(x.index_select(0, idx)) for x in (th0, m0, v0))
        oracle.adamw(acc_o, th_o, m_o, v_o, step=step, **hp_kwargs(hp))
        assert_f32_close(to_host(th.index_select(0, idx)), th_o, f"bucket {b} master")
        assert_f32_close(to_host(m.index_select(0, idx)), m_o, f"bucket {b} exp_avg")
        assert_f32_close(to_host(v.index_select(0, idx)), v_o, f"bucket {b} exp_avg_sq")


# ------------------------------------------------------------------ d=12288 unit
def test_layer_d12288_shard(fp):
    cfg = CONFIGS["c4_layer_d12288_nd8"]
    world, hp, rank = cfg.world, cfg.hp, cfg.ranks[0]
    S = cfg.units()[0] // world
    say(f"d12288 unit S={S}")
    grads = gen.torch_bf16_normal(world * S, cfg.grad_sigma, cfg.seed, (gen.STREAM_GRAD,), dev()).view(world, S)
    th = gen.torch_normal_f32(S, cfg.master_sigma, cfg.seed, (gen.STREAM_MASTER,), dev())
    m = gen.torch_normal_f32(S, 1e-4, cfg.seed, (gen.STREAM_EXP_AVG,), dev())
    v = gen.torch_normal_f32(S, 1e-3, cfg.seed, (gen.STREAM_EXP_AVG_SQ,), dev()).square_()
    idx = torch.from_numpy(_samples(S, 1 << 20, cfg.seed, 8)).to(dev())
    g_s = _gather_rows(grads, idx)
    th_o, m_o, v_o = (to_host(x.index_select(0, idx)) for x in (th, m, v))
    others = gen.torch_bf16_normal(world * S, cfg.master_sigma, cfg.seed, (gen.STREAM_SHARD,), dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    acc = torch.empty(S, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    ws = fp.new_workspace(dev(), S)
    step = 2
    fp.shard_step(grads, acc, th, m, v, [None if q == rank else others[q * S:(q + 1) * S] for q in range(world)],
                  full, rank, scale=1.0 / world, step=step, found_inf=flag, sq_norm=sq, workspace=ws,
                  flags=fp.FP_STEP_KEEP_GRAD, **hp_kwargs(hp))
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    acc_o = oracle.reduce(g_s, np.float32(1.0 / world))
    assert_f32_bitexact(to_host(acc.index_select(0, idx)), acc_o, "reduced gradient")
    oracle.adamw(acc_o, th_o, m_o, v_o, step=step, **hp_kwargs(hp))
    assert_f32_close(to_host(th.index_select(0, idx)), th_o, "master")
    assert_f32_close(to_host(m.index_select(0, idx)), m_o, "exp_avg")
    assert_f32_close(to_host(v.index_select(0, idx)), v_o, "exp_avg_sq")
    own = full[rank * S:(rank + 1) * S]
    assert_bf16_within_1ulp(_bf16_host(own.index_select(0, idx)), oracle.f32_to_bf16(th_o), "own shard")
    assert torch.equal(own, _torch_cast(th))
    assert torch.equal(full[S:], others[S:])                      # rank 0: every other shard
    norm = float(acc.double().square().sum().item())
    assert float(sq.item()) == pytest.approx(norm, rel=norm_rel_tol(S))


def test_layer_d12288_pack(fp):
    """The d=12288 layer's 12 fp32 tensors (1.81G elements, 7.25 GB) packed as
    the bench packs them: every tensor's range of the FlatParameter equal to
    the tensor bit for bit, and every rank's views of the right lengths."""
    cfg = CONFIGS["c4_layer_d12288_nd8"]
    numel = [math.prod(s) for s in cfg.shapes]
    say(f"d12288 pack: {len(numel)} tensors, {sum(numel)} elements")
    plan = fp.Plan(cfg.shapes, cfg.world)
    tensors = [gen.torch_normal_f32(n, 1.0, cfg.seed, (gen.STREAM_TENSOR, i), dev()).view(s)
               for i, (n, s) in enumerate(zip(numel, cfg.shapes))]
    flat = plan.pack(tensors)
    torch.cuda.synchronize()
    o = 0
    for i, t in enumerate(tensors):
        assert torch.equal(flat[o:o + numel[i]].view(torch.int32), t.reshape(-1).view(torch.int32)), f"tensor {i}"
        o += numel[i]
    assert o == plan.padded                               # 8 divides T: no padding
    S = plan.shard
    for q in range(cfg.world):
        _, ln, _ = oracle.views(numel, cfg.world, q)
        assert [v.numel() for v in plan.views(flat[q * S:(q + 1) * S], q)] == list(ln)
    plan.close()


# ------------------------------------------------------------------ 10k ragged tensors
def test_ragged_10k_pack(fp):
    cfg = CONFIGS["c5_ragged10k_nd64"]
    numel = [s[0] for s in cfg.shapes]
    say(f"ragged pack: {len(numel)} tensors, {sum(numel)} elements")
    plan = fp.Plan(cfg.shapes, cfg.world)
    tensors = [gen.torch_normal_f32(n, 1.0, cfg.seed, (gen.STREAM_TENSOR, i), dev()) for i, n in enumerate(numel)]
    flat = plan.pack(tensors)
    torch.cuda.synchronize()
    o = 0
    for i, t in enumerate(tensors):
        assert torch.equal(flat[o:o + numel[i]].view(torch.int32), t.view(torch.int32)), f"tensor {i}"
        o += numel[i]
    assert not flat[o:].view(torch.int32).any(), "padding must be zero"
    pos = _samples(plan.padded, 8192, cfg.seed, 9)
    ti, off = oracle.locate_sorted(numel, pos)
    got = to_host(flat[torch.from_numpy(pos).to(dev())]).view(np.uint32)
    want = np.zeros(pos.size, np.uint32)                      # padding positions stay 0
    for u in np.unique(ti[ti >= 0]):
        sel = np.flatnonzero(ti == u)
        vals = tensors[u].index_select(0, torch.from_numpy(off[sel]).to(dev()))
        want[sel] = to_host(vals).view(np.uint32)
    np.testing.assert_array_equal(got, want)
    S = plan.shard
    for q in cfg.ranks:
        views = plan.views(flat[q * S:(q + 1) * S], q)
        bo, ln, to = oracle.views(numel, cfg.world, q)
        assert [v.numel() for v in views] == list(ln)


@pytest.mark.parametrize("inject", [True, False])
@pytest.mark.parametrize("rank", [0, 63])
def test_ragged_10k_step(fp, rank, inject):
    cfg = CONFIGS["c5_ragged10k_nd64"]
    world, hp = cfg.world, cfg.hp
    T = sum(s[0] for s in cfg.shapes)
    _, P, S = oracle.geometry([T], world)
    say(f"ragged step rank={rank} inject_inf={inject} S={S}")
    grads = gen.torch_bf16_normal(world * S, cfg.grad_sigma, cfg.seed, (gen.STREAM_GRAD, rank), dev()).view(world, S)
    valid = S - (P - T) if rank == world - 1 else S           # non-padding elements of this shard
    if rank == world - 1:
        grads[:, valid:] = 0                                  # padding gradients are zero
    if inject:
        for q in range(world):
            p = torch.from_numpy(gen.positions(valid, cfg.inf_fraction, cfg.seed, gen.STREAM_INF, rank, q)).to(dev())
            grads[q].index_fill_(0, p, 0x7F80)
    th = gen.torch_normal_f32(S, cfg.master_sigma, cfg.seed, (gen.STREAM_MASTER, rank), dev())
    m = gen.torch_normal_f32(S, 1e-4, cfg.seed, (gen.STREAM_EXP_AVG, rank), dev())
    v = gen.torch_normal_f32(S, 1e-3, cfg.seed, (gen.STREAM_EXP_AVG_SQ, rank), dev()).square_()
    th0, m0, v0 = th.clone(), m.clone(), v.clone()
    idx = torch.from_numpy(_samples(S, 1 << 18, cfg.seed, 10, rank)).to(dev())
    g_s = _gather_rows(grads, idx)
    others = gen.torch_bf16_normal(world * S, cfg.master_sigma, cfg.seed, (gen.STREAM_SHARD, rank), dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    acc = torch.empty(S, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    ws = fp.new_workspace(dev(), S)
    fp.shard_step(grads, acc, th, m, v, [None if q == rank else others[q * S:(q + 1) * S] for q in range(world)],
                  full, rank, scale=1.0 / world, step=3, found_inf=flag, workspace=ws, **hp_kwargs(hp))
    torch.cuda.synchronize()
    assert int(flag.item()) == (1 if inject else 0)
    own = full[rank * S:(rank + 1) * S]
    assert _others_equal(full, others, rank, S)
    if inject:
        for a, b in ((th, th0), (m, m0), (v, v0)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "state must be untouched"
        assert torch.equal(own, _torch_cast(th0))
    else:
        acc_o = oracle.reduce(g_s, np.float32(1.0 / world))
        th_o, m_o, v_o = (to_host(x.index_select(0, idx)) for x in (th0, m0, v0))
        oracle.adamw(acc_o, th_o, m_o, v_o, step=3, **hp_kwargs(hp))
        assert_f32_close(to_host(th.index_select(0, idx)), th_o, "master")
        assert_f32_close(to_host(m.index_select(0, idx)), m_o, "exp_avg")
        assert_f32_close(to_host(v.index_select(0, idx)), v_o, "exp_avg_sq")
        assert torch.equal(own, _torch_cast(th))
    assert fp.workspace_timeouts(ws) == 0
