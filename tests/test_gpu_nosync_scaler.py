"""GPU parity of the steps on either side of the reduce against the oracle.

* fp_local_accumulate / fp_local_finish (accumulation without
  communication, "Infra: Data Parallel", Naive-DP gradient-accumulation
  paragraph; "PyTorch FSDP ..." section 3.4): bitwise (non-finite floats by
  class) on ragged sizes, odd element offsets, specials; composed with the
  shard step into a no_sync step.
* fp_grad_coef, fp_scaler_update and the gradient factor of AdamW and of the
  step entry points ("PyTorch FSDP ..." section 3.5, sharded gradient
  scaler): the factor within a few fp64 ulps, the loss-scale trajectory
  exactly, AdamW state within 1e-6 rel / 1e-9 abs, bf16 parameters within
  1 ulp; clipping by the reduced gradient's norm through the separate entry
  points.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (assert_bf16_equal, assert_bf16_within_1ulp, assert_f32_bitexact, assert_f32_close,
                        dev, hp_kwargs, say, to_dev, to_host)
from workloads import gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()


def _at(h, offset, dtype=torch.int16):
    """A device copy of host array h starting `offset` elements into its own buffer."""
    buf = torch.zeros(h.size + offset + 8, dtype=dtype, device=dev())
    v = buf[offset:offset + h.size]
    if h.size:
        v.copy_(to_dev(h))
    return v


def _grads(n, seed, m, q, specials):
    g = gen.bf16_normal(n, 1e-2, seed, gen.STREAM_GRAD, m, q)
    if specials and n:
        r = np.random.default_rng(seed * 7 + m)
        pool = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F7F, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x7FC1],
                        np.uint16)
        idx = r.integers(0, n, size=max(1, n // 50))
        g[idx] = pool[r.integers(0, pool.size, size=idx.size)]
    return g


@pytest.mark.parametrize("n", [1, 3, 4, 1023, 2048 * 5 + 3, 100003])
@pytest.mark.parametrize("n_micro", [1, 2, 4])
def test_local_accumulation_matches_oracle(fp, n, n_micro):
    off = n % 4
    say(f"local accumulate n={n} n_micro={n_micro} offset={off}")
    seed = 40 + n_micro
    gs = [_grads(n, seed, m, 0, specials=n > 8) for m in range(n_micro)]
    local_o = None
    local = torch.zeros(n, dtype=torch.float32, device=dev())
    for m in range(n_micro - 1):
        local_o = oracle.local_accumulate(gs[m], local_o, accumulate=m > 0)
        fp.local_accumulate(_at(gs[m], off), local, accumulate=m > 0)
    out = _at(np.zeros(n, np.uint16), (off + 1) % 4)
    fp.local_finish(_at(gs[-1], off), out, local if n_micro > 1 else None, accumulate=n_micro > 1)
    want = oracle.local_finish(gs[-1], local_o, accumulate=n_micro > 1)
    torch.cuda.synchronize()
    if n_micro > 1:
        assert_f32_bitexact(to_host(local), local_o, "local sum")
    assert_bf16_equal(to_host(out), want, "exchanged row")


def test_local_accumulation_empty(fp):
    local = torch.zeros(4, dtype=torch.float32, device=dev())
    fp.local_accumulate(torch.zeros(0, dtype=torch.int16, device=dev()), local[:0], accumulate=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("world,n_micro,S", [(8, 4, 1_574_528), (4, 2, 100_003)])
def test_no_sync_step_matches_oracle(fp, world, n_micro, S):
    """A no_sync step of rank 1: every rank accumulates its micro-batches
    locally over its slice, rounds once to bf16, and the shard step reduces
    those rows with 1/(N n); against the oracle's same composition."""
    rank, seed = 1, 77
    say(f"no_sync step world={world} n_micro={n_micro} S={S}")
    g = [[gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, m, q) for q in range(world)] for m in range(n_micro)]
    th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER)
    others = [gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, q) for q in range(world)]
    rows_o = []
    for q in range(world):
        loc = None
        for m in range(n_micro - 1):
            loc = oracle.local_accumulate(g[m][q], loc, accumulate=m > 0)
        rows_o.append(oracle.local_finish(g[-1][q], loc, accumulate=n_micro > 1))
    th_o, m_o, v_o, acc_o = th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.float32)
    # the exchanged rows are one "micro-batch" of the reduce, scaled by 1/(N n)
    oracle.reduce(rows_o, np.float32(1.0 / (world * n_micro)), acc_o)
    flag_o = oracle.found_inf(acc_o)
    oracle.adamw(acc_o, th_o, m_o, v_o, step=1, skip=bool(flag_o), **hp_kwargs(HP))
    full_o = oracle.unshard([oracle.f32_to_bf16(th_o) if q == rank else others[q] for q in range(world)])

    rows = []
    local = torch.zeros(S, dtype=torch.float32, device=dev())
    for q in range(world):
        for m in range(n_micro - 1):
            fp.local_accumulate(to_dev(g[m][q]), local, accumulate=m > 0)
        out = torch.empty(S, dtype=torch.int16, device=dev())
        fp.local_finish(to_dev(g[-1][q]), out, local, accumulate=n_micro > 1)
        rows.append(out)
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    d_th, d_m, d_v = to_dev(th), torch.zeros(S, dtype=torch.float32, device=dev()), \
        torch.zeros(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    shards = [to_dev(o) for o in others]
    shards[rank] = None
    fp.shard_step(rows, acc, d_th, d_m, d_v, shards, full, rank, scale=1.0 / (world * n_micro),
                  found_inf=flag, step=1, workspace=fp.new_workspace(dev(), S), **hp_kwargs(HP))
    torch.cuda.synchronize()
    for q in range(world):
        assert_bf16_equal(to_host(rows[q]), rows_o[q], f"row of rank {q}")
    assert int(flag.item()) == flag_o
    assert_f32_close(to_host(d_th), th_o, "master")
    assert_f32_close(to_host(d_m), m_o, "exp_avg")
    assert_f32_close(to_host(d_v), v_o, "exp_avg_sq")
    fh = to_host(full)
    own = slice(rank * S, (rank + 1) * S)
    assert_bf16_within_1ulp(fh[own], full_o[own], "own shard")
    mask = np.ones(world * S, bool)
    mask[own] = False
    assert_bf16_equal(fh[mask], full_o[mask], "other shards")


# ------------------------------------------------------------------ scaler and clipping
def _rel_close(got, want, rel):
    return abs(got - want) <= rel * abs(want)


@pytest.mark.parametrize("sq,L,M", [(4.0, 1.0, 0.0), (4.0, 2.0, 0.5), (1e6, 65536.0, 1.0), (1e-10, 1024.0, 5.0),
                                    (0.0, 1.0, 1.0), (2.5e9, 3.0, 7.25), (123.0, 2.0 ** 24, 0.0)])
def test_grad_coef_matches_oracle(fp, sq, L, M):
    say(f"grad coef sq={sq} scale={L} max_norm={M}")
    coef = torch.zeros(1, dtype=torch.float64, device=dev())
    fp.grad_coef(coef, sq_norm=torch.tensor([sq], dtype=torch.float64, device=dev()),
                 loss_scale=torch.tensor([L], dtype=torch.float32, device=dev()), max_norm=M)
    want = oracle.grad_coef(sq, L, M)
    assert _rel_close(float(coef.item()), want, 4e-16)
    fp.grad_coef(coef, max_norm=0.0)
    assert float(coef.item()) == 1.0


def test_loss_scale_trajectory_matches_oracle(fp):
    say("scaler trajectory")
    r = np.random.default_rng(9)
    flags = (r.random(60) < 0.2).astype(np.int32)
    scale = torch.tensor([65536.0], dtype=torch.float32, device=dev())
    clean = torch.zeros(1, dtype=torch.int32, device=dev())
    fi = torch.zeros(1, dtype=torch.int32, device=dev())
    s_o, c_o = 65536.0, 0
    for f in flags:
        fi.fill_(int(f))
        fp.scaler_update(fi, scale, clean, growth_interval=4, growth_factor=2.0, backoff_factor=0.5)
        s_o, c_o = oracle.scaler_update(int(f), s_o, c_o, growth_interval=4)
        assert (float(scale.item()), int(clean.item())) == (s_o, c_o)
    # non-power-of-two factors: one fp32 multiply each
    fi.fill_(1)
    fp.scaler_update(fi, scale, clean, growth_factor=1.7, backoff_factor=0.37, growth_interval=1)
    s_o, c_o = oracle.scaler_update(1, s_o, c_o, growth_factor=1.7, backoff_factor=0.37, growth_interval=1)
    assert float(scale.item()) == s_o


@pytest.mark.parametrize("S", [1, 4099, 1_000_003])
def test_adamw_with_gradient_factor(fp, S):
    """Loss-scaled gradient, unscaled and clipped through the factor: the
    reduce's Sum g^2 -> fp_grad_coef -> fp_adamw_shard."""
    say(f"adamw with factor S={S}")
    L, world, seed = 1024.0, 4, 5
    grads = [gen.bf16_normal(S, 1e-3 * L, seed, gen.STREAM_GRAD, 0, q) for q in range(world)]
    th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER)
    acc_o = oracle.reduce(grads, np.float32(1.0 / world))
    sq_o = oracle.sq_norm(acc_o)
    M = 0.3 * math.sqrt(sq_o) / L          # clips
    coef_o = oracle.grad_coef(sq_o, L, M)
    th_o, m_o, v_o = th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    oracle.adamw(acc_o, th_o, m_o, v_o, step=1, coef=coef_o, **hp_kwargs(HP))

    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    fp.reduce_shard([to_dev(x) for x in grads], acc, scale=1.0 / world, found_inf=flag, sq_norm=sq,
                    workspace=fp.new_workspace(dev(), S))
    coef = torch.zeros(1, dtype=torch.float64, device=dev())
    fp.grad_coef(coef, sq_norm=sq, loss_scale=torch.tensor([L], dtype=torch.float32, device=dev()), max_norm=M)
    d_th, d_m, d_v = to_dev(th), torch.zeros(S, dtype=torch.float32, device=dev()), \
        torch.zeros(S, dtype=torch.float32, device=dev())
    out = torch.zeros(S, dtype=torch.int16, device=dev())
    fp.adamw_shard(acc, d_th, d_m, d_v, step=1, found_inf=flag, param_bf16=out, grad_coef=coef,
                   **hp_kwargs(HP))
    torch.cuda.synchronize()
    assert _rel_close(float(sq.item()), sq_o, 1e-12)
    assert _rel_close(float(coef.item()), coef_o, 1e-11)
    assert coef_o < 1.0 / L
    assert_f32_close(to_host(d_th), th_o, "master")
    assert_f32_close(to_host(d_m), m_o, "exp_avg")
    assert_f32_close(to_host(d_v), v_o, "exp_avg_sq")
    assert_bf16_within_1ulp(to_host(out), oracle.f32_to_bf16(th_o), "bf16 copy")


@pytest.mark.parametrize("flags_name", ["exact", "twophase", "noskip"])
@pytest.mark.parametrize("S", [131_075, 1_574_528])
def test_step_with_gradient_factor(fp, flags_name, S):
    """The fused step entry point with a loss-scale unscale factor set before
    the step, on each of its paths, against the oracle."""
    flags = {"exact": fp.FP_STEP_EXACT_SKIP, "twophase": fp.FP_STEP_NO_COOP,
             "noskip": fp.FP_STEP_NO_SKIP}[flags_name]
    world, rank, seed, L = 8, 3, 13, 4096.0
    say(f"step with factor path={flags_name} S={S}")
    grads = [gen.bf16_normal(S, 1e-3 * L, seed, gen.STREAM_GRAD, 0, q) for q in range(world)]
    th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER)
    others = [gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, q) for q in range(world)]
    coef_o = oracle.grad_coef(0.0, L, 0.0)
    acc_o = oracle.reduce(grads, np.float32(1.0 / world))
    th_o, m_o, v_o = th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    oracle.adamw(acc_o, th_o, m_o, v_o, step=1, coef=coef_o, **hp_kwargs(HP))
    full_o = oracle.unshard([oracle.f32_to_bf16(th_o) if q == rank else others[q] for q in range(world)])

    coef = torch.zeros(1, dtype=torch.float64, device=dev())
    fp.grad_coef(coef, loss_scale=torch.tensor([L], dtype=torch.float32, device=dev()))
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    d_th, d_m, d_v = to_dev(th), torch.zeros(S, dtype=torch.float32, device=dev()), \
        torch.zeros(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    shards = [to_dev(o) for o in others]
    shards[rank] = None
    call = fp.ShardStep([to_dev(x) for x in grads], acc, d_th, d_m, d_v, shards, full, rank,
                        scale=1.0 / world, found_inf=flag, workspace=fp.new_workspace(dev(), S), flags=flags,
                        grad_coef=coef, **hp_kwargs(HP))
    if flags_name == "exact":
        assert call.path() == fp.FP_PATH_ONE_PASS
    call(1)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    assert_f32_close(to_host(d_th), th_o, "master")
    assert_f32_close(to_host(d_m), m_o, "exp_avg")
    assert_f32_close(to_host(d_v), v_o, "exp_avg_sq")
    fh = to_host(full)
    own = slice(rank * S, (rank + 1) * S)
    assert_bf16_within_1ulp(fh[own], full_o[own], "own shard")


def test_units_step_with_gradient_factor(fp):
    """The multi-unit step with the factor: every unit's update uses it."""
    world, rank, seed, L = 4, 2, 17, 256.0
    sizes = [10_001, 4, 65_536, 3]
    say("units step with factor")
    grads = [[gen.bf16_normal(S, 1e-3 * L, seed, gen.STREAM_GRAD, u, q) for q in range(world)]
             for u, S in enumerate(sizes)]
    others = [[gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, u, q) for q in range(world)]
              for u, S in enumerate(sizes)]
    d_grads = [[to_dev(x) for x in row] for row in grads]
    d_shards = [[to_dev(x) if q != rank else None for q, x in enumerate(row)] for row in others]
    fulls = [torch.zeros(world * S, dtype=torch.int16, device=dev()) for S in sizes]
    units = fp.Units(d_grads, rank, d_shards, fulls)
    P = units.partition
    th = gen.normal_f32(P, 0.02, seed, gen.STREAM_MASTER)
    coef = torch.zeros(1, dtype=torch.float64, device=dev())
    fp.grad_coef(coef, loss_scale=torch.tensor([L], dtype=torch.float32, device=dev()))
    acc = torch.zeros(P, dtype=torch.float32, device=dev())
    d_th, d_m, d_v = to_dev(th), torch.zeros(P, dtype=torch.float32, device=dev()), \
        torch.zeros(P, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    units.step(acc, d_th, d_m, d_v, scale=1.0 / world, step=1, found_inf=flag, grad_coef=coef, **hp_kwargs(HP))
    torch.cuda.synchronize()
    got_th = to_host(d_th)
    for u, S in enumerate(sizes):
        o = units.offsets[u]
        acc_o = oracle.reduce(grads[u], np.float32(1.0 / world))
        th_o, m_o, v_o = th[o:o + S].copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
        oracle.adamw(acc_o, th_o, m_o, v_o, step=1, coef=1.0 / L, **hp_kwargs(HP))
        assert_f32_close(got_th[o:o + S], th_o, f"unit {u} master")
        own = to_host(fulls[u])[rank * S:(rank + 1) * S]
        assert_bf16_within_1ulp(own, oracle.f32_to_bf16(th_o), f"unit {u} own shard")


def test_no_sync_full_611m_unit(fp):
    """The 611M-parameter model's whole unit on one rank, 4 micro-batches
    accumulated without communication: the fp32 local sum after three and
    the exchanged bf16 row after the fourth, checked against the oracle at
    2^14 sampled positions (the oracle gets the gathered inputs)."""
    from workloads import CONFIGS
    cfg = CONFIGS["c3_611m_buckets_nd16"]
    n = sum(cfg.units())
    say(f"no_sync full unit n={n}")
    idx = torch.from_numpy(np.sort(np.random.default_rng(3).choice(n, 1 << 14, replace=False))).to(dev())
    local = torch.empty(n, dtype=torch.float32, device=dev())
    picked = []
    for m in range(cfg.n_micro):
        g = gen.torch_bf16_normal(n, cfg.grad_sigma, cfg.seed, (gen.STREAM_GRAD, m), dev())
        picked.append(g.index_select(0, idx).cpu().numpy().view(np.uint16))
        if m < cfg.n_micro - 1:
            fp.local_accumulate(g, local, accumulate=m > 0)
        else:
            out = torch.empty(n, dtype=torch.int16, device=dev())
            fp.local_finish(g, out, local, accumulate=True)
        del g
    torch.cuda.synchronize()
    loc_o = None
    for m in range(cfg.n_micro - 1):
        loc_o = oracle.local_accumulate(picked[m], loc_o, accumulate=m > 0)
    row_o = oracle.local_finish(picked[-1], loc_o, accumulate=True)
    assert_f32_bitexact(local.index_select(0, idx).cpu().numpy(), loc_o, "local sum")
    assert_bf16_equal(out.index_select(0, idx).cpu().numpy().view(np.uint16), row_o, "exchanged row")
