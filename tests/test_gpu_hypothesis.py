"""Property-based GPU parity: hypothesis draws small random cases and the
GPU must match the oracle on each.

* pack: random tensor counts, shapes (0-d, empty and ragged ones), 2- or
  4-byte elements with arbitrary bit patterns (NaN payloads, -0), N_d from
  1 to 64, bit for bit, plus every rank's views;
* reduce: N_d in {1, 2, 3, 8, 16, 64}, odd S, rows starting at odd element
  offsets, gradients drawn from a pool of bf16 specials (signed zeros,
  subnormals, the largest finite values, +-inf, NaN) mixed with normals,
  one or two micro-batches: bitwise, non-finite values by class;
* the shard step on the same kind of inputs (finite gradients whose sum may
  still overflow fp32), every path, in place or with separate output state;
* the multi-unit step: one to eight units of random sizes (empty, shorter
  than a quad, ragged, several workgroups), N_d up to 16, one to three
  micro-batches, rows at odd element offsets, an overflow in a random unit
  or none, in place or with separate output partitions, with or without the
  norm: every unit against the oracle's unit-by-unit step with one overflow
  decision for all.
Examples are derandomised (a fixed sequence per test) so that a failure
repeats; no example database is written.
"""

import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from gpu_common import (assert_bf16_equal, assert_bf16_within_1ulp, assert_f32_bitexact, assert_f32_close,
                        dev, hp_kwargs, to_dev, to_host)
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()
SETTINGS = settings(max_examples=60, deadline=None, database=None, derandomize=True,
                    suppress_health_check=list(HealthCheck))

SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80,
                     0x7F80, 0xFF80, 0x7FC0, 0xFFC1], dtype=np.uint16)
FINITE_SPECIALS = SPECIALS[:10]

shape_st = st.lists(st.integers(0, 9), min_size=0, max_size=3).map(tuple)


def _rows_at(host_rows, offset):
    out = []
    for h in host_rows:
        buf = torch.zeros(h.size + offset + 8, dtype=torch.int16, device=dev())
        v = buf[offset:offset + h.size]
        v.copy_(to_dev(h))
        out.append(v)
    return out


def _grads(r, world, S, specials, frac):
    rows = []
    for _ in range(world):
        x = (r.standard_normal(S) * 1e-2).astype(np.float32)
        h = (x.view(np.uint32) >> 16).astype(np.uint16)
        pick = r.random(S) < frac
        h[pick] = r.choice(specials, size=int(pick.sum()))
        rows.append(h)
    return rows


@SETTINGS
@given(shapes=st.lists(st.one_of(shape_st, st.tuples(st.integers(0, 5000))), min_size=1, max_size=12),
       world=st.sampled_from([1, 2, 3, 4, 7, 8, 64]), esize=st.sampled_from([2, 4]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_pack_matches_oracle(fp, shapes, world, esize, seed):
    r = np.random.default_rng(seed)
    dt = np.uint16 if esize == 2 else np.uint32
    host = [r.integers(0, 2 ** (8 * esize), size=math.prod(s), dtype=np.uint64).astype(dt).reshape(s)
            for s in shapes]
    want = oracle.pack(host, world)
    tdt = torch.int16 if esize == 2 else torch.int32
    dev_t = [torch.from_numpy(h.reshape(-1).view(np.int16 if esize == 2 else np.int32).copy()).to(dev())
             .view(s) for h, s in zip(host, shapes)]
    plan = fp.Plan(shapes, world)
    flat = plan.pack(dev_t)
    torch.cuda.synchronize()
    got = flat.cpu().numpy().view(dt)
    assert flat.dtype == tdt and np.array_equal(got, want)
    numel = [math.prod(s) for s in shapes]
    for q in range(world):
        bo, ln, to = oracle.views(numel, world, q)
        assert [v.numel() for v in plan.views(flat[q * plan.shard:(q + 1) * plan.shard], q)] == list(ln)
    plan.close()


@SETTINGS
@given(world=st.sampled_from([1, 2, 3, 8, 16, 64]), S=st.integers(1, 3000), offset=st.integers(0, 7),
       micro=st.integers(1, 2), frac=st.sampled_from([0.0, 0.05, 0.5]), seed=st.integers(0, 2 ** 31 - 1))
def test_reduce_matches_oracle(fp, world, S, offset, micro, frac, seed):
    r = np.random.default_rng(seed)
    scale = np.float32(1.0 / (world * micro))
    acc_o = np.zeros(S, np.float32)
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    for m in range(micro):
        rows = _grads(r, world, S, SPECIALS, frac)
        oracle.reduce(rows, scale, acc_o, accumulate=m > 0)
        fp.reduce_shard(_rows_at(rows, offset), acc, scale=float(scale), accumulate=m > 0, found_inf=flag)
    torch.cuda.synchronize()
    assert_f32_bitexact(to_host(acc), acc_o, "acc")
    assert int(flag.item()) == oracle.found_inf(acc_o)


@SETTINGS
@given(world=st.sampled_from([1, 2, 3, 8, 16]), S=st.integers(1, 5000), rank_frac=st.floats(0, 0.999),
       flags=st.sampled_from([0, 1, 4]), step=st.integers(1, 5), frac=st.sampled_from([0.0, 0.2]),
       out_of_place=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_step_matches_oracle(fp, world, S, rank_frac, flags, step, frac, out_of_place, seed):
    r = np.random.default_rng(seed)
    rank = int(rank_frac * world)
    rows = _grads(r, world, S, FINITE_SPECIALS, frac)
    others = _grads(r, world, S, FINITE_SPECIALS, 0.0)
    th = (r.standard_normal(S) * 0.02).astype(np.float32)
    m0 = (r.standard_normal(S) * 1e-4).astype(np.float32) if step > 1 else np.zeros(S, np.float32)
    v0 = ((r.standard_normal(S) * 1e-3) ** 2).astype(np.float32) if step > 1 else np.zeros(S, np.float32)
    acc_o, th_o, m_o, v_o = np.zeros(S, np.float32), th.copy(), m0.copy(), v0.copy()
    full_o, flag_o, _ = oracle.shard_step([rows], acc_o, th_o, m_o, v_o, others, rank, hp=HP, step=step)
    if flags & fp.FP_STEP_NO_SKIP and flag_o:      # no gate: the update runs on the overflowed values
        th_o, m_o, v_o = th.copy(), m0.copy(), v0.copy()
        oracle.adamw(acc_o, th_o, m_o, v_o, step=step, skip=False, **hp_kwargs(HP))
        full_o = full_o.copy()
        full_o[rank * S:(rank + 1) * S] = oracle.f32_to_bf16(th_o)

    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    d_th, d_m, d_v = to_dev(th), to_dev(m0), to_dev(v0)
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    ws = fp.new_workspace(dev(), S)
    shards = [None if q == rank else to_dev(others[q]) for q in range(world)]
    outs = [torch.full((S,), 9.0, dtype=torch.float32, device=dev()) for _ in range(3)] if out_of_place else None
    fp.shard_step(_rows_at(rows, 0), acc, d_th, d_m, d_v, shards, full, rank, scale=1.0 / world, step=step,
                  found_inf=flag, workspace=ws, flags=flags, out=outs, **hp_kwargs(HP))
    torch.cuda.synchronize()
    assert int(flag.item()) == flag_o
    res = (d_th, d_m, d_v)
    if out_of_place:
        for name, got, x in zip(("master", "exp_avg", "exp_avg_sq"), res, (th, m0, v0)):
            assert_f32_bitexact(to_host(got), x, f"input {name} unchanged")
        res = outs
    for name, got, want in zip(("master", "exp_avg", "exp_avg_sq"), res, (th_o, m_o, v_o)):
        if flag_o and not flags & fp.FP_STEP_NO_SKIP:
            assert_f32_bitexact(to_host(got), want, f"{name} untouched on overflow")
        else:
            assert_f32_close(to_host(got), want, name)
    fh = to_host(full)
    own = slice(rank * S, (rank + 1) * S)
    assert_bf16_within_1ulp(fh[own], full_o[own], "own shard")
    mask = np.ones(world * S, bool)
    mask[own] = False
    assert_bf16_equal(fh[mask], full_o[mask], "other shards")
    assert fp.workspace_timeouts(ws) == 0


@settings(max_examples=40, deadline=None, database=None, derandomize=True,
          suppress_health_check=list(HealthCheck))
@given(world=st.sampled_from([1, 2, 3, 8, 16]), sizes=st.lists(st.integers(0, 6000), min_size=1, max_size=8),
       rank_frac=st.floats(0, 0.999), n_micro=st.integers(1, 3), step=st.integers(1, 3),
       flags=st.sampled_from([0, 1, 2]), inf=st.booleans(), offset=st.integers(0, 7),
       out_of_place=st.booleans(), with_norm=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_units_match_oracle(fp, world, sizes, rank_frac, n_micro, step, flags, inf, offset, out_of_place,
                            with_norm, seed):
    from test_gpu_units import _units_case
    rank = int(rank_frac * world)
    inf_unit = seed % len(sizes) if inf else None
    _units_case(fp, sizes, world, rank, n_micro, step, seed % 100_000, flags, inf_unit=inf_unit, offset=offset,
                with_norm=with_norm, out_of_place=out_of_place)
