"""GPU parity of the multi-unit entry points (fp_units_*) against the oracle.

Several units (DDP buckets / FSDP units) of one rank are reduced, updated and
gathered with one launch per stage.  The oracle runs its single-unit routines
unit by unit and takes one overflow decision for the whole step, as the
definition requires: a non-finite value in any unit skips every unit's
update.  Sizes include empty units, units shorter than a quad, ragged tails
and units spanning several workgroups; gradient rows start at odd element
offsets in some cases (the realigning kernels).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (assert_bf16_equal, assert_bf16_within_1ulp, assert_f32_bitexact,
                        assert_f32_close, dev, hp_kwargs, say, to_dev, to_host, norm_rel_tol)
from workloads import gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()


def _rows(host_rows, offset):
    out = []
    for h in host_rows:
        buf = torch.zeros(h.size + offset + 8, dtype=torch.int16, device=dev())
        v = buf[offset:offset + h.size]
        v.copy_(to_dev(h))
        out.append(v)
    return out


def _units_case(fp, sizes, world, rank, n_micro, step, seed, flags, inf_unit=None, offset=0,
                with_norm=True, out_of_place=False, want_path=None):
    U = len(sizes)
    scale = np.float32(1.0 / (world * n_micro))
    micro = [[[gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, u, m, q) for q in range(world)]
              for u, S in enumerate(sizes)] for m in range(n_micro)]
    if inf_unit is not None and sizes[inf_unit] > 0:
        micro[-1][inf_unit][world - 1][sizes[inf_unit] // 2] = 0xFF80     # -inf
    th = [gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER, u) for u, S in enumerate(sizes)]
    m0 = [gen.normal_f32(S, 1e-4, seed, gen.STREAM_EXP_AVG, u) if step > 1 else np.zeros(S, np.float32)
          for u, S in enumerate(sizes)]
    v0 = [gen.normal_f32(S, 1e-3, seed, gen.STREAM_EXP_AVG_SQ, u) ** 2 if step > 1
          else np.zeros(S, np.float32) for u, S in enumerate(sizes)]
    others = [[gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, u, q) for q in range(world)]
              for u, S in enumerate(sizes)]

    # oracle: unit by unit, one overflow decision for the step
    acc_o = [np.zeros(S, np.float32) for S in sizes]
    for m in range(n_micro):
        for u in range(U):
            if sizes[u]:
                oracle.reduce(micro[m][u], scale, acc_o[u], accumulate=m > 0)
    flag_o = int(any(oracle.found_inf(a) for a in acc_o if a.size))
    norm_o = sum(oracle.sq_norm(a) for a in acc_o if a.size)
    skip = bool(flag_o) and not flags & fp.FP_STEP_NO_SKIP
    th_o, m_o, v_o = [x.copy() for x in th], [x.copy() for x in m0], [x.copy() for x in v0]
    full_o = []
    for u in range(U):
        if sizes[u]:
            oracle.adamw(acc_o[u], th_o[u], m_o[u], v_o[u], step=step, skip=skip, **hp_kwargs(HP))
        own = oracle.f32_to_bf16(th_o[u])
        full_o.append(oracle.unshard([own if q == rank else others[u][q] for q in range(world)])
                      if sizes[u] else np.zeros(0, np.uint16))

    # GPU
    grads_d = [[_rows(micro[m][u], offset) for u in range(U)] for m in range(n_micro)]
    shards_d = [[None if q == rank else to_dev(others[u][q]) for q in range(world)] for u in range(U)]
    full_d = [torch.zeros(max(1, world * S), dtype=torch.int16, device=dev()) for S in sizes]
    plans = [fp.Units(grads_d[m], rank, shards=shards_d, full=full_d) for m in range(n_micro)]
    P = plans[0].partition
    assert all(p.partition == P and p.offsets == plans[0].offsets for p in plans)
    offs = plans[0].offsets
    assert offs[0] == 0 and all(o % 4 == 0 for o in offs)
    acc = torch.zeros(P, dtype=torch.float32, device=dev())
    state = [torch.zeros(P, dtype=torch.float32, device=dev()) for _ in range(3)]
    for u in range(U):
        for t, h in zip(state, (th[u], m0[u], v0[u])):
            plans[0].unit_slice(t, u).copy_(to_dev(h))
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev()) if with_norm else None
    ws = plans[0].new_workspace() if with_norm else None
    out = None
    if out_of_place:
        state0 = [t.clone() for t in state]
        out = [torch.full((P,), 7.0, dtype=torch.float32, device=dev()) for _ in range(3)]
    if want_path is not None:
        assert plans[-1].step_path(acc, *state, found_inf=flag, flags=flags, out=out, sq_norm=sq,
                                   workspace=ws) == want_path
    for m in range(n_micro - 1):
        plans[m].reduce(acc, scale=float(scale), accumulate=m > 0, found_inf=flag)
    plans[-1].step(acc, *state, scale=float(scale), accumulate=n_micro > 1, step=step, found_inf=flag,
                   sq_norm=sq, workspace=ws, flags=flags, out=out, **hp_kwargs(HP))
    torch.cuda.synchronize()

    assert int(flag.item()) == flag_o
    if out_of_place:
        for t, t0 in zip(state, state0):
            assert torch.equal(t.view(torch.int32), t0.view(torch.int32)), "input state written"
        state = out
    for u in range(U):
        got = [to_host(plans[0].unit_slice(t, u)) for t in state]
        if skip:
            for g, w0 in zip(got, (th[u], m0[u], v0[u])):
                assert_f32_bitexact(g, w0, f"unit {u}: state must be untouched on overflow")
        else:
            for name, g, w in zip(("master", "exp_avg", "exp_avg_sq"), got, (th_o[u], m_o[u], v_o[u])):
                assert_f32_close(g, w, f"unit {u} {name}")
        S = sizes[u]
        fh = to_host(full_d[u])[:world * S]
        own = slice(rank * S, (rank + 1) * S)
        assert_bf16_within_1ulp(fh[own], full_o[u][own], f"unit {u} own shard")
        mask = np.ones(world * S, bool)
        mask[own] = False
        assert_bf16_equal(fh[mask], full_o[u][mask], f"unit {u} other shards")
        if flags & fp.FP_STEP_KEEP_GRAD or not (flags & fp.FP_STEP_NO_SKIP or out_of_place):
            assert_f32_bitexact(to_host(plans[0].unit_slice(acc, u)), acc_o[u], f"unit {u} reduced gradient")
    if with_norm and np.isfinite(norm_o):
        assert float(sq.item()) == pytest.approx(norm_o, rel=norm_rel_tol(sum(sizes)))
    for p in plans:
        p.close()


@pytest.mark.parametrize("flags", [0, 1, 3])
def test_units_small(fp, flags):
    say(f"units small flags={flags}")
    _units_case(fp, [12, 0, 3, 4, 29, 2049], world=2, rank=1, n_micro=1, step=1, seed=1, flags=flags)


@pytest.mark.parametrize("seed", range(8))
def test_units_random(fp, seed):
    r = np.random.default_rng(9000 + seed)
    world = int(r.choice([1, 2, 3, 8, 16]))
    U = int(r.integers(1, 9))
    sizes = [int(r.choice([0, 1, 5, 64, 1001, 2048 * 3 + 7, 20_000])) for _ in range(U)]
    rank = int(r.integers(0, world))
    n_micro = int(r.choice([1, 2, 4]))
    step = int(r.choice([1, 3]))
    flags = int(r.choice([0, 1, 2]))
    inf_unit = int(r.integers(0, U)) if seed % 3 == 2 else None
    offset = int(r.integers(1, 8)) if seed % 2 else 0
    say(f"units seed={seed} world={world} sizes={sizes} rank={rank} n_micro={n_micro} step={step} "
        f"flags={flags} inf_unit={inf_unit} offset={offset}")
    _units_case(fp, sizes, world, rank, n_micro, step, 300 + seed, flags, inf_unit=inf_unit,
                offset=offset)


def test_units_overflow_in_one_unit_skips_all(fp):
    say("units: overflow in the last unit skips every unit")
    _units_case(fp, [4096, 5000, 777], world=8, rank=3, n_micro=2, step=2, seed=7, flags=0, inf_unit=2)


def test_units_equal_single_unit_steps(fp):
    """Without overflow, the multi-unit step equals one fp_shard_step per unit, bitwise."""
    say("units vs per-unit shard steps")
    world, rank, sizes = 4, 2, [3000, 1024, 17]
    r = np.random.default_rng(5)
    grads = [[to_dev(gen.bf16_normal(S, 1e-3, 5, gen.STREAM_GRAD, u, 0, q)) for q in range(world)]
             for u, S in enumerate(sizes)]
    others = [[None if q == rank else to_dev(gen.bf16_normal(S, 0.02, 5, gen.STREAM_SHARD, u, q))
               for q in range(world)] for u, S in enumerate(sizes)]
    th = [to_dev(r.standard_normal(S).astype(np.float32) * 0.02) for S in sizes]
    full_a = [torch.zeros(world * S, dtype=torch.int16, device=dev()) for S in sizes]
    full_b = [torch.zeros(world * S, dtype=torch.int16, device=dev()) for S in sizes]
    plan = fp.Units(grads, rank, shards=others, full=full_a)
    P = plan.partition
    acc, m, v, master = (torch.zeros(P, dtype=torch.float32, device=dev()) for _ in range(4))
    for u in range(len(sizes)):
        plan.unit_slice(master, u).copy_(th[u])
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    plan.step(acc, master, m, v, scale=1.0 / world, step=1, found_inf=flag, **hp_kwargs(HP))
    for u, S in enumerate(sizes):
        a1, m1, v1 = (torch.zeros(S, dtype=torch.float32, device=dev()) for _ in range(3))
        t1 = th[u].clone()
        f1 = torch.zeros(1, dtype=torch.int32, device=dev())
        fp.shard_step(grads[u], a1, t1, m1, v1, others[u], full_b[u], rank, scale=1.0 / world, step=1,
                      found_inf=f1, flags=fp.FP_STEP_NO_COOP, **hp_kwargs(HP))
        torch.cuda.synchronize()
        assert torch.equal(plan.unit_slice(master, u).view(torch.int32), t1.view(torch.int32))
        assert torch.equal(plan.unit_slice(m, u).view(torch.int32), m1.view(torch.int32))
        assert torch.equal(plan.unit_slice(v, u).view(torch.int32), v1.view(torch.int32))
        assert torch.equal(full_a[u], full_b[u])
    plan.close()


@pytest.mark.parametrize("tail", [7_000, 20_480, 45_001])
def test_units_equal_buckets_with_a_tail(fp, tail):
    """Equal buckets plus a last one that is shorter, equal or longer (the
    workgroup-to-unit mapping by division), at 16 ranks and 4 micro-batches."""
    say(f"units equal buckets tail={tail}")
    _units_case(fp, [20_480] * 5 + [tail], world=16, rank=0, n_micro=4, step=2, seed=21, flags=0)


@pytest.mark.parametrize("flags", [0, 1, 2])
@pytest.mark.parametrize("inf_unit", [None, 4])
def test_units_speculative(fp, flags, inf_unit):
    """Separate output partitions: the fused launch writes every unit's update
    there, and with exact skip a last kernel restores the input state (and
    recasts every own slice) on overflow; the input partitions are only read."""
    say(f"units speculative flags={flags} inf_unit={inf_unit}")
    _units_case(fp, [12, 0, 3, 2049, 20_480, 777], world=8, rank=5, n_micro=2, step=3, seed=31, flags=flags,
                inf_unit=inf_unit, offset=1, out_of_place=True)


def test_units_speculative_equal_buckets_16_ranks(fp):
    say("units speculative: equal buckets, 16 ranks, 4 micro-batches")
    _units_case(fp, [20_480] * 5 + [45_001], world=16, rank=0, n_micro=4, step=2, seed=22, flags=0,
                out_of_place=True)


@pytest.mark.parametrize("mode", ["noskip", "speculative", "speculative_overflow"])
def test_units_split_launch(fp, mode):
    """Partitions of 2^24 elements and more: the fused reduce + AdamW launch and
    the copies of every unit's other shards in a launch of their own (odd unit
    sizes, so copy sources and units start off the 16-byte grid)."""
    say(f"units split launch: {mode}")
    sizes = [8_388_613, 8_388_611, 1001]
    if mode == "noskip":
        _units_case(fp, sizes, world=3, rank=1, n_micro=1, step=2, seed=41, flags=fp.FP_STEP_NO_SKIP,
                    want_path=fp.FP_PATH_NO_SKIP_SPLIT)
    else:
        _units_case(fp, sizes, world=3, rank=1, n_micro=2, step=2, seed=42, flags=0, out_of_place=True,
                    inf_unit=1 if mode == "speculative_overflow" else None, want_path=fp.FP_PATH_SPECULATIVE_SPLIT)
