"""Invariants of the device entry points that hold whatever the values.

* Guard bands: every output buffer sits inside a larger allocation whose
  bytes before and after it hold a canary pattern; after the call the
  canaries must be intact (no write outside the output), for ragged sizes
  and, where the ABI allows it, outputs starting at odd element offsets.
* Paths agree: the one-pass, two-phase and fused no-skip shard steps (and
  the multi-unit step against the single-unit one) compute the same
  arithmetic, so on overflow-free inputs their master / moments, reduced
  gradient and full bf16 buffer are bitwise equal; only the gradient norm's
  summation tree depends on the grid (compared to 1e-12 relative).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import assert_f32_close, dev, hp_kwargs, say, to_dev, to_host
from workloads import gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()
CANARY = 0x5A
GUARD = 4096                                   # bytes of canary on each side


class Guarded:
    """An n-element view `off` elements into a canary-filled allocation."""

    def __init__(self, n, dtype, off=0, init=None):
        esize = torch.empty(0, dtype=dtype).element_size()
        g = GUARD // esize
        self.buf = torch.empty(g + off + n + g, dtype=dtype, device=dev())
        self.buf.view(torch.uint8).fill_(CANARY)
        self.lo, self.n = g + off, n
        self.view = self.buf[self.lo:self.lo + n]
        if init is not None:
            self.view.copy_(init)

    def intact(self):
        b = self.buf.view(torch.uint8)
        es = self.buf.element_size()
        lo, hi = self.lo * es, (self.lo + self.n) * es
        return bool((b[:lo] == CANARY).all()) and bool((b[hi:] == CANARY).all())


def _check(*gs):
    torch.cuda.synchronize()
    for i, g in enumerate(gs):
        assert g.intact(), f"output {i} was written outside its range"


def _rows(world, S, seed, sigma=1e-3):
    """The ranks' bf16 rows, each in its own allocation (never empty, so that a
    zero-length row still has an address)."""
    out = []
    for q in range(world):
        buf = torch.zeros(S + 8, dtype=torch.int16, device=dev())
        buf[:S].copy_(to_dev(gen.bf16_normal(S, sigma, seed, gen.STREAM_GRAD, 0, 0, q)))
        out.append(buf[:S])
    return out


SIZES = [1, 3, 4, 7, 1023, 1025, 4097, 100_003]


@pytest.mark.parametrize("S", SIZES)
def test_guards_reduce_and_adamw(fp, S):
    say(f"guards: reduce / hybrid / adamw S={S}")
    grads = _rows(4, S, S)
    for acc_mode in (False, True):
        acc = Guarded(S, torch.float32, init=torch.ones(S, device=dev()))
        sq = Guarded(1, torch.float64)
        ws = Guarded(fp.workspace_bytes(S), torch.uint8, init=torch.zeros(fp.workspace_bytes(S), dtype=torch.uint8,
                                                                            device=dev()))
        flag = Guarded(1, torch.int32, init=torch.zeros(1, dtype=torch.int32, device=dev()))
        fp.reduce_shard(grads, acc.view, scale=0.25, accumulate=acc_mode, found_inf=flag.view, sq_norm=sq.view,
                        workspace=ws.view)
        _check(acc, sq, ws, flag)
        fp.reduce_shard_hybrid(grads, acc.view, group=2, scale=0.25, accumulate=acc_mode, found_inf=flag.view,
                               sq_norm=sq.view, workspace=ws.view)
        _check(acc, sq, ws, flag)
    g = torch.randn(S, device=dev()) * 1e-3
    for off in (0, 1, 3):
        th = Guarded(S, torch.float32, init=torch.randn(S, device=dev()) * 0.02)
        m = Guarded(S, torch.float32, init=torch.zeros(S, device=dev()))
        v = Guarded(S, torch.float32, init=torch.zeros(S, device=dev()))
        out = Guarded(S, torch.int16, off=off)
        fp.adamw_shard(g, th.view, m.view, v.view, step=1, param_bf16=out.view, **hp_kwargs(HP))
        _check(th, m, v, out)


@pytest.mark.parametrize("S,world,off", [(1, 2, 0), (5, 3, 1), (4097, 8, 3), (100_003, 5, 6), (65_536, 16, 0)])
def test_guards_unshard_and_local(fp, S, world, off):
    say(f"guards: unshard / no_sync S={S} world={world} offset={off}")
    shards = _rows(world, S, 7 + S)
    full = Guarded(world * S, torch.int16, off=off)
    fp.unshard(shards, full.view)
    _check(full)
    assert torch.equal(full.view.view(world, S), torch.stack(shards))
    local = Guarded(S, torch.float32)
    fp.local_accumulate(shards[0], local.view, accumulate=False)
    fp.local_accumulate(shards[1], local.view, accumulate=True)
    out = Guarded(S, torch.int16, off=off)
    fp.local_finish(shards[-1], out.view, local.view, accumulate=True)
    _check(local, out)


def test_guards_scalars(fp):
    say("guards: grad coef / scaler update")
    coef = Guarded(1, torch.float64)
    sq = torch.tensor([4.0], dtype=torch.float64, device=dev())
    ls = torch.tensor([2.0], dtype=torch.float32, device=dev())
    fp.grad_coef(coef.view, sq_norm=sq, loss_scale=ls, max_norm=0.5)
    scale = Guarded(1, torch.float32, init=torch.tensor([1024.0], device=dev()))
    count = Guarded(1, torch.int32, init=torch.tensor([3], dtype=torch.int32, device=dev()))
    fi = torch.zeros(1, dtype=torch.int32, device=dev())
    fp.scaler_update(fi, scale.view, count.view, growth_interval=10)
    _check(coef, scale, count)
    assert int(count.view.item()) == 4


@pytest.mark.parametrize("esize", [2, 4])
def test_guards_pack_dim0_reshard(fp, esize):
    say(f"guards: pack / dim-0 / reshard, element size {esize}")
    dtype = torch.int16 if esize == 2 else torch.float32
    shapes = [(37, 5), (4096,), (), (3, 3, 3), (1,), (0, 4), (10_001,)]
    world = 7
    tensors = [(torch.arange(int(np.prod(s)), device=dev()) % 1000).to(dtype).view(s) for s in shapes]
    plan = fp.Plan(shapes, world)
    flat = Guarded(plan.padded, dtype)           # fp32 flat: 16-byte aligned, as required
    plan.pack(tensors, flat.view)
    _check(flat)
    d0 = fp.Shard0Plan(shapes, world)
    for rank, off in ((-1, 1), (0, 3), (world - 1, 0)):
        n = d0.shard * (world if rank < 0 else 1)
        dst = Guarded(n, dtype, off=off)
        d0.pack(tensors, dst.view, rank=rank)
        _check(dst)
    gathered = d0.pack(tensors)
    params = [Guarded(int(np.prod(s)), dtype, off=i % 4) for i, s in enumerate(shapes)]
    d0.unpack(gathered, [p.view.view(s) for p, s in zip(params, shapes)])
    _check(*params)
    for p, t in zip(params, tensors):
        assert torch.equal(p.view, t.reshape(-1))
    T = plan.numel
    rs = fp.ReshardPlan(T, world, 3)
    old = [flat.view[q * plan.shard:(q + 1) * plan.shard] for q in range(world)]
    for rank, off in ((-1, 1), (2, 5)):
        n = rs.shard_new * (3 if rank < 0 else 1)
        dst = Guarded(n, dtype, off=off)
        rs.reshard(old, dst.view, rank=rank)
        _check(dst)
    for p in (plan, d0, rs):
        p.close()


def _step_buffers(world, S, rank, seed, full_off):
    grads = _rows(world, S, seed)
    others = _rows(world, S, seed + 1, 0.02)
    th = torch.randn(S, device=dev()) * 0.02
    m = torch.randn(S, device=dev()) * 1e-4
    v = (torch.randn(S, device=dev()) * 1e-3) ** 2
    shards = [None if q == rank else others[q] for q in range(world)]
    out = dict(acc=Guarded(S, torch.float32), th=Guarded(S, torch.float32, init=th),
               m=Guarded(S, torch.float32, init=m), v=Guarded(S, torch.float32, init=v),
               full=Guarded(world * S, torch.int16, off=full_off), sq=Guarded(1, torch.float64),
               flag=Guarded(1, torch.int32, init=torch.zeros(1, dtype=torch.int32, device=dev())))
    return grads, shards, out


@pytest.mark.parametrize("world,S,rank,full_off", [(8, 1_574_528, 1, 0), (3, 100_003, 2, 3), (5, 4097, 0, 1),
                                                   (2, 3, 1, 0)])
def test_step_paths_agree_and_stay_in_bounds(fp, world, S, rank, full_off):
    say(f"paths agree + guards: world={world} S={S} rank={rank} full offset={full_off}")
    results = {}
    for name, flags in (("one-pass", 0), ("two-phase", fp.FP_STEP_NO_COOP), ("no-skip", fp.FP_STEP_NO_SKIP)):
        torch.manual_seed(5)
        grads, shards, b = _step_buffers(world, S, rank, 60, full_off)
        ws = Guarded(fp.workspace_bytes(S), torch.uint8,
                     init=torch.zeros(fp.workspace_bytes(S), dtype=torch.uint8, device=dev()))
        call = fp.ShardStep(grads, b["acc"].view, b["th"].view, b["m"].view, b["v"].view, shards, b["full"].view,
                            rank, scale=1.0 / world, found_inf=b["flag"].view, sq_norm=b["sq"].view,
                            workspace=ws.view, flags=flags | fp.FP_STEP_KEEP_GRAD, **hp_kwargs(HP))
        if name == "one-pass" and S > 3:
            assert call.path() == fp.FP_PATH_ONE_PASS
        call(3)
        _check(*b.values(), ws)
        assert int(b["flag"].view.item()) == 0
        results[name] = {k: g.view.clone() for k, g in b.items()}
    ref = results["one-pass"]
    for name in ("two-phase", "no-skip"):
        for k in ("acc", "th", "m", "v", "full", "flag"):
            assert torch.equal(results[name][k].view(torch.uint8), ref[k].view(torch.uint8)), f"{name}: {k}"
        assert float(results[name]["sq"].item()) == pytest.approx(float(ref["sq"].item()), rel=1e-12)
    # the reduced gradient against the oracle (bitwise), as an anchor
    rows = [to_host(g) for g in _rows(world, S, 60)]
    acc_o = oracle.reduce(rows, np.float32(1.0 / world))
    np.testing.assert_array_equal(to_host(ref["acc"]).view(np.uint32), acc_o.view(np.uint32))


def test_units_step_equals_single_unit_steps(fp):
    """Each unit of a multi-unit step ends bitwise where a single-unit step of
    the same unit does, in both skip modes (no overflow), with guard bands
    around the partition state and every unit's full buffer."""
    sizes, world, rank = [4097, 1, 100_003, 0, 65_536], 4, 3
    say(f"units vs single steps: sizes={sizes}")
    torch.manual_seed(9)
    grads = [_rows(world, S, 300 + u) for u, S in enumerate(sizes)]
    others = [[None if q == rank else r for q, r in enumerate(_rows(world, S, 400 + u, 0.02))]
              for u, S in enumerate(sizes)]
    th0 = [torch.randn(S, device=dev()) * 0.02 for S in sizes]
    for flags in (0, fp.FP_STEP_NO_SKIP):
        fulls = [Guarded(max(1, world * S), torch.int16, off=u % 3) for u, S in enumerate(sizes)]
        plan = fp.Units(grads, rank, shards=others, full=[f.view for f in fulls])
        P = plan.partition
        state = [Guarded(P, torch.float32, init=torch.zeros(P, device=dev())) for _ in range(4)]
        for u in range(len(sizes)):
            plan.unit_slice(state[1].view, u).copy_(th0[u])
        flag = torch.zeros(1, dtype=torch.int32, device=dev())
        plan.step(state[0].view, state[1].view, state[2].view, state[3].view, scale=1.0 / world, step=1,
                  found_inf=flag, flags=flags | fp.FP_STEP_KEEP_GRAD, **hp_kwargs(HP))
        _check(*state, *fulls)
        for u, S in enumerate(sizes):
            if S == 0:
                continue
            acc = torch.zeros(S, device=dev())
            th, m, v = th0[u].clone(), torch.zeros(S, device=dev()), torch.zeros(S, device=dev())
            full = torch.zeros(world * S, dtype=torch.int16, device=dev())
            f1 = torch.zeros(1, dtype=torch.int32, device=dev())
            fp.shard_step(grads[u], acc, th, m, v, others[u], full, rank, scale=1.0 / world, step=1,
                          found_inf=f1, flags=flags | fp.FP_STEP_KEEP_GRAD, **hp_kwargs(HP))
            torch.cuda.synchronize()
            for name, got, want in (("acc", state[0], acc), ("master", state[1], th), ("exp_avg", state[2], m),
                                    ("exp_avg_sq", state[3], v)):
                g = plan.unit_slice(got.view, u)
                assert torch.equal(g.view(torch.int32), want.view(torch.int32)), f"unit {u} {name}"
            assert torch.equal(fulls[u].view[:world * S], full), f"unit {u} full"
        # the anchor: unit 2's master against the oracle
        S = sizes[2]
        acc_o = oracle.reduce([to_host(r) for r in grads[2]], np.float32(1.0 / world))
        th_o = to_host(th0[2]).copy()
        m_o, v_o = np.zeros(S, np.float32), np.zeros(S, np.float32)
        oracle.adamw(acc_o, th_o, m_o, v_o, step=1, skip=False, **hp_kwargs(HP))
        assert_f32_close(to_host(plan.unit_slice(state[1].view, 2)), th_o, "unit 2 master")
        plan.close()


@pytest.mark.parametrize("world,rank,full_off", [(8, 3, 0), (3, 1, 1)])
def test_split_no_skip_step_at_large_shards(fp, world, rank, full_off):
    """From 2^24 elements on, the no-skip step runs the fused reduce + AdamW +
    cast at reduced occupancy and the copies in a launch of their own: on
    overflow-free inputs it ends bitwise where the two-phase exact-skip step
    does, writes nothing outside its outputs, and its reduced gradient matches
    the oracle at sampled positions."""
    S = (1 << 24) + 3 if world > 4 else (1 << 26) + 3
    say(f"split no-skip vs two-phase: world={world} S={S} rank={rank} full offset={full_off}")
    grads = [gen.torch_bf16_normal(S, 1e-3, 70, (gen.STREAM_GRAD, q), dev()) for q in range(world)]
    others = [gen.torch_bf16_normal(S, 0.02, 70, (gen.STREAM_SHARD, q), dev()) for q in range(world)]
    shards = [None if q == rank else others[q] for q in range(world)]
    th0 = gen.torch_normal_f32(S, 0.02, 70, (gen.STREAM_MASTER,), dev())
    m0 = gen.torch_normal_f32(S, 1e-4, 70, (gen.STREAM_EXP_AVG,), dev())
    v0 = gen.torch_normal_f32(S, 1e-3, 70, (gen.STREAM_EXP_AVG_SQ,), dev()).square()
    results = {}
    for name, flags, want in (("split", fp.FP_STEP_NO_SKIP, fp.FP_PATH_NO_SKIP_SPLIT),
                              ("two-phase", fp.FP_STEP_NO_COOP, fp.FP_PATH_TWO_PHASE)):
        b = dict(acc=Guarded(S, torch.float32), th=Guarded(S, torch.float32, init=th0),
                 m=Guarded(S, torch.float32, init=m0), v=Guarded(S, torch.float32, init=v0),
                 full=Guarded(world * S, torch.int16, off=full_off), sq=Guarded(1, torch.float64),
                 flag=Guarded(1, torch.int32, init=torch.zeros(1, dtype=torch.int32, device=dev())))
        ws = Guarded(fp.workspace_bytes(S), torch.uint8,
                     init=torch.zeros(fp.workspace_bytes(S), dtype=torch.uint8, device=dev()))
        call = fp.ShardStep(grads, b["acc"].view, b["th"].view, b["m"].view, b["v"].view, shards, b["full"].view,
                            rank, scale=1.0 / world, found_inf=b["flag"].view, sq_norm=b["sq"].view,
                            workspace=ws.view, flags=flags | fp.FP_STEP_KEEP_GRAD, **hp_kwargs(HP))
        assert call.path() == want
        call(2)
        _check(*b.values(), ws)
        assert int(b["flag"].view.item()) == 0
        results[name] = {k: g.view.clone() for k, g in b.items()}
        del b, ws, call
        torch.cuda.empty_cache()
    for k in ("acc", "th", "m", "v", "full", "flag"):
        assert torch.equal(results["split"][k].view(torch.uint8), results["two-phase"][k].view(torch.uint8)), k
    assert float(results["split"]["sq"].item()) == pytest.approx(float(results["two-phase"]["sq"].item()), rel=1e-12)
    idx = torch.from_numpy(np.sort(np.random.default_rng(3).choice(S, 1 << 12, replace=False))).to(dev())
    rows = [to_host(g.index_select(0, idx)) for g in grads]
    want = oracle.reduce(rows, np.float32(1.0 / world))
    got = to_host(results["split"]["acc"].index_select(0, idx))
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("world,S,rank,full_off,overflow", [(3, 300_001, 1, 1, False), (8, 4_099, 7, 0, True),
                                                            (1, 7, 0, 3, True), (8, (1 << 24) + 1, 2, 1, True)])
def test_speculative_step_writes_only_its_outputs(fp, world, S, rank, full_off, overflow):
    """The speculative step (separate output state), on the one-pass kernel and
    as the fused pass plus restore kernel, writes only the output state, full
    and the flag / norm, leaves its input state unchanged, and ends bitwise
    where the in-place two-phase step does, overflowed or not."""
    say(f"speculative guard bands: world={world} S={S} rank={rank} full offset={full_off} overflow={overflow}")
    grads = [gen.torch_bf16_normal(S, 1e-3, 75, (gen.STREAM_GRAD, q), dev()) for q in range(world)]
    if overflow:
        grads[world - 1][S // 2] = 0x7F80
    others = [gen.torch_bf16_normal(S, 0.02, 75, (gen.STREAM_SHARD, q), dev()) for q in range(world)]
    shards = [None if q == rank else others[q] for q in range(world)]
    init = [gen.torch_normal_f32(S, 0.02, 75, (gen.STREAM_MASTER,), dev()),
            gen.torch_normal_f32(S, 1e-4, 75, (gen.STREAM_EXP_AVG,), dev()),
            gen.torch_normal_f32(S, 1e-3, 75, (gen.STREAM_EXP_AVG_SQ,), dev()).square()]
    results = {}
    fused = fp.FP_PATH_SPECULATIVE_SPLIT if S >= 1 << 24 else fp.FP_PATH_SPECULATIVE
    modes = {"speculative-one-pass": (fp.FP_STEP_EXACT_SKIP, fp.FP_PATH_SPECULATIVE_ONE_PASS if S <= 2_000_000
                                      else fused),
             "speculative": (fp.FP_STEP_EXACT_SKIP | fp.FP_STEP_NO_COOP, fused),
             "two-phase": (fp.FP_STEP_NO_COOP, fp.FP_PATH_TWO_PHASE)}
    for name, (flags, want_path) in modes.items():
        st = [Guarded(S, torch.float32, init=t) for t in init]
        out = [Guarded(S, torch.float32, init=torch.full((S,), 5.0, device=dev())) for _ in range(3)]
        b = dict(acc=Guarded(S, torch.float32), full=Guarded(world * S, torch.int16, off=full_off),
                 sq=Guarded(1, torch.float64),
                 flag=Guarded(1, torch.int32, init=torch.zeros(1, dtype=torch.int32, device=dev())))
        ws = Guarded(fp.workspace_bytes(S), torch.uint8,
                     init=torch.zeros(fp.workspace_bytes(S), dtype=torch.uint8, device=dev()))
        spec = name != "two-phase"
        call = fp.ShardStep(grads, b["acc"].view, *[g.view for g in st], shards, b["full"].view, rank,
                            scale=1.0 / world, found_inf=b["flag"].view, sq_norm=b["sq"].view, workspace=ws.view,
                            flags=flags, out=[g.view for g in out] if spec else None, **hp_kwargs(HP))
        assert call.path() == want_path
        call(3)
        _check(*st, *out, *b.values(), ws)
        assert int(b["flag"].view.item()) == (1 if overflow else 0)
        if spec:
            for g, t in zip(st, init):
                assert torch.equal(g.view.view(torch.uint8), t.view(torch.uint8)), "input state changed"
        results[name] = [g.view.clone() for g in (out if spec else st)] + [b["full"].view.clone()]
        del st, out, b, ws, call
        torch.cuda.empty_cache()
    for name in ("speculative-one-pass", "speculative"):
        for i, (x, y) in enumerate(zip(results[name], results["two-phase"])):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{name}: buffer {i} differs"
