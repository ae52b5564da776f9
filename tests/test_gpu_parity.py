"""GPU parity of every entry point against the CPU oracle on small, ragged cases.

Sizes span several 8-element chunks, several workgroups and a ragged tail;
world sizes cover 1, odd, powers of two and the 128-rank maximum; pointers
are deliberately misaligned (slices at odd offsets); payloads include NaN,
+-inf, -0 and subnormals.  The bar: pack / unshard / views and the
fixed-order reduce bitwise (non-finite floats by class), AdamW fp32 state
within 1e-6 rel / 1e-9 abs, bf16 parameters within 1 ulp.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (assert_bf16_equal, assert_bf16_within_1ulp, assert_f32_bitexact,
                        assert_f32_close, dev, hp_kwargs, say, to_dev, to_host, norm_rel_tol)
from workloads import CONFIGS, gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()


def _special_bf16(r, n):
    """bf16 patterns that stress the reduce: signed zeros, subnormals, extremes."""
    pool = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80],
                    dtype=np.uint16)
    return pool[r.integers(0, pool.size, size=n)]


def _grads_with_offset(host_rows, offset):
    """Device copies of the rows, each starting `offset` elements into its own buffer."""
    out = []
    for h in host_rows:
        buf = torch.zeros(h.size + offset + 8, dtype=torch.int16, device=dev())
        v = buf[offset:offset + h.size]
        v.copy_(to_dev(h))
        out.append(v)
    return out


# ------------------------------------------------------------------ reduce
@pytest.mark.parametrize("seed", range(24))
def test_reduce_random(fp, seed):
    r = np.random.default_rng(1000 + seed)
    world = int(r.choice([1, 2, 3, 5, 8, 16, 33, 64, 128]))
    S = int(r.choice([0, 1, 7, 8, 9, 63, 2048, 2049, 4095 + 8 * int(r.integers(0, 500))]))
    n_micro = int(r.integers(1, 4))
    offset = int(r.integers(0, 8)) if seed % 3 else 0
    say(f"reduce seed={seed} world={world} S={S} n_micro={n_micro} offset={offset}")
    scale = np.float32(1.0 / (world * n_micro))
    acc_o = np.zeros(S, np.float32)
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    ws = fp.new_workspace(dev(), S)
    for m in range(n_micro):
        rows = [gen.bf16_normal(S, 10.0 ** -int(r.integers(0, 4)), seed, gen.STREAM_GRAD, 0, m, q)
                for q in range(world)]
        if seed % 4 == 1 and S:
            for q in range(world):
                idx = r.integers(0, S, size=max(1, S // 10))
                rows[q][idx] = _special_bf16(r, idx.size)
        oracle.reduce(rows, scale, acc_o, accumulate=m > 0)
        grads = _grads_with_offset(rows, offset) if offset else to_dev(np.stack(rows)) if S else \
            [torch.zeros(0, dtype=torch.int16, device=dev())] * world
        fp.reduce_shard(grads, acc, scale=float(scale), accumulate=m > 0, found_inf=flag,
                        sq_norm=sq if m == n_micro - 1 else None, workspace=ws)
    torch.cuda.synchronize()
    assert_f32_bitexact(to_host(acc), acc_o, "acc")
    assert int(flag.item()) == oracle.found_inf(acc_o)
    want = oracle.sq_norm(acc_o)
    got = float(sq.item())
    if math.isfinite(want):
        assert got == pytest.approx(want, rel=1e-12, abs=0)
    else:
        assert not math.isfinite(got)


def test_reduce_nonfinite_cases(fp):
    say("reduce non-finite cases")
    fin = np.array([0x3F80, 0xC000, 0x3F00] * 5, dtype=np.uint16)   # 1, -2, 0.5
    cases = []
    a = fin.copy(); a[1] = 0x7F80; cases.append([a, fin])                 # +inf
    b = fin.copy(); b[1] = 0xFF80; cases.append([a, b])                   # inf - inf = NaN
    c = fin.copy(); c[14] = 0x7FC1; cases.append([fin, c])                # NaN in the tail
    big = np.full(15, 0x7F7F, np.uint16); cases.append([big, big])         # fp32 sum overflow
    cases.append([fin, fin])                                               # finite
    for rows in cases:
        acc_o = oracle.reduce(rows, np.float32(0.5))
        acc = torch.zeros(15, dtype=torch.float32, device=dev())
        flag = torch.zeros(1, dtype=torch.int32, device=dev())
        fp.reduce_shard(to_dev(np.stack(rows)), acc, scale=0.5, found_inf=flag)
        torch.cuda.synchronize()
        assert_f32_bitexact(to_host(acc), acc_o, "acc")
        assert int(flag.item()) == oracle.found_inf(acc_o)


# ------------------------------------------------------------------ AdamW + cast
@pytest.mark.parametrize("seed", range(16))
def test_adamw_random(fp, seed):
    r = np.random.default_rng(2000 + seed)
    S = int(r.choice([1, 5, 8, 17, 1000, 8 * 4096 + 3, 100_003]))
    step = int(r.choice([1, 2, 3, 10, 1000]))
    scale = float(r.choice([1.0, 1e-3, 3e-5]))
    skip = seed % 5 == 4
    out_off = int(r.integers(0, 8))
    say(f"adamw seed={seed} S={S} step={step} scale={scale} skip={skip} out_offset={out_off}")
    g = gen.normal_f32(S, scale, seed, gen.STREAM_GRAD)
    th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER)
    m = gen.normal_f32(S, scale * 0.3, seed, gen.STREAM_EXP_AVG) if step > 1 else np.zeros(S, np.float32)
    v = (gen.normal_f32(S, scale, seed, gen.STREAM_EXP_AVG_SQ) ** 2 if step > 1
         else np.zeros(S, np.float32))
    if seed % 4 == 3:
        th[: S // 3] = 0.0
        g[: S // 5] = 0.0
    th_o, m_o, v_o = th.copy(), m.copy(), v.copy()
    oracle.adamw(g, th_o, m_o, v_o, step=step, skip=skip, **hp_kwargs(HP))
    want_bf16 = oracle.f32_to_bf16(th_o)

    d_th, d_m, d_v = to_dev(th), to_dev(m), to_dev(v)
    flag = torch.tensor([1 if skip else 0], dtype=torch.int32, device=dev())
    out_buf = torch.zeros(S + 16, dtype=torch.int16, device=dev())
    out = out_buf[out_off:out_off + S]
    fp.adamw_shard(to_dev(g), d_th, d_m, d_v, step=step, found_inf=flag, param_bf16=out, **hp_kwargs(HP))
    torch.cuda.synchronize()
    for name, got, want in (("master", d_th, th_o), ("exp_avg", d_m, m_o), ("exp_avg_sq", d_v, v_o)):
        gh = to_host(got)
        if skip:
            assert_f32_bitexact(gh, want, name)
        else:
            assert_f32_close(gh, want, name)
    assert_bf16_within_1ulp(to_host(out), want_bf16, "param_bf16")
    guard = to_host(out_buf)
    assert not guard[:out_off].any() and not guard[out_off + S:].any(), "wrote outside param_bf16"


def test_cast_every_upper_half(fp):
    """bf16 rounding of 65536 x 16 fp32 patterns (every sign / exponent / upper
    mantissa with each class of dropped bits), through fp_adamw_shard with the
    update skipped, so the output is exactly the cast of the input."""
    say("cast dense")
    upper = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lowers = [0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF, 0x1234, 0x8765,
              0x7FFE, 0x8002, 0x4000, 0x0100, 0xFF00, 0xABCD]
    x = np.concatenate([(upper | np.uint32(lo)).view(np.float32) for lo in lowers])
    z = np.zeros_like(x)
    d_x = to_dev(x)
    out = torch.zeros(x.size, dtype=torch.int16, device=dev())
    flag = torch.ones(1, dtype=torch.int32, device=dev())
    fp.adamw_shard(to_dev(z), d_x, to_dev(z), to_dev(z), step=1, found_inf=flag, param_bf16=out,
                   **hp_kwargs(HP))
    torch.cuda.synchronize()
    assert_bf16_equal(to_host(out), oracle.f32_to_bf16(x), "bf16 cast")
    assert_f32_bitexact(to_host(d_x), x, "master untouched on skip")


# ------------------------------------------------------------------ unshard
@pytest.mark.parametrize("seed", range(12))
def test_unshard_random(fp, seed):
    r = np.random.default_rng(3000 + seed)
    world = int(r.choice([1, 2, 3, 7, 8, 64, 128]))
    S = int(r.choice([1, 3, 8, 13, 1000, 2049, 65_541]))
    full_off = int(r.integers(0, 8))
    skip_q = int(r.integers(0, world)) if seed % 2 else -1
    say(f"unshard seed={seed} world={world} S={S} full_offset={full_off} skip={skip_q}")
    shards = [gen.bf16_normal(S, 1.0, seed, gen.STREAM_SHARD, q) for q in range(world)]
    full_buf = torch.full((world * S + 16,), -1, dtype=torch.int16, device=dev())
    full = full_buf[full_off:full_off + world * S]
    d = _grads_with_offset(shards, int(r.integers(0, 8)))
    if skip_q >= 0:
        d[skip_q] = None
    fp.unshard(d, full)
    torch.cuda.synchronize()
    want = oracle.unshard(shards)
    if skip_q >= 0:
        want[skip_q * S:(skip_q + 1) * S] = 0xFFFF
    assert_bf16_equal(to_host(full), want, "full")
    h = to_host(full_buf)
    assert np.all(h[:full_off] == 0xFFFF) and np.all(h[full_off + world * S:] == 0xFFFF)


# ------------------------------------------------------------------ pack + views
@pytest.mark.parametrize("seed", range(16))
def test_pack_random(fp, seed):
    r = np.random.default_rng(4000 + seed)
    n_t = int(r.integers(1, 40))
    shapes = []
    for _ in range(n_t):
        k = int(r.integers(0, 4))
        shapes.append(tuple(int(x) for x in r.integers(0 if r.random() < 0.1 else 1, 40, size=k)))
    if seed % 4 == 0:
        shapes.append((9000,))            # spans two pack workgroups
    world = int(r.choice([1, 2, 3, 8, 64, 1000]))
    dtype = np.float32 if seed % 2 == 0 else np.uint16
    say(f"pack seed={seed} tensors={len(shapes)} world={world} dtype={np.dtype(dtype).name}")
    host = []
    for i, s in enumerate(shapes):
        x = gen.normal_f32(math.prod(s), 1.0, seed, gen.STREAM_TENSOR, i)
        if seed % 3 == 0 and x.size:
            x[0] = np.float32("nan")
            x.view(np.uint32)[-1] = 0x80000000
        host.append((x if dtype == np.float32 else gen.bf16_bits_trunc(x)).reshape(s))
    # sources at odd element offsets inside larger buffers
    srcs = []
    for h in host:
        off = int(r.integers(0, 4))
        buf = torch.zeros(h.size + off + 4, dtype=torch.float32 if dtype == np.float32 else torch.int16,
                          device=dev())
        v = buf[off:off + h.size]
        v.copy_(to_dev(h.reshape(-1)))
        srcs.append(v.view(h.shape))
    plan = fp.Plan(shapes, world)
    flat = plan.pack(srcs)
    torch.cuda.synchronize()
    want = oracle.pack(host, world)
    got = to_host(flat)
    assert got.view(np.uint8).tobytes() == want.view(np.uint8).tobytes()
    for h, v in zip(host, plan.views(flat, -1)):
        assert tuple(v.shape) == h.shape
        assert to_host(v).reshape(-1).view(np.uint8).tobytes() == np.ascontiguousarray(h).reshape(-1).view(np.uint8).tobytes()
    S = plan.shard
    numel = [math.prod(s) for s in shapes]
    for q in sorted(set([0, world - 1, int(r.integers(0, world))])):
        shard = flat[q * S:(q + 1) * S]
        bo, ln, to = oracle.views(numel, world, q)
        for i, v in enumerate(plan.views(shard, q)):
            assert v.numel() == ln[i]
            if ln[i]:
                assert np.array_equal(to_host(v).view(np.uint8),
                                      host[i].reshape(-1)[to[i]:to[i] + ln[i]].view(np.uint8))


def test_pack_worked_example_and_views(fp):
    say("pack FSDP1 worked example")
    cfg = CONFIGS["c1_three_4x2_nd2"]
    tensors = [torch.arange(8, dtype=torch.float32, device=dev()).view(4, 2) + 100 * (i + 1) for i in range(3)]
    plan = fp.Plan(cfg.shapes, 2)
    flat = plan.pack(tensors)
    torch.cuda.synchronize()
    assert plan.shard == 12
    w1, w2, w3 = [t.reshape(-1) for t in tensors]
    assert torch.equal(flat[:12], torch.cat([w1, w2[:4]]))
    assert torch.equal(flat[12:], torch.cat([w2[4:], w3]))
    r0 = plan.views(flat[:12], 0)
    r1 = plan.views(flat[12:], 1)
    assert [v.numel() for v in r0] == [8, 4, 0] and [v.numel() for v in r1] == [0, 4, 8]
    full_views = plan.views(flat, -1)
    full_views[1][3, 1] = -5.0                       # views alias the flat buffer
    assert float(flat[15]) == -5.0


# ------------------------------------------------------------------ whole step
def _step_case(fp, world, S, rank, n_micro, step, seed, flags, inf=False, grad_off=0, workspace=True,
               grad_sigma=1e-3, master_sigma=0.02):
    hp = HP
    scale = np.float32(1.0 / (world * n_micro))
    micro = [[gen.bf16_normal(S, grad_sigma, seed, gen.STREAM_GRAD, 0, m, q) for q in range(world)]
             for m in range(n_micro)]
    if inf and S:
        micro[-1][world // 2][S // 2] = 0x7F80
    th = gen.normal_f32(S, master_sigma, seed, gen.STREAM_MASTER)
    m0 = gen.normal_f32(S, 1e-4, seed, gen.STREAM_EXP_AVG) if step > 1 else np.zeros(S, np.float32)
    v0 = (gen.normal_f32(S, 1e-3, seed, gen.STREAM_EXP_AVG_SQ) ** 2 if step > 1 else np.zeros(S, np.float32))
    others = [gen.bf16_normal(S, master_sigma, seed, gen.STREAM_SHARD, q) for q in range(world)]

    acc_o, th_o, m_o, v_o = np.zeros(S, np.float32), th.copy(), m0.copy(), v0.copy()
    full_o, flag_o, norm_o = oracle.shard_step(micro, acc_o, th_o, m_o, v_o, others, rank, hp=hp, step=step)
    if flags & fp.FP_STEP_NO_SKIP:        # no gate: the oracle's update runs regardless
        th_o, m_o, v_o = th.copy(), m0.copy(), v0.copy()
        oracle.adamw(acc_o, th_o, m_o, v_o, step=step, skip=False, **hp_kwargs(hp))
        own = oracle.f32_to_bf16(th_o)
        full_o = full_o.copy()
        full_o[rank * S:(rank + 1) * S] = own

    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev()) if workspace else None
    ws = fp.new_workspace(dev(), S) if workspace else None
    for m in range(n_micro - 1):
        fp.reduce_shard(_grads_with_offset(micro[m], grad_off), acc, scale=float(scale),
                        accumulate=m > 0, found_inf=flag)
    d_th, d_m, d_v = to_dev(th), to_dev(m0), to_dev(v0)
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    shards = [to_dev(o) for o in others]
    shards[rank] = None
    call = fp.ShardStep(_grads_with_offset(micro[-1], grad_off), acc, d_th, d_m, d_v, shards, full,
                        rank, scale=float(scale), accumulate=n_micro > 1, found_inf=flag, sq_norm=sq,
                        workspace=ws, flags=flags, **hp_kwargs(hp))
    path = call.path()
    if flags & fp.FP_STEP_NO_SKIP:
        assert path == fp.FP_PATH_NO_SKIP
    elif not workspace or flags & fp.FP_STEP_NO_COOP:
        assert path == fp.FP_PATH_TWO_PHASE
    elif flags & fp.FP_STEP_KEEP_GRAD and n_micro > 1:
        # the kept gradient would overwrite an input accumulator before the barrier
        assert path == fp.FP_PATH_TWO_PHASE
    elif S <= 2_000_000:                  # far inside MI355X's co-resident capacity
        assert path == fp.FP_PATH_ONE_PASS
    call(step)
    torch.cuda.synchronize()
    assert int(flag.item()) == flag_o
    gh = [to_host(x) for x in (d_th, d_m, d_v)]
    if flag_o and not flags & fp.FP_STEP_NO_SKIP:
        for got, want in zip(gh, (th, m0, v0)):
            assert_f32_bitexact(got, want, "state must be untouched on overflow")
    else:
        for name, got, want in zip(("master", "exp_avg", "exp_avg_sq"), gh, (th_o, m_o, v_o)):
            assert_f32_close(got, want, name)
    full_h = to_host(full)
    own = slice(rank * S, (rank + 1) * S)
    assert_bf16_within_1ulp(full_h[own], full_o[own], "own shard")
    mask = np.ones(world * S, bool)
    mask[own] = False
    assert_bf16_equal(full_h[mask], full_o[mask], "other shards")
    if flags & fp.FP_STEP_KEEP_GRAD:
        assert_f32_bitexact(to_host(acc), acc_o, "kept gradient")
    if workspace and math.isfinite(norm_o):
        assert float(sq.item()) == pytest.approx(norm_o, rel=norm_rel_tol(S))
    if workspace:
        assert fp.workspace_timeouts(ws) == 0, "grid barrier wait gave up"
    return full_h


@pytest.mark.parametrize("rank", [0, 1])
@pytest.mark.parametrize("flags", [0, 1, 2, 3, 4, 6])
def test_step_worked_example(fp, rank, flags):
    """The three (4, 2) weights over two ranks with the workload's own draws:
    gradients and masters N(0, 1), one AdamW step."""
    cfg = CONFIGS["c1_three_4x2_nd2"]
    say(f"step C1 rank={rank} flags={flags}")
    _step_case(fp, world=cfg.world, S=12, rank=rank, n_micro=cfg.n_micro, step=1, seed=cfg.seed, flags=flags,
               grad_sigma=cfg.grad_sigma, master_sigma=cfg.master_sigma)


@pytest.mark.parametrize("flags", [0, 4])
def test_step_without_workspace(fp, flags):
    say(f"step without workspace flags={flags}")
    _step_case(fp, world=8, S=10_001, rank=5, n_micro=2, step=3, seed=3, flags=flags, inf=False,
               workspace=False)
    _step_case(fp, world=8, S=10_001, rank=5, n_micro=1, step=3, seed=4, flags=flags, inf=True,
               workspace=False)


@pytest.mark.parametrize("seed", range(14))
def test_step_random(fp, seed):
    r = np.random.default_rng(5000 + seed)
    world = int(r.choice([1, 2, 3, 8, 16, 64]))
    S = int(r.choice([1, 9, 64, 1001, 8 * 2048 + 5, 50_000]))
    rank = int(r.integers(0, world))
    n_micro = int(r.choice([1, 2, 4]))
    step = int(r.choice([1, 2, 7]))
    flags = int(r.choice([0, 0, 1, 2, 4, 6]))
    inf = seed % 4 == 3
    off = int(r.integers(0, 8)) if seed % 2 else 0
    say(f"step seed={seed} world={world} S={S} rank={rank} n_micro={n_micro} step={step} "
        f"flags={flags} inf={inf} grad_offset={off}")
    _step_case(fp, world, S, rank, n_micro, step, 77 + seed, flags, inf=inf, grad_off=off)


# ------------------------------------------------------------------ invariants
def test_allreduce_equals_reduce_scatter_then_allgather(fp):
    """Reducing every rank's shard and gathering equals reducing the whole buffer."""
    world, S = 8, 3001
    say("invariant AR = RS + AG")
    full_grads = np.stack([gen.bf16_normal(world * S, 1e-3, 9, gen.STREAM_GRAD, q) for q in range(world)])
    d = to_dev(full_grads)
    whole = torch.zeros(world * S, dtype=torch.float32, device=dev())
    fp.reduce_shard(d, whole, scale=1.0 / world)
    pieces = []
    for q in range(world):
        acc = torch.zeros(S, dtype=torch.float32, device=dev())
        fp.reduce_shard(d[:, q * S:(q + 1) * S], acc, scale=1.0 / world)
        pieces.append(acc)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(pieces).view(torch.int32), whole.view(torch.int32))


def test_adamw_shardwise_equals_whole_buffer(fp):
    world, S = 4, 1237
    say("invariant: AdamW shard by shard = whole buffer")
    P = world * S
    g, th = to_dev(gen.normal_f32(P, 1e-3, 3, gen.STREAM_GRAD)), to_dev(gen.normal_f32(P, 0.02, 3, 0))
    m = to_dev(gen.normal_f32(P, 1e-4, 3, gen.STREAM_EXP_AVG))
    v = to_dev(gen.normal_f32(P, 1e-3, 3, gen.STREAM_EXP_AVG_SQ) ** 2)
    whole = [x.clone() for x in (th, m, v)]
    fp.adamw_shard(g, *whole, step=5, **hp_kwargs(HP))
    parts = [x.clone() for x in (th, m, v)]
    for q in range(world):
        sl = slice(q * S, (q + 1) * S)
        # shard starts that are not 16-byte aligned go through a copy
        tmp = [x[sl].clone() for x in parts]
        fp.adamw_shard(g[sl].clone(), *tmp, step=5, **hp_kwargs(HP))
        for x, t in zip(parts, tmp):
            x[sl] = t
    torch.cuda.synchronize()
    for a, b in zip(whole, parts):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("S", [2_000_003, 2_900_001, 3_500_002])
def test_step_near_the_one_pass_capacity(fp, S):
    """Shards around the one-pass kernel's co-resident capacity: lanes that
    keep 2 quads, lanes that keep 4, and the two-kernel fallback."""
    say(f"step near one-pass capacity S={S}")
    _step_case(fp, world=2, S=S, rank=1, n_micro=1, step=2, seed=11, flags=0)
    _step_case(fp, world=2, S=S, rank=0, n_micro=2, step=1, seed=12, flags=0, inf=True)


def test_step_is_bitwise_reproducible(fp):
    say("invariant: reproducible step")
    outs = []
    for _ in range(2):
        outs.append(_step_case(fp, world=8, S=40_003, rank=3, n_micro=2, step=2, seed=5, flags=0))
    assert np.array_equal(outs[0], outs[1])


def test_pack_same_buffers_new_contents(fp):
    """fp_pack calls that reuse the previous call's buffers skip the pointer
    upload and the checks: they must still see the current contents, and a
    switch to other buffers and back must upload again."""
    say("pack same buffers, new contents")
    shapes = [(300, 9), (5000,), (), (7, 3)]
    plan = fp.Plan(shapes, 8)
    sets = []
    for k in range(2):
        host = [gen.bf16_bits_trunc(gen.normal_f32(math.prod(s), 1.0, 500 + k, gen.STREAM_TENSOR, i)).reshape(s)
                for i, s in enumerate(shapes)]
        dev_t = [to_dev(h.reshape(-1)).view(h.shape) for h in host]
        sets.append([host, dev_t])
    flat = torch.zeros(plan.padded, dtype=torch.int16, device=dev())
    outs = []
    for step, k in enumerate([0, 0, 1, 0, 1, 1]):
        host, dev_t = sets[k]
        if step == 1:                         # new contents in the same buffers
            host = [gen.bf16_bits_trunc(gen.normal_f32(math.prod(s), 1.0, 900, gen.STREAM_TENSOR, i)).reshape(s)
                    for i, s in enumerate(shapes)]
            for d, h in zip(dev_t, host):
                d.copy_(to_dev(h.reshape(-1)).view(h.shape))
            sets[k][0] = host
        plan.pack(dev_t, flat)
        outs.append((flat.clone(), [h.copy() for h in host]))
    torch.cuda.synchronize()
    for step, (got, host) in enumerate(outs):
        assert np.array_equal(to_host(got), oracle.pack(host, 8)), f"call {step}"


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_pack_many_small_tensors(fp, dtype):
    """20 000 tensors of 0 to 1200 elements (each small tensor one gathering
    entry) between a few larger ones (copy entries), each source at an odd
    element offset."""
    r = np.random.default_rng(17 if dtype == np.float32 else 18)
    sizes = r.integers(0, 1200, size=20_000)
    sizes[::997] = 5000                                   # a few copy entries between runs
    shapes = [(int(n),) for n in sizes]
    say(f"pack many small tensors dtype={np.dtype(dtype).name}")
    flat_host = gen.normal_f32(int(sizes.sum()), 1.0, 7, gen.STREAM_TENSOR)
    if dtype == np.uint16:
        flat_host = gen.bf16_bits_trunc(flat_host)
    host, o = [], 0
    for n in sizes:
        host.append(flat_host[o:o + n])
        o += n
    tdt = torch.float32 if dtype == np.float32 else torch.int16
    big = torch.zeros(int(sizes.sum()) + 3 * len(sizes) + 8, dtype=tdt, device=dev())
    srcs, o = [], 0
    for i, h in enumerate(host):
        o += 1 + i % 3                                    # odd element offsets
        v = big[o:o + h.size]
        if h.size:
            v.copy_(to_dev(h))
        srcs.append(v)
        o += h.size
    plan = fp.Plan(shapes, 64)
    flat = plan.pack(srcs)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(flat).view(np.uint8), oracle.pack(host, 64).view(np.uint8))
