"""GPU parity of the per-parameter dim-0 layout (fp_shard0_*) against the oracle.

Every parameter of a group is cut along dim 0 over N_d ranks, ceil(d0/N_d)
rows per rank with zero rows past d0, and a rank's chunks sit back to back
in one buffer ("Infra: Data Parallel", FSDP2 sections and the FSDP1 / FSDP2
comparison figure).  The copies move bits, so the bar is byte equality:
rank buffers and the gathered layout from fp_shard0_pack, the parameters
from fp_shard0_unpack.  Cases: the pages' worked examples, random groups
with 0-d, empty and uneven parameters at worlds 1 .. 128, sources and
destinations at odd element offsets, NaN / -0 payloads, destinations
pre-filled with garbage (the padding must be written), repeated calls with
other buffers, the Transformer-layer group of d=1024 and d=12288 at eight
ranks and the 10k-tensor group at 64 ranks at full size.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden
from gpu_common import dev, say, to_dev, to_host
from workloads import CONFIGS, gen

pytestmark = pytest.mark.gpu


def _host_params(shapes, dtype, seed, specials=False):
    out = []
    for i, s in enumerate(shapes):
        x = gen.normal_f32(math.prod(s), 1.0, seed, gen.STREAM_TENSOR, i)
        if specials and x.size:
            x[0] = np.float32("nan")
            x.view(np.uint32)[-1] = 0x80000000
        out.append((x if dtype == np.float32 else gen.bf16_bits_trunc(x)).reshape(s))
    return out


def _torch_dtype(dtype):
    return torch.float32 if dtype == np.float32 else torch.int16


def _at_offset(n, dtype, off, fill=None):
    """A device tensor of n elements starting `off` elements into its own buffer."""
    buf = torch.empty(n + off + 8, dtype=_torch_dtype(dtype), device=dev())
    if fill is None:
        buf.zero_()
    else:
        buf.fill_(fill)
    return buf[off:off + n]


def _params_on_device(host, dtype, r):
    out = []
    for h in host:
        v = _at_offset(h.size, dtype, int(r.integers(0, 4))).view(h.shape)
        if h.size:
            v.copy_(to_dev(h.reshape(-1)).view(h.shape))
        out.append(v)
    return out


def _same(a, b):
    """Byte equality without copies."""
    a = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    b = np.ascontiguousarray(b).reshape(-1).view(np.uint8)
    return a.shape == b.shape and bool(np.array_equal(a, b))


def test_shard0_worked_examples(fp):
    """The pages' examples: three (4, 2) weights over 2 ranks (rank 0 the
    first two rows of each, 12 elements per rank); an (8, 4) weight over 4."""
    g = load_golden("fsdp2_dim0_examples.json")
    for ex in g["examples"]:
        shapes = [tuple(s) for s in ex["shapes"]]
        world = ex["world"]
        say(f"shard0 worked example shapes={shapes} world={world}")
        params = [torch.arange(math.prod(s), dtype=torch.float32, device=dev()).view(s) + 100 * (i + 1)
                  for i, s in enumerate(shapes)]
        plan = fp.Shard0Plan(shapes, world)
        assert plan.shard == ex["elements_per_rank"]
        full = plan.pack(params)
        torch.cuda.synchronize()
        for q in range(world):
            buf = plan.pack(params, rank=q)
            torch.cuda.synchronize()
            assert torch.equal(buf, full[q * plan.shard:(q + 1) * plan.shard])
            lo, hi = ex["rows_of_rank"][str(q)]
            for p, v in zip(params, plan.views(buf, q)):
                assert tuple(v.shape) == tuple(ex["local_shape"])
                assert torch.equal(v, p[lo:hi])
        back = plan.unpack(full)
        torch.cuda.synchronize()
        for p, b in zip(params, back):
            assert torch.equal(p, b)


@pytest.mark.parametrize("seed", range(12))
def test_shard0_random_groups(fp, seed):
    r = np.random.default_rng(7000 + seed)
    shapes = []
    for _ in range(int(r.integers(1, 25))):
        k = int(r.integers(0, 4))
        shapes.append(tuple(int(x) for x in r.integers(0 if r.random() < 0.1 else 1, 30, size=k)))
    if seed % 3 == 0:
        shapes.append((3001, 7))            # many workgroups, uneven rows
    if seed % 4 == 1:
        shapes.append((5, 9000))            # few rows, long rows
    world = int(r.choice([1, 2, 3, 8, 64, 128]))
    dtype = np.float32 if seed % 2 == 0 else np.uint16
    say(f"shard0 seed={seed} params={len(shapes)} world={world} dtype={np.dtype(dtype).name}")
    host = _host_params(shapes, dtype, seed, specials=seed % 3 == 0)
    params = _params_on_device(host, dtype, r)
    plan = fp.Shard0Plan(shapes, world)
    S = plan.shard
    garbage = -7 if dtype == np.uint16 else float("nan")

    want_full = np.concatenate([oracle.shard0_pack(host, world, q) for q in range(world)]) if S else \
        np.zeros(0, dtype)
    full = _at_offset(world * S, dtype, int(r.integers(0, 4)), fill=garbage)
    plan.pack(params, full)
    torch.cuda.synchronize()
    assert _same(to_host(full), want_full)

    for q in sorted(set([0, world - 1, int(r.integers(0, world))])):
        buf = _at_offset(S, dtype, int(r.integers(0, 4)), fill=garbage)
        plan.pack(params, buf, rank=q)
        torch.cuda.synchronize()
        assert _same(to_host(buf), oracle.shard0_pack(host, world, q)), f"rank {q}"

    want = oracle.shard0_unpack(want_full, shapes, world)
    outs = [_at_offset(math.prod(s), dtype, int(r.integers(0, 4)), fill=garbage).view(s) for s in shapes]
    src = _at_offset(world * S, dtype, int(r.integers(0, 4)))
    if S:
        src.copy_(to_dev(want_full))
    plan.unpack(src, outs)
    torch.cuda.synchronize()
    for i, (o, w) in enumerate(zip(outs, want)):
        assert _same(to_host(o), w), f"parameter {i}"
        assert _same(w, host[i])


@pytest.mark.parametrize("world", [3, 8])
@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_shard0_small_and_large_pieces(fp, world, dtype):
    """Per-rank pieces on both sides of the size where the kernel switches
    from one copy per piece to one gathering workgroup set per parameter,
    with uneven last ranks and odd element offsets."""
    shapes = [(1000, 37), (2047,), (2048 * 3 + 1,), (4096 * 8,), (9, 511), (7, 4097), (1,), (2, 1025)]
    say(f"shard0 piece sizes world={world} dtype={np.dtype(dtype).name}")
    r = np.random.default_rng(world)
    host = _host_params(shapes, dtype, 31 + world, specials=True)
    params = _params_on_device(host, dtype, r)
    plan = fp.Shard0Plan(shapes, world)
    S = plan.shard
    want_full = np.concatenate([oracle.shard0_pack(host, world, q) for q in range(world)])
    full = _at_offset(world * S, dtype, 3, fill=-7 if dtype == np.uint16 else float("nan"))
    plan.pack(params, full)
    torch.cuda.synchronize()
    assert _same(to_host(full), want_full)
    for q in range(world):
        buf = _at_offset(S, dtype, q % 4, fill=-7 if dtype == np.uint16 else float("nan"))
        plan.pack(params, buf, rank=q)
        torch.cuda.synchronize()
        assert _same(to_host(buf), oracle.shard0_pack(host, world, q)), f"rank {q}"
    want = oracle.shard0_unpack(want_full, shapes, world)
    outs = [_at_offset(math.prod(s), dtype, 1 + i % 3, fill=0).view(s) for i, s in enumerate(shapes)]
    plan.unpack(full, outs)
    torch.cuda.synchronize()
    for i, (o, w) in enumerate(zip(outs, want)):
        assert _same(to_host(o), w), f"parameter {i}"


def test_shard0_same_buffers_new_contents(fp):
    """Calls that reuse the previous call's buffers skip the pointer upload:
    they must still see the current contents, and a switch to other buffers
    and back must upload again."""
    shapes = [(300, 9), (5000,), ()]
    world = 8
    plan = fp.Shard0Plan(shapes, world)
    say("shard0 same buffers, new contents")
    r = np.random.default_rng(5)
    sets = []
    for k in range(2):
        h = _host_params(shapes, np.uint16, 200 + k)
        sets.append((h, _params_on_device(h, np.uint16, r)))
    full = torch.empty(world * plan.shard, dtype=torch.int16, device=dev())
    outs = []
    for step, k in enumerate([0, 0, 1, 0, 1, 1]):
        h, p = sets[k]
        if step == 1:                       # new contents in the same buffers
            h = _host_params(shapes, np.uint16, 300)
            for x, y in zip(p, h):
                x.copy_(to_dev(y.reshape(-1)).view(y.shape))
            sets[0] = (h, p)
        plan.pack(p, full)
        outs.append((full.clone(), [x.copy() for x in h]))
    torch.cuda.synchronize()
    for step, (got, h) in enumerate(outs):
        want = np.concatenate([oracle.shard0_pack(h, world, q) for q in range(world)])
        assert _same(to_host(got), want), f"call {step}"


def test_shard0_repeated_calls_new_buffers(fp):
    """The per-call pointer table: consecutive calls with other buffers,
    without a synchronisation in between, each see their own pointers."""
    shapes = [(37, 5), (11,), (), (64, 3)]
    world = 4
    plan = fp.Shard0Plan(shapes, world)
    say("shard0 repeated calls")
    hosts, outs = [], []
    for k in range(6):
        h = _host_params(shapes, np.uint16, 90 + k)
        p = _params_on_device(h, np.uint16, np.random.default_rng(k))
        hosts.append(h)
        outs.append((plan.pack(p, rank=k % world), p))
    torch.cuda.synchronize()
    for k, (buf, _) in enumerate(outs):
        assert _same(to_host(buf), oracle.shard0_pack(hosts[k], world, k % world))


@pytest.mark.parametrize("name", ["c2_layer_d1024_nd8", "c4_layer_d12288_nd8"])
def test_shard0_transformer_layer_full_size(fp, name):
    """The Transformer-layer group at full size in bf16 (the gathered
    parameters and the reduce-scatter input are bf16): gradients of every
    parameter to the rank-major layout, and the gathered layout back to the
    parameters, compared in full with the oracle."""
    cfg = CONFIGS[name]
    world = cfg.world
    say(f"shard0 full size {name} world={world}")
    shapes = list(cfg.shapes)
    params = [gen.torch_bf16_normal(math.prod(s), 1e-3, 11, (gen.STREAM_TENSOR, i), dev()).view(s)
              for i, s in enumerate(shapes)]
    plan = fp.Shard0Plan(shapes, world)
    full = plan.pack(params)
    torch.cuda.synchronize()
    host = [to_host(p) for p in params]
    del params
    got = to_host(full)
    del full
    S = plan.shard
    want_full = np.concatenate([oracle.shard0_pack(host, world, q) for q in range(world)])
    assert got.size == want_full.size
    for q in range(world):
        assert _same(got[q * S:(q + 1) * S], want_full[q * S:(q + 1) * S]), f"rank {q}"
    del got
    outs = plan.unpack(to_dev(want_full))
    torch.cuda.synchronize()
    want = oracle.shard0_unpack(want_full, shapes, world)
    for i, (o, w) in enumerate(zip(outs, want)):
        assert _same(to_host(o), w), f"parameter {i}"


def test_shard0_ragged_10k_full_size(fp):
    """The 10k-tensor group at 64 ranks at full size (2.73G bf16 elements, the
    parameters views of one allocation, as the bench lays them out): every
    rank's rows in full against the oracle, and the gathered layout back into
    the parameters, which must reproduce them bit for bit (the oracle's
    unpack inverts its pack, a CPU pin)."""
    cfg = CONFIGS["c5_ragged10k_nd64"]
    world = cfg.world
    shapes = list(cfg.shapes)
    numel = [math.prod(s) for s in shapes]
    T = sum(numel)
    offs = [0]
    for n in numel[:-1]:
        offs.append(offs[-1] + n)
    say(f"shard0 full size c5: {len(shapes)} parameters, {T} elements, world={world}")
    flat = gen.torch_bf16_normal(T, 1e-3, 12, (gen.STREAM_TENSOR,), dev())
    plan = fp.Shard0Plan(shapes, world)
    full = plan.pack([flat[o:o + n].view(s) for o, n, s in zip(offs, numel, shapes)])
    torch.cuda.synchronize()
    host_flat = to_host(flat)
    host = [host_flat[o:o + n].reshape(s) for o, n, s in zip(offs, numel, shapes)]
    got = to_host(full)
    S = plan.shard
    assert got.size == world * S
    for q in range(world):
        assert _same(got[q * S:(q + 1) * S], oracle.shard0_pack(host, world, q)), f"rank {q}"
    del host, host_flat, got
    back = torch.empty_like(flat)
    plan.unpack(full, [back[o:o + n].view(s) for o, n, s in zip(offs, numel, shapes)])
    torch.cuda.synchronize()
    assert torch.equal(back, flat)
    plan.close()


@pytest.mark.parametrize("rank", [0, 3])
def test_shard0_step_composition(fp, rank):
    """One step in the dim-0 layout with the flat step's kernels: every
    rank's full-shape bf16 gradients to the rank-major layout
    (fp_shard0_pack), this rank's fixed-order reduce + AdamW + bf16 cast +
    copy of the other ranks' shards (fp_shard_step on the S-element shard),
    then the gathered buffer back to full-shape parameters
    (fp_shard0_unpack); against the oracle's same composition.  Uneven
    first dims put zero padding rows in the shards: their gradient is 0 and
    so is their master weight, so they stay 0."""
    from gpu_common import assert_bf16_within_1ulp, assert_f32_close, hp_kwargs
    from workloads.configs import AdamW
    hp = AdamW()
    shapes = [(48, 32), (48,), (13, 7), (), (5,), (2, 3000)]
    world, seed = 4, 21
    say(f"shard0 step composition rank={rank}")
    plan = fp.Shard0Plan(shapes, world)
    S = plan.shard
    grads = [[gen.bf16_normal(math.prod(s), 1e-3, seed, gen.STREAM_GRAD, q, i).reshape(s)
              for i, s in enumerate(shapes)] for q in range(world)]
    master = [gen.normal_f32(math.prod(s), 0.02, seed, gen.STREAM_MASTER, i).reshape(s)
              for i, s in enumerate(shapes)]
    others = [oracle.f32_to_bf16(oracle.shard0_pack(master, world, q)) for q in range(world)]

    rows_o = [oracle.shard0_pack(grads[q], world, rank) for q in range(world)]
    th_o = oracle.shard0_pack(master, world, rank)
    acc_o, m_o, v_o = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.float32)
    full_o, flag_o, _ = oracle.shard_step([rows_o], acc_o, th_o, m_o, v_o, others, rank, hp=hp, step=1)
    params_o = oracle.shard0_unpack(full_o, shapes, world)

    r = np.random.default_rng(rank)
    bufs = [plan.pack(_params_on_device(grads[q], np.uint16, r)) for q in range(world)]
    rows = [b[rank * S:(rank + 1) * S] for b in bufs]
    th = plan.pack(_params_on_device(master, np.float32, r), rank=rank)
    acc, m, v = (torch.zeros(S, dtype=torch.float32, device=dev()) for _ in range(3))
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    shards = [to_dev(o) for o in others]
    shards[rank] = None
    fp.shard_step(rows, acc, th, m, v, shards, full, rank, scale=1.0 / world, found_inf=flag, step=1,
                  **hp_kwargs(hp))
    params = plan.unpack(full)
    torch.cuda.synchronize()
    assert int(flag.item()) == flag_o == 0
    assert_f32_close(to_host(th), th_o, "master shard")
    assert_f32_close(to_host(m), m_o, "exp_avg")
    assert_f32_close(to_host(v), v_o, "exp_avg_sq")
    for i, (p, w) in enumerate(zip(params, params_o)):
        assert_bf16_within_1ulp(to_host(p).reshape(-1), w.reshape(-1), f"parameter {i}")
