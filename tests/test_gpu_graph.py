"""The step under HIP graph capture, replayed as bench.py times it.

One step per buffer set is captured into one graph (the overflow flag cleared
by a fill kernel inside it) and the graph is replayed several times, with
unrelated eager work, an eager library call and a synchronisation between
replays.  After every replay, each set's master / moments, full bf16 buffer,
flag and norm must equal, bit for bit, the same sequence of steps launched
eagerly (the kernels are deterministic); one pass sees an injected +inf in
one set, so the flag cleared inside the graph and the skip it gates are
replayed too.  The first eager pass is checked against the oracle as well.  Paths: the one-pass step at the d=1024 layer's
shard shape (S = 1,574,528, N_d = 8), the two-phase and the fused no-skip
step at the same shape, the no-skip step from 2^24 elements on (fused update
and copies in two launches) at S = 2^24 + 3, N_d = 8, and the multi-unit
reduce + step over unequal units with two micro-batches.
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
REPLAYS = 4


def _row_tensor(rows):
    """The ranks' rows cut from one tensor, each starting on a 128-byte line."""
    S = rows[0].size
    Sp = -(-S // 64) * 64
    t = torch.zeros(len(rows), Sp + 64, dtype=torch.int16, device=dev())
    for q, h in enumerate(rows):
        t[q, :S].copy_(to_dev(h))
    return t[:, :S]


def _interleave(fp, scratch):
    """Eager work between replays: a torch kernel, a library call, a sync."""
    scratch["x"].mul_(1.0001).add_(1.0)
    fp.unshard(scratch["shards"], scratch["full"])
    torch.cuda.synchronize()


def _scratch(fp):
    shards = [torch.full((5000,), q, dtype=torch.int16, device=dev()) for q in range(3)]
    return {"x": torch.ones(1 << 20, device=dev()), "shards": shards,
            "full": torch.zeros(3 * 5000, dtype=torch.int16, device=dev())}


def _single_sets(fp, world, S, rank, flags, n_sets=2, seed=40):
    sets = []
    for k in range(n_sets):
        grads = [gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, k, 0, q) for q in range(world)]
        others = [gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, k, q) for q in range(world)]
        th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER, k)
        s = dict(grads_h=grads, others_h=others, th_h=th,
                 grads=_row_tensor(grads),
                 shards=[None if q == rank else to_dev(others[q]) for q in range(world)],
                 acc=torch.zeros(S, dtype=torch.float32, device=dev()),
                 state=[to_dev(th), torch.zeros(S, dtype=torch.float32, device=dev()),
                        torch.zeros(S, dtype=torch.float32, device=dev())],
                 full=torch.zeros(world * S, dtype=torch.int16, device=dev()),
                 flag=torch.zeros(1, dtype=torch.int32, device=dev()),
                 sq=torch.zeros(1, dtype=torch.float64, device=dev()),
                 ws=fp.new_workspace(dev(), S))
        s["init"] = [t.clone() for t in s["state"]]
        s["call"] = fp.ShardStep(s["grads"], s["acc"], *s["state"], s["shards"], s["full"], rank,
                                 scale=1.0 / world, found_inf=s["flag"], sq_norm=s["sq"], workspace=s["ws"],
                                 flags=flags, **hp_kwargs(HP))
        sets.append(s)
    return sets


def _snapshot(s):
    return [t.clone() for t in (*s["state"], s["full"], s["flag"], s["sq"])]


def _run_single(sets):
    for k, s in enumerate(sets):
        s["flag"].zero_()
        s["call"](k + 1)                   # set k takes step number k + 1 in every pass


def _inject(sets, r, on):
    """Pass 1 sees a +inf gradient in set 1 (rank 5, element S // 3): that set's
    step is skipped (or, without the gate, updates with the inf)."""
    if r == 1:
        g = sets[1]["grads"]
        g[5, g.shape[1] // 3] = 0x7F80 if on else int(sets[1]["grads_h"][5][g.shape[1] // 3].view(np.int16))


def _restore(s):
    for t, t0 in zip(s["state"], s["init"]):
        t.copy_(t0)
    s["full"].zero_()
    s["sq"].zero_()


def _assert_same(got, want, what):
    names = ("master", "exp_avg", "exp_avg_sq", "full", "found_inf", "sq_norm")
    for name, g, w in zip(names, got, want):
        assert torch.equal(g.view(torch.uint8), w.view(torch.uint8)), f"{what}: {name} differs"


@pytest.mark.parametrize("flags,path", [(0, "one-pass"), (4, "two-phase"), (1, "no-skip")])
def test_step_graph_replays_match_eager(fp, flags, path):
    world, S, rank = 8, 1_574_528, 1
    say(f"graph replays: step path={path} S={S} N={world}")
    sets = _single_sets(fp, world, S, rank, flags)
    want_path = {"one-pass": fp.FP_PATH_ONE_PASS, "two-phase": fp.FP_PATH_TWO_PHASE,
                 "no-skip": fp.FP_PATH_NO_SKIP}[path]
    assert sets[0]["call"].path() == want_path
    scratch = _scratch(fp)

    # eager reference: REPLAYS passes over the sets, a snapshot after each
    eager = []
    for r in range(REPLAYS):
        _inject(sets, r, True)
        _run_single(sets)
        _inject(sets, r, False)
        torch.cuda.synchronize()
        eager.append([_snapshot(s) for s in sets])
        if r == 1:
            assert int(sets[1]["flag"].item()) == 1 and int(sets[0]["flag"].item()) == 0
        if r == 0:
            # the first pass against the oracle (set 0: step 1)
            s = sets[0]
            acc_o, th_o = np.zeros(S, np.float32), s["th_h"].copy()
            m_o, v_o = np.zeros(S, np.float32), np.zeros(S, np.float32)
            full_o, flag_o, _ = oracle.shard_step([s["grads_h"]], acc_o, th_o, m_o, v_o, s["others_h"], rank,
                                                  hp=HP, step=1)
            assert flag_o == 0 and int(s["flag"].item()) == 0
            for name, g, w in zip(("master", "exp_avg", "exp_avg_sq"), s["state"], (th_o, m_o, v_o)):
                assert_f32_close(to_host(g), w, name)
    for s in sets:
        _restore(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run_single(sets)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        _inject(sets, r, True)
        graph.replay()
        _inject(sets, r, False)
        torch.cuda.synchronize()
        for k, s in enumerate(sets):
            _assert_same(_snapshot(s), eager[r][k], f"replay {r}, set {k}")
        _interleave(fp, scratch)
        for k, s in enumerate(sets):
            assert fp.workspace_timeouts(s["ws"]) == 0
    del graph


def test_split_no_skip_graph_replays_match_eager(fp):
    world, S, rank = 8, (1 << 24) + 3, 6
    say(f"graph replays: split no-skip step S={S} N={world}")
    seed = 43
    grads = torch.stack([gen.torch_bf16_normal(S, 1e-3, seed, (gen.STREAM_GRAD, q), dev()) for q in range(world)])
    others = [gen.torch_bf16_normal(S, 0.02, seed, (gen.STREAM_SHARD, q), dev()) for q in range(world)]
    shards = [None if q == rank else others[q] for q in range(world)]
    init = [gen.torch_normal_f32(S, 0.02, seed, (gen.STREAM_MASTER,), dev()),
            gen.torch_normal_f32(S, 1e-4, seed, (gen.STREAM_EXP_AVG,), dev()),
            gen.torch_normal_f32(S, 1e-3, seed, (gen.STREAM_EXP_AVG_SQ,), dev()).square()]
    state = [t.clone() for t in init]
    acc = torch.zeros(S, dtype=torch.float32, device=dev())
    full = torch.zeros(world * S, dtype=torch.int16, device=dev())
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    ws = fp.new_workspace(dev(), S)
    call = fp.ShardStep(grads, acc, *state, shards, full, rank, scale=1.0 / world, found_inf=flag, sq_norm=sq,
                        workspace=ws, flags=fp.FP_STEP_NO_SKIP, **hp_kwargs(HP))
    assert call.path() == fp.FP_PATH_NO_SKIP_SPLIT
    pos = S - 2                            # pass 1 sees +inf here in rank 4's row (the ragged tail)
    keep = int(grads[4, pos].item())
    scratch = _scratch(fp)

    steps = [2, 3, 2, 3]                   # the step number is a launch argument: one graph per number

    def run(r):
        if r == 1:
            grads[4, pos] = 0x7F80
        flag.zero_()
        call(steps[r])

    def after(r):
        if r == 1:
            grads[4, pos] = keep

    def snap():
        return [t.clone() for t in (*state, full, flag, sq)]

    eager = []
    for r in range(REPLAYS):
        run(r)
        torch.cuda.synchronize()
        after(r)
        eager.append(snap())
        assert int(flag.item()) == (1 if r == 1 else 0)
        if r == 0:
            # the first pass against the oracle at sampled positions
            idx = torch.from_numpy(np.sort(np.random.default_rng(5).choice(S, 1 << 12, replace=False))).to(dev())
            rows = [to_host(grads[q].index_select(0, idx)) for q in range(world)]
            g_o = oracle.reduce(rows, np.float32(1.0 / world))
            th_o, m_o, v_o = (to_host(t.index_select(0, idx)) for t in init)
            oracle.adamw(g_o, th_o, m_o, v_o, step=2, skip=False, **hp_kwargs(HP))
            for name, g, w in zip(("master", "exp_avg", "exp_avg_sq"), state, (th_o, m_o, v_o)):
                assert_f32_close(to_host(g.index_select(0, idx)), w, name)
    for t, t0 in zip(state, init):
        t.copy_(t0)
    full.zero_()
    sq.zero_()
    torch.cuda.synchronize()

    graphs = {}
    for n in (2, 3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            flag.zero_()
            call(n)
        graphs[n] = g
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        if r == 1:
            grads[4, pos] = 0x7F80
        graphs[steps[r]].replay()
        torch.cuda.synchronize()
        after(r)
        _assert_same(snap(), eager[r], f"replay {r}")
        _interleave(fp, scratch)
        assert fp.workspace_timeouts(ws) == 0
    del graphs


def test_units_graph_replays_match_eager(fp):
    sizes, world, rank, n_micro = [70_001, 0, 131_072, 3, 250_000], 4, 2, 2
    say(f"graph replays: units sizes={sizes} N={world} micro={n_micro}")
    seed = 41
    grads = [[[_row_tensor([gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, u, m, q)])[0]
               for q in range(world)] for u, S in enumerate(sizes)] for m in range(n_micro)]
    others = [[None if q == rank else to_dev(gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, u, q))
               for q in range(world)] for u, S in enumerate(sizes)]
    full = [torch.zeros(max(1, world * S), dtype=torch.int16, device=dev()) for S in sizes]
    plans = [fp.Units(grads[m], rank, shards=others, full=full) for m in range(n_micro)]
    P = plans[0].partition
    acc = torch.zeros(P, dtype=torch.float32, device=dev())
    state = [torch.zeros(P, dtype=torch.float32, device=dev()) for _ in range(3)]
    for u, S in enumerate(sizes):
        plans[0].unit_slice(state[0], u).copy_(to_dev(gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER, u)))
    init = [t.clone() for t in state]
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    sq = torch.zeros(1, dtype=torch.float64, device=dev())
    ws = plans[0].new_workspace()
    scale = 1.0 / (world * n_micro)
    scratch = _scratch(fp)

    def run():
        flag.zero_()
        plans[0].reduce(acc, scale=scale, accumulate=False, found_inf=flag)
        plans[1].step(acc, *state, scale=scale, accumulate=True, step=1, found_inf=flag, sq_norm=sq,
                      workspace=ws, **hp_kwargs(HP))

    def snap():
        return [t.clone() for t in (*state, acc, flag, sq, *full)]

    eager = []
    for _ in range(REPLAYS):
        run()
        torch.cuda.synchronize()
        eager.append(snap())
    assert int(flag.item()) == 0
    for t, t0 in zip(state, init):
        t.copy_(t0)
    for f in full:
        f.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        graph.replay()
        torch.cuda.synchronize()
        for i, (g, w) in enumerate(zip(snap(), eager[r])):
            assert torch.equal(g.view(torch.uint8), w.view(torch.uint8)), f"replay {r}: buffer {i} differs"
        _interleave(fp, scratch)
    del graph
    for p in plans:
        p.close()
