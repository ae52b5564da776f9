"""The speculative exact-skip step (separate output state buffers).

The fused pass stores the update to the output buffers without waiting for
the overflow check, and a last kernel restores the input state into them on
overflow; a shard that fits the one-pass kernel takes it instead, with the
outputs as store targets and the input state copied to them on overflow.  Its results must equal, bit for bit, those of the in-place
two-phase exact-skip step on the same inputs (the same per-element
arithmetic), with the input buffers left untouched:
* finite gradients, shards from 1 element to a few tiles with a ragged tail,
  N_d in {1, 3, 8}, against the oracle as well;
* an overflow in this micro-batch, and one left by an earlier micro-batch
  (flag already set, accumulate): outputs = inputs, own shard = bf16 of the
  unchanged master;
* shards of 2^24 elements and more (the split launches), finite and overflowed;
* a run of steps alternating two calls with swapped buffers: eagerly, with
  an overflow in the middle, and replayed from one captured graph.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import assert_bf16_equal, assert_f32_close, dev, hp_kwargs, say, to_dev, to_host
from workloads import gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _same(a, b, what):
    assert torch.equal(_bits(a), _bits(b)), what


class Case:
    """One rank's step inputs on the device, host copies kept for the oracle."""

    def __init__(self, world, S, rank, seed, on_device=False):
        self.world, self.S, self.rank = world, S, rank
        if on_device:
            self.grads = [gen.torch_bf16_normal(S, 1e-3, seed, (gen.STREAM_GRAD, q), dev()) for q in range(world)]
            others = [gen.torch_bf16_normal(S, 0.02, seed, (gen.STREAM_SHARD, q), dev()) for q in range(world)]
            self.state0 = [gen.torch_normal_f32(S, 0.02, seed, (gen.STREAM_MASTER,), dev()),
                           gen.torch_normal_f32(S, 1e-4, seed, (gen.STREAM_EXP_AVG,), dev()),
                           gen.torch_normal_f32(S, 1e-3, seed, (gen.STREAM_EXP_AVG_SQ,), dev()).square()]
            self.host = None
        else:
            g = [gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, 0, 0, q) for q in range(world)]
            o = [gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, 0, q) for q in range(world)]
            th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER, 0)
            m = gen.normal_f32(S, 1e-4, seed, gen.STREAM_EXP_AVG, 0)
            v = np.square(gen.normal_f32(S, 1e-3, seed, gen.STREAM_EXP_AVG_SQ, 0))
            self.host = dict(grads=g, others=o, state=(th, m, v))
            self.grads = [to_dev(h) for h in g]
            others = [to_dev(h) for h in o]
            self.state0 = [to_dev(x) for x in (th, m, v)]
        self.shards = [None if q == rank else others[q] for q in range(world)]

    def buffers(self):
        S = self.S
        return dict(acc=torch.zeros(max(S, 1), dtype=torch.float32, device=dev()),
                    state=[t.clone() for t in self.state0],
                    out=[torch.full((max(S, 1),), 7.0, dtype=torch.float32, device=dev()) for _ in range(3)],
                    full=torch.zeros(max(self.world * S, 1), dtype=torch.int16, device=dev()),
                    flag=torch.zeros(1, dtype=torch.int32, device=dev()),
                    sq=torch.zeros(1, dtype=torch.float64, device=dev()),
                    ws=fp_mod().new_workspace(dev(), S))

    def call(self, b, flags, speculative, step, accumulate=False, state=None, out=None):
        fp = fp_mod()
        state = b["state"] if state is None else state
        out = (b["out"] if speculative else None) if out is None else out
        return fp.ShardStep(self.grads, b["acc"][:self.S], *[t[:self.S] for t in state], self.shards,
                            b["full"][:self.world * self.S], self.rank, scale=1.0 / self.world,
                            found_inf=b["flag"], sq_norm=b["sq"], workspace=b["ws"], flags=flags,
                            accumulate=accumulate,
                            out=None if out is None else [t[:self.S] for t in out], **hp_kwargs(HP))


_FP = {}


def fp_mod():
    return _FP["fp"]


@pytest.fixture(autouse=True)
def _keep_fp(fp):
    _FP["fp"] = fp


def _run_pair(fp, case, step, inject=None, preset_flag=False):
    """The speculative step in its two forms -- on the one-pass kernel (when the
    shard fits it) and as the fused pass plus the restore kernel -- and the
    in-place two-phase step, on the same inputs."""
    res = {}
    for name, spec, flags in (("spec1", True, fp.FP_STEP_EXACT_SKIP),
                              ("spec", True, fp.FP_STEP_EXACT_SKIP | fp.FP_STEP_NO_COOP),
                              ("two", False, fp.FP_STEP_NO_COOP)):
        b = case.buffers()
        accumulate = False
        if preset_flag:
            # an earlier micro-batch overflowed: its flag stays set, acc holds it
            b["flag"].fill_(1)
            fp.reduce_shard(case.grads, b["acc"][:case.S], scale=1.0 / case.world, accumulate=False)
            accumulate = True
        if inject is not None:
            q, j = inject
            keep = case.grads[q][j].clone()
            case.grads[q][j] = 0x7F80
        call = case.call(b, flags, spec, step, accumulate=accumulate)
        fused = fp.FP_PATH_SPECULATIVE_SPLIT if case.S >= 1 << 24 else fp.FP_PATH_SPECULATIVE
        path = call.path()
        if name == "spec1":
            if case.S <= 2_000_000:               # far inside MI355X's co-resident capacity
                assert path == fp.FP_PATH_SPECULATIVE_ONE_PASS
            else:
                assert path in (fp.FP_PATH_SPECULATIVE_ONE_PASS, fused)
        else:
            assert path == (fused if spec else fp.FP_PATH_TWO_PHASE)
        call(step)
        torch.cuda.synchronize()
        if inject is not None:
            case.grads[q][j] = keep
        res[name] = b
        assert fp.workspace_timeouts(b["ws"]) == 0
    return res


def _check_pair(case, res, overflow):
    S = case.S
    two = res["two"]
    for key in ("spec1", "spec"):
        spec = res[key]
        for i, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
            _same(spec["state"][i][:S], case.state0[i][:S], f"{key}: input {name} untouched")
            _same(spec["out"][i][:S], two["state"][i][:S], f"{key}: out {name} = two-phase {name}")
            if overflow:
                _same(spec["out"][i][:S], case.state0[i][:S], f"{key}: out {name} = input on overflow")
        _same(spec["full"], two["full"], f"{key}: full")
        assert int(spec["flag"].item()) == int(two["flag"].item()) == (1 if overflow else 0)
        assert float(spec["sq"].item()) == pytest.approx(float(two["sq"].item()), rel=1e-12, nan_ok=True)


@pytest.mark.parametrize("world,S,rank", [(1, 1, 0), (3, 5, 2), (8, 4099, 1), (8, 1_574_531, 6), (3, 300_001, 0)])
def test_speculative_matches_two_phase_and_oracle(fp, world, S, rank):
    say(f"speculative step: world={world} S={S} rank={rank}")
    case = Case(world, S, rank, seed=80 + S % 97)
    res = _run_pair(fp, case, step=3)
    _check_pair(case, res, overflow=False)
    spec = res["spec1"]
    if S <= 300_001:
        h = case.host
        acc_o = np.zeros(S, np.float32)
        th_o, m_o, v_o = (x.copy() for x in h["state"])
        full_o, flag_o, _ = oracle.shard_step([h["grads"]], acc_o, th_o, m_o, v_o, h["others"], rank, hp=HP, step=3)
        assert flag_o == 0
        for name, got, want in zip(("master", "exp_avg", "exp_avg_sq"), spec["out"], (th_o, m_o, v_o)):
            assert_f32_close(to_host(got[:S]), want, name)
        own = slice(rank * S, (rank + 1) * S)
        fh = to_host(spec["full"][:world * S])
        mask = np.ones(world * S, bool)
        mask[own] = False
        assert_bf16_equal(fh[mask], full_o[mask], "other shards")


@pytest.mark.parametrize("world,S,rank,where", [(3, 5, 1, "this"), (8, 4099, 7, "this"), (8, 1_574_531, 2, "this"),
                                                 (8, 4099, 3, "earlier"), (3, 300_001, 0, "earlier")])
def test_speculative_overflow_restores_state(fp, world, S, rank, where):
    say(f"speculative step overflow ({where} micro-batch): world={world} S={S} rank={rank}")
    case = Case(world, S, rank, seed=90 + S % 89)
    if where == "this":
        res = _run_pair(fp, case, step=2, inject=(world - 1, S - 1))
    else:
        res = _run_pair(fp, case, step=2, preset_flag=True)
    _check_pair(case, res, overflow=True)
    # the own shard holds bf16 of the unchanged master
    own = to_host(res["spec1"]["full"][rank * S:(rank + 1) * S])
    assert_bf16_equal(own, oracle.f32_to_bf16(to_host(case.state0[0][:S])), "own shard")


@pytest.mark.parametrize("inject", [None, (5, 12_345)])
def test_speculative_split_at_large_shards(fp, inject):
    world, S, rank = 8, (1 << 24) + 3, 4
    say(f"speculative split step: world={world} S={S} inject={inject}")
    case = Case(world, S, rank, seed=71, on_device=True)
    res = _run_pair(fp, case, step=4, inject=inject)
    _check_pair(case, res, overflow=inject is not None)
    del res
    torch.cuda.empty_cache()


def test_speculative_alternating_buffers_eager_and_graph(fp):
    """Steps 1..4 alternate two calls with swapped input / output buffers;
    step 2 overflows.  The state after each step equals that of the in-place
    two-phase step run on the same sequence, eagerly and from a graph that
    holds the four calls (replayed twice, with eager work between)."""
    world, S, rank = 8, 400_003, 3
    say(f"speculative alternating buffers: world={world} S={S}")
    case = Case(world, S, rank, seed=77)
    pos = (2, S // 2)
    keep = case.grads[2][S // 2].clone()

    # in-place reference sequence
    ref = case.buffers()
    ref_call = case.call(ref, fp.FP_STEP_NO_COOP, False, 1)
    want = []
    for k in range(1, 5):
        if k == 2:
            case.grads[pos[0]][pos[1]] = 0x7F80
        ref["flag"].zero_()
        ref_call(k)
        torch.cuda.synchronize()
        case.grads[pos[0]][pos[1]] = keep
        want.append([t.clone() for t in (*ref["state"], ref["full"], ref["flag"])])

    b = case.buffers()
    A, B = b["state"], b["out"]
    calls = [case.call(b, fp.FP_STEP_EXACT_SKIP, True, 1, state=A, out=B),
             case.call(b, fp.FP_STEP_EXACT_SKIP, True, 1, state=B, out=A)]

    def run(k):
        b["flag"].zero_()
        calls[(k - 1) % 2](k)

    def check(k, what):
        cur = B if k % 2 == 1 else A
        for i, name in enumerate(("master", "exp_avg", "exp_avg_sq")):
            _same(cur[i], want[k - 1][i], f"{what} step {k}: {name}")
        _same(b["full"], want[k - 1][3], f"{what} step {k}: full")
        _same(b["flag"], want[k - 1][4], f"{what} step {k}: flag")

    for k in range(1, 5):
        if k == 2:
            case.grads[pos[0]][pos[1]] = 0x7F80
        run(k)
        torch.cuda.synchronize()
        case.grads[pos[0]][pos[1]] = keep
        check(k, "eager")

    # the four calls captured in one graph; each replay starts from the
    # initial state (no overflow this time) and must equal the same four
    # calls made eagerly from it
    graph = torch.cuda.CUDAGraph()
    for t, t0 in zip(A, case.state0):
        t.copy_(t0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for k in range(1, 5):
            run(k)
    torch.cuda.synchronize()
    for r in range(2):
        for t, t0 in zip(A, case.state0):
            t.copy_(t0)
        B[0].fill_(3.0)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (*A, *B, b["full"], b["flag"])]
        for t, t0 in zip(A, case.state0):
            t.copy_(t0)
        for k in range(1, 5):
            run(k)
        torch.cuda.synchronize()
        for i, (g, w) in enumerate(zip(got, (*A, *B, b["full"], b["flag"]))):
            _same(g, w, f"replay {r}: buffer {i}")
        x = torch.ones(1 << 20, device=dev())
        x.mul_(1.5)
        torch.cuda.synchronize()
    del graph
