"""The one-pass step's grid barrier: its decision, the overflow flag it leaves,
and the give-up path.

* A wait that gives up (workgroups not resident together) must cancel the
  step for every workgroup alike: no state, no own-shard element and no
  accumulator element that is an input is written; FP_FLAG_GAVE_UP is OR-ed
  into the flag and bits already set survive.  The test entry
  fp_step_test_give_up forces that outcome from the host (a barrier that
  waits for one workgroup more than the launch holds, with a short wait), so
  every kernel still ends normally.  The step run again with FP_STEP_NO_COOP
  after clearing the bit gives the oracle's result.
* The flag is only ever OR-ed into: a bit left by an earlier call makes the
  one-pass step skip and stays set.
* Many consecutive one-pass calls on one workspace, with and without
  overflow, each take the right decision (the barrier's counters and its
  generation tag are reused correctly) and no wait gives up.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (assert_bf16_equal, assert_bf16_within_1ulp, assert_f32_bitexact,
                        assert_f32_close, dev, hp_kwargs, say, to_dev, to_host)
from workloads import gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()
CANARY_BF16 = 0x5A5A
CANARY_F32 = 7.0


def _bits(t):
    return t.contiguous().view(torch.uint8)


class OnePass:
    """One rank's one-pass step at N = 8 with host copies for the oracle."""

    def __init__(self, fp, S=100_003, world=8, rank=3, seed=41, inf_at=None):
        self.fp, self.S, self.world, self.rank = fp, S, world, rank
        g = [gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, 0, 0, q) for q in range(world)]
        if inf_at is not None:
            g[world - 1][inf_at] = 0x7F80
        o = [gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, 0, q) for q in range(world)]
        th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER, 0)
        m = gen.normal_f32(S, 1e-4, seed, gen.STREAM_EXP_AVG, 0)
        v = np.square(gen.normal_f32(S, 1e-3, seed, gen.STREAM_EXP_AVG_SQ, 0))
        self.host = dict(grads=g, others=o, state=(th, m, v))
        self.grads = to_dev(np.stack(g))
        self.shards = [None if q == rank else to_dev(o[q]) for q in range(world)]
        self.state = [to_dev(x) for x in (th, m, v)]
        self.state0 = [t.clone() for t in self.state]
        self.acc = torch.full((S,), CANARY_F32, dtype=torch.float32, device=dev())
        self.full = torch.full((world * S,), CANARY_BF16, dtype=torch.int16, device=dev())
        self.flag = torch.zeros(1, dtype=torch.int32, device=dev())
        self.ws = fp.new_workspace(dev(), S)

    def call(self, flags=0, out=None):
        return self.fp.ShardStep(self.grads, self.acc, *self.state, self.shards, self.full, self.rank,
                                 scale=1.0 / self.world, found_inf=self.flag, workspace=self.ws, flags=flags,
                                 out=out, **hp_kwargs(HP))

    def oracle_step(self, step):
        h = self.host
        th, m, v = (x.copy() for x in h["state"])
        acc = np.zeros(self.S, np.float32)
        full, flag, _ = oracle.shard_step([h["grads"]], acc, th, m, v, h["others"], self.rank, hp=HP, step=step)
        return acc, (th, m, v), full, flag

    def own(self):
        return self.full[self.rank * self.S:(self.rank + 1) * self.S]


@pytest.mark.parametrize("keep_grad", [False, True])
@pytest.mark.parametrize("prior", [0, 1])
def test_give_up_stores_nothing_and_keeps_the_flag(fp, prior, keep_grad):
    say(f"one-pass give-up: prior flag {prior}, keep_grad {keep_grad}")
    c = OnePass(fp)
    flags = fp.FP_STEP_KEEP_GRAD if keep_grad else 0
    step = c.call(flags)
    assert step.path() == fp.FP_PATH_ONE_PASS
    c.flag.fill_(prior)
    step.test_give_up(2)
    torch.cuda.synchronize()
    assert int(c.flag.item()) == prior | fp.FP_FLAG_GAVE_UP
    assert fp.workspace_timeouts(c.ws) > 0
    for t, t0, name in zip(c.state, c.state0, ("master", "exp_avg", "exp_avg_sq")):
        assert torch.equal(_bits(t), _bits(t0)), f"{name} written by a cancelled step"
    assert bool((c.own() == CANARY_BF16).all()), "own shard written by a cancelled step"
    acc_o, state_o, full_o, flag_o = c.oracle_step(2)
    fh = to_host(c.full)
    own = slice(c.rank * c.S, (c.rank + 1) * c.S)
    mask = np.ones(c.world * c.S, bool)
    mask[own] = False
    assert_bf16_equal(fh[mask], full_o[mask], "other shards (copied beside the barrier)")
    if keep_grad:
        assert_f32_bitexact(to_host(c.acc), acc_o, "kept reduced gradient")
    else:
        assert bool((c.acc == CANARY_F32).all()), "acc written by a cancelled step"

    # the caller's recovery: clear the bit, fresh barrier state, the two-kernel form
    c.flag.bitwise_and_(fp.FP_FLAG_OVERFLOW)
    c.ws.zero_()
    c.call(flags | fp.FP_STEP_NO_COOP)(2)
    torch.cuda.synchronize()
    assert int(c.flag.item()) == (prior | flag_o)
    skip = bool(prior or flag_o)
    th0, m0, v0 = c.host["state"]
    if skip:
        for t, t0 in zip(c.state, c.state0):
            assert torch.equal(_bits(t), _bits(t0))
        assert_bf16_equal(to_host(c.own()), oracle.f32_to_bf16(th0), "own shard of a skipped step")
    else:
        for t, w, name in zip(c.state, state_o, ("master", "exp_avg", "exp_avg_sq")):
            assert_f32_close(to_host(t), w, name)
        assert_bf16_within_1ulp(to_host(c.own()), full_o[own], "own shard")


@pytest.mark.parametrize("inject", [False, True])
def test_speculative_one_pass_give_up_and_decisions(fp, inject):
    """The one-pass kernel with separate output state: a give-up writes neither
    the inputs nor the outputs; run normally, the outputs get the update, or
    on overflow the input state, and the inputs stay untouched."""
    say(f"speculative one-pass: give-up, then a normal call (overflow {inject})")
    c = OnePass(fp, S=90_001, seed=44, inf_at=777 if inject else None)
    out = [torch.full((c.S,), CANARY_F32, dtype=torch.float32, device=dev()) for _ in range(3)]
    step = c.call(out=out)
    assert step.path() == fp.FP_PATH_SPECULATIVE_ONE_PASS
    step.test_give_up(3)
    torch.cuda.synchronize()
    assert int(c.flag.item()) == fp.FP_FLAG_GAVE_UP
    assert all(bool((t == CANARY_F32).all()) for t in out), "outputs written by a cancelled step"
    assert bool((c.own() == CANARY_BF16).all())
    c.flag.zero_()
    c.ws.zero_()
    step(3)
    torch.cuda.synchronize()
    assert int(c.flag.item()) == int(inject)
    for t, t0 in zip(c.state, c.state0):
        assert torch.equal(_bits(t), _bits(t0)), "input state written"
    acc_o, state_o, full_o, flag_o = c.oracle_step(3)
    assert flag_o == int(inject)
    for t, w, name in zip(out, state_o, ("master", "exp_avg", "exp_avg_sq")):
        if inject:
            assert_f32_bitexact(to_host(t), w, f"{name} of a skipped step")
        else:
            assert_f32_close(to_host(t), w, name)
    own = slice(c.rank * c.S, (c.rank + 1) * c.S)
    assert_bf16_within_1ulp(to_host(c.own()), full_o[own], "own shard")


@pytest.mark.parametrize("prior", [2, 3])
def test_one_pass_never_clears_the_flag(fp, prior):
    """Bits left by an earlier call (a give-up, an overflow) make the step skip
    and stay set; the own shard gets the cast of the unchanged master."""
    say(f"one-pass with prior flag {prior}")
    c = OnePass(fp, S=70_001, seed=42)
    step = c.call()
    assert step.path() == fp.FP_PATH_ONE_PASS
    c.flag.fill_(prior)
    step(4)
    torch.cuda.synchronize()
    assert int(c.flag.item()) == prior | fp.FP_FLAG_OVERFLOW
    for t, t0 in zip(c.state, c.state0):
        assert torch.equal(_bits(t), _bits(t0))
    assert_bf16_equal(to_host(c.own()), oracle.f32_to_bf16(c.host["state"][0]), "own shard")
    assert fp.workspace_timeouts(c.ws) == 0


def test_one_pass_decisions_over_many_calls(fp):
    """Twelve one-pass calls on one workspace alternating finite and overflowed
    gradients: every decision right, state updated only on finite calls."""
    say("one-pass: 12 consecutive calls, alternating overflow")
    fin = OnePass(fp, S=50_000, seed=43)
    bad = OnePass(fp, S=50_000, seed=43, inf_at=12_345)
    ws = fp.new_workspace(dev(), fin.S)
    for c in (fin, bad):
        c.ws = ws
    steps = {id(c): c.call() for c in (fin, bad)}
    th, m, v = (x.copy() for x in fin.host["state"])
    t = 0
    for k in range(12):
        c = bad if k % 3 == 1 else fin
        c.flag.zero_()
        if c is fin:
            t += 1
            steps[id(c)](t)
        else:
            c.state = [x.clone() for x in fin.state]
            steps[id(c)] = c.call()
            steps[id(c)](t + 1)
        torch.cuda.synchronize()
        if c is fin:
            assert int(c.flag.item()) == 0, f"call {k}"
            acc = oracle.reduce(fin.host["grads"], np.float32(1.0 / fin.world))
            oracle.adamw(acc, th, m, v, step=t, **hp_kwargs(HP))
            for g, w in zip(fin.state, (th, m, v)):
                assert_f32_close(to_host(g), w, f"call {k}")
        else:
            assert int(c.flag.item()) == 1, f"call {k}"
            for g, w in zip(c.state, fin.state):
                assert torch.equal(_bits(g), _bits(w)), f"call {k}: overflowed step updated the state"
    assert fp.workspace_timeouts(ws) == 0
