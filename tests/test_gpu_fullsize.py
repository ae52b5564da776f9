"""Full-array oracle parity of the step at the workloads' full sizes, built and
launched exactly as bench.py times them (its workload classes, one buffer set).

* 611M-parameter model in 47 buckets of 25 MiB (46 x 819,200 + 504,300
  elements per rank), N_d = 16, 4 micro-batches, rank 0: three multi-unit
  reduce launches and the multi-unit step, in place (two-phase) and
  speculative (separate output partitions), compared with the oracle on
  every element of the 38.2M-element partition: the reduced gradient
  bitwise, the fp32 state within 1e-6 rel / 1e-9 abs, every bucket's own
  bf16 shard within 1 ulp and its other shards bitwise; then the same with
  one +inf in the last bucket (the whole step skipped).
* d=12288 layer unit, N_d = 8, rank 0 (226.5M-element shard): two steps
  (t = 1 and t = 2) of the in-place exact skip (two-phase; its reduced
  gradient in acc bitwise) and of the speculative step (split launches),
  every element against the oracle.
* 10k ragged tensors at N_d = 64 (42.6M-element shard), ranks 0 and 63:
  one step of each form, every element against the oracle.
The oracle is the serial C code of oracle/, fed the same input bytes copied
back from the device.
"""

import numpy as np
import pytest
import torch

import bench
import oracle
from gpu_common import assert_bf16_within_1ulp, assert_f32_bitexact, assert_f32_close, dev, hp_kwargs, say, to_host
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

MODES = {"inplace_exact": (0, False), "speculative": (0, True)}


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _host_rows(rows):
    """[N, S] (or a list of N 1-D) int16 device tensors -> list of N contiguous host uint16 arrays."""
    return [np.ascontiguousarray(to_host(r)) for r in rows]


# ------------------------------------------------------------------ 611M buckets
@pytest.mark.parametrize("inject", [False, True])
@pytest.mark.parametrize("mode", list(MODES))
def test_611m_buckets_as_benchmarked(fp, mode, inject):
    cfg = CONFIGS["c3_611m_buckets_nd16"]
    flags, oop = MODES[mode]
    rank, N, n = cfg.ranks[0], cfg.world, cfg.n_micro
    say(f"611M buckets as benchmarked: mode={mode} inject={inject}")
    w = bench.Bucketed(cfg, rank, dev(), flags, oop, n_sets=1)
    assert w.path == (fp.FP_PATH_SPECULATIVE_SPLIT if oop else fp.FP_PATH_TWO_PHASE)
    s = w.sets[0]
    sizes, offs = w.sizes, w.offsets
    assert len(sizes) == 47 and sizes[:46] == [819_200] * 46 and sizes[46] == 504_300
    assert s["plans"][0].offsets == offs and s["plans"][0].partition == w.S == 38_187_500
    if inject:                                    # one +inf in the last bucket, last micro-batch
        s["grads"][n - 1][N - 1, offs[46] + 12_345] = 0x7F80
    S = w.S
    grads = [_host_rows(s["grads"][m][:, :S]) for m in range(n)]
    state_in, state_out = w.state_io(0)
    th0, m0, v0 = (to_host(t).copy() for t in state_in)
    w.step(0)
    torch.cuda.synchronize()
    scale = np.float32(1.0 / (N * n))
    acc_o = np.zeros(S, np.float32)
    for b, (o, Sb) in enumerate(zip(offs, sizes)):
        for m in range(n):
            oracle.reduce([g[o:o + Sb] for g in grads[m]], scale, acc_o[o:o + Sb], accumulate=m > 0)
    flag_o = oracle.found_inf(acc_o)
    assert flag_o == int(inject)
    assert int(s["found_inf"].item()) == flag_o
    if not oop:
        assert_f32_bitexact(to_host(s["acc"]), acc_o, "reduced gradient of the partition")
    th, m_, v = th0.copy(), m0.copy(), v0.copy()
    oracle.adamw(acc_o, th, m_, v, step=1, skip=bool(flag_o), **hp_kwargs(cfg.hp))
    result = state_out if oop else state_in
    if oop:
        for t, h in zip(state_in, (th0, m0, v0)):
            assert np.array_equal(to_host(t).view(np.uint32), h.view(np.uint32)), "input state written"
    for t, want, name in zip(result, (th, m_, v), ("master", "exp_avg", "exp_avg_sq")):
        got = to_host(t)
        if flag_o:
            assert_f32_bitexact(got, want, f"{name} of a skipped step")
        else:
            assert_f32_close(got, want, name)
    own_o = oracle.f32_to_bf16(th)
    for b, (o, Sb) in enumerate(zip(offs, sizes)):
        full = s["full"][b]
        own = full[rank * Sb:(rank + 1) * Sb]
        assert_bf16_within_1ulp(to_host(own), own_o[o:o + Sb], f"bucket {b} own shard")
        for q in range(N):
            if q != rank:
                assert torch.equal(full[q * Sb:(q + 1) * Sb], s["others"][q, o:o + Sb]), f"bucket {b} shard {q}"


# ------------------------------------------------------------------ single units
def _single_unit_steps(fp, name, rank, mode, steps):
    cfg = CONFIGS[name]
    flags, oop = MODES[mode]
    N = cfg.world
    w = bench.SingleUnit(cfg, rank, dev(), flags, oop, n_sets=1)
    s = w.sets[0]
    S = w.S
    say(f"{name} rank={rank} mode={mode} S={S} path={bench.PATH_NAMES[w.path]}")
    grads = _host_rows(s["grads"])
    state_in, _ = w.state_io(0)
    th, m, v = (to_host(t).copy() for t in state_in)
    for i in range(steps):
        state_in, state_out = w.state_io(i)
        before = [t.clone() for t in state_in] if oop else None
        w.step(i)
        torch.cuda.synchronize()
        assert int(s["found_inf"].item()) == 0
        acc = oracle.reduce(grads, np.float32(1.0 / N))
        assert oracle.found_inf(acc) == 0
        oracle.adamw(acc, th, m, v, step=i + 1, **hp_kwargs(cfg.hp))
        if oop:
            for t, t0 in zip(state_in, before):
                assert torch.equal(_bits(t), _bits(t0)), "input state written"
            del before
        else:                                     # the two-phase step passes the reduced gradient through acc
            assert_f32_bitexact(to_host(s["acc"]), acc, f"reduced gradient of step {i + 1}")
        result = state_out if oop else state_in
        for t, want, nm in zip(result, (th, m, v), ("master", "exp_avg", "exp_avg_sq")):
            assert_f32_close(to_host(t), want, f"{nm} after step {i + 1}")
        full = s["full"]
        assert_bf16_within_1ulp(to_host(full[rank * S:(rank + 1) * S]), oracle.f32_to_bf16(th),
                                f"own shard after step {i + 1}")
        for q in range(N):
            if q != rank:
                assert torch.equal(full[q * S:(q + 1) * S], s["shards"][q]), f"shard {q} after step {i + 1}"
    assert fp.workspace_timeouts(s["workspace"]) == 0
    return w


@pytest.mark.parametrize("mode", list(MODES))
def test_d12288_layer_two_steps_every_element(fp, mode):
    cfg = CONFIGS["c4_layer_d12288_nd8"]
    w = _single_unit_steps(fp, cfg.name, cfg.ranks[0], mode, steps=2)
    assert w.path == (fp.FP_PATH_SPECULATIVE_SPLIT if MODES[mode][1] else fp.FP_PATH_TWO_PHASE)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("rank", [0, 63])
def test_ragged_10k_step_every_element(fp, rank, mode):
    cfg = CONFIGS["c5_ragged10k_nd64"]
    w = _single_unit_steps(fp, cfg.name, rank, mode, steps=1)
    assert w.path == (fp.FP_PATH_SPECULATIVE_SPLIT if MODES[mode][1] else fp.FP_PATH_TWO_PHASE)
