"""fp_shard_step_noalloc against fp_shard_step with a workspace.

The entry point for callers that cannot allocate keeps the step's scratch
(grid-barrier state, norm partials) in an array inside the library.  Its
results must equal, bit for bit, those of fp_shard_step with a
caller-provided workspace on the same inputs: here on three calls in a row
on one GPU -- a one-pass-sized shard with the gradient norm, then a smaller
one at another N_d and rank with an overflow (the barrier's decision), then
a two-kernel step with the norm -- so that the library's array is reused by
every call after the first.
"""

import numpy as np
import pytest
import torch

from gpu_common import dev, hp_kwargs, say, to_dev
from workloads import gen
from workloads.configs import AdamW

pytestmark = pytest.mark.gpu
HP = AdamW()


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _inputs(world, S, rank, seed, inf_at=None):
    g = np.stack([gen.bf16_normal(S, 1e-3, seed, gen.STREAM_GRAD, 0, 0, q) for q in range(world)])
    if inf_at is not None:
        g[world - 1, inf_at] = 0x7F80
    o = [gen.bf16_normal(S, 0.02, seed, gen.STREAM_SHARD, 0, q) for q in range(world)]
    th = gen.normal_f32(S, 0.02, seed, gen.STREAM_MASTER, 0)
    m = gen.normal_f32(S, 1e-4, seed, gen.STREAM_EXP_AVG, 0)
    v = np.square(gen.normal_f32(S, 1e-3, seed, gen.STREAM_EXP_AVG_SQ, 0))
    return dict(grads=to_dev(g), shards=[None if q == rank else to_dev(o[q]) for q in range(world)],
                state=[to_dev(x) for x in (th, m, v)])


def _run(fp, inp, world, S, rank, flags, with_norm, library_scratch, step):
    b = dict(acc=torch.zeros(S, dtype=torch.float32, device=dev()),
             state=[t.clone() for t in inp["state"]],
             full=torch.zeros(world * S, dtype=torch.int16, device=dev()),
             flag=torch.zeros(1, dtype=torch.int32, device=dev()),
             sq=torch.full((1,), -1.0, dtype=torch.float64, device=dev()) if with_norm else None)
    ws = None if library_scratch else fp.new_workspace(dev(), S)
    call = fp.ShardStep(inp["grads"], b["acc"], *b["state"], inp["shards"], b["full"], rank,
                        scale=1.0 / world, found_inf=b["flag"], sq_norm=b["sq"], workspace=ws, flags=flags,
                        library_scratch=library_scratch, **hp_kwargs(HP))
    path = call.path() if not library_scratch else None
    call(step)
    torch.cuda.synchronize()
    return b, path


CASES = [  # (world, S, rank, flags, with_norm, inf_at): each call smaller than or unlike the one before
    (8, 1_574_528, 1, 2, True, None),       # one-pass path, kept gradient, norm
    (3, 100_003, 2, 0, False, 4_321),       # smaller, overflow: the barrier's decision
    (16, 65_537, 0, 4, True, None),         # two-kernel path with the norm partials
]


def test_noalloc_step_equals_workspace_step(fp):
    for k, (world, S, rank, flags, with_norm, inf_at) in enumerate(CASES):
        say(f"no-alloc call {k}: world={world} S={S} rank={rank} flags={flags} norm={with_norm} inf={inf_at}")
        inp = _inputs(world, S, rank, 70 + k, inf_at)
        want, path = _run(fp, inp, world, S, rank, flags, with_norm, False, k + 1)
        got, _ = _run(fp, inp, world, S, rank, flags, with_norm, True, k + 1)
        if k == 0:
            assert path == fp.FP_PATH_ONE_PASS
        assert int(got["flag"].item()) == int(want["flag"].item()) == (1 if inf_at is not None else 0)
        for name in ("acc", "full"):
            if name == "acc" and not flags & fp.FP_STEP_KEEP_GRAD:
                continue
            assert torch.equal(_bits(got[name]), _bits(want[name])), f"call {k}: {name}"
        for g, w_, nm in zip(got["state"], want["state"], ("master", "exp_avg", "exp_avg_sq")):
            assert torch.equal(_bits(g), _bits(w_)), f"call {k}: {nm}"
        if with_norm:
            assert float(got["sq"].item()) == float(want["sq"].item()) >= 0.0, f"call {k}: norm"
