"""Pins of the oracle's AdamW shard update.

The pages name AdamW and fix its state (fp32 master, two fp32 moments,
k = 12 bytes per parameter; "Infra: Data Parallel" ZeRO figure legend,
"4.1 数据并行详解" section 7) but do not write the update; the oracle
follows decoupled weight decay (Loshchilov & Hutter) with bias correction.

What fixes the expected values:
* closed forms: at step 1 the bias-corrected moments are g and g^2, so the
  update is lr * g / (|g| + eps); with g = 0 only the decay acts; with a
  constant gradient and no decay every step moves by lr * g / (|g| + eps);
* torch.optim.AdamW (a library implementation of the same update) run in
  float64 from the same fp32 state, one step at a time;
* the elementwise property of "Infra: Data Parallel" (ZeRO-1 paragraph):
  updating the shards one by one equals updating the whole buffer.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen
from workloads.configs import AdamW

HP = AdamW()


def _ulp_dist(a, b):
    """Distance in units of the last place between float32 arrays (sign-magnitude ordered)."""
    def key(x):
        i = x.view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7FFFFFFF), i)
    return np.abs(key(np.asarray(a, np.float32)) - key(np.asarray(b, np.float32)))


def _run(grad, master, m, v, step, hp=HP, skip=False):
    master, m, v = master.copy(), m.copy(), v.copy()
    oracle.adamw(grad, master, m, v, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                 weight_decay=hp.weight_decay, step=step, skip=skip)
    return master, m, v


def test_first_step_closed_form():
    S = 4096
    g = gen.normal_f32(S, 1.0, 1, gen.STREAM_GRAD)
    th = gen.normal_f32(S, 0.02, 1, gen.STREAM_MASTER)
    z = np.zeros(S, np.float32)
    t1, m1, v1 = _run(g, th, z, z, step=1)
    g64, th64 = g.astype(np.float64), th.astype(np.float64)
    np.testing.assert_allclose(m1, (1 - HP.beta1) * g64, rtol=1e-7, atol=0)
    np.testing.assert_allclose(v1, (1 - HP.beta2) * g64 ** 2, rtol=1e-7, atol=0)
    want = th64 * (1 - HP.lr * HP.weight_decay) - HP.lr * g64 / (np.abs(g64) + HP.eps)
    np.testing.assert_allclose(t1, want, rtol=1e-6, atol=1e-9)
    assert _ulp_dist(t1, want.astype(np.float32)).max() <= 1


def test_zero_gradient_only_decays():
    S = 1000
    th = gen.normal_f32(S, 1.0, 2, gen.STREAM_MASTER)
    z = np.zeros(S, np.float32)
    for step in (1, 2, 50):
        t1, m1, v1 = _run(z, th, z, z, step=step)
        np.testing.assert_array_equal(m1, z)
        np.testing.assert_array_equal(v1, z)
        want = (th.astype(np.float64) * (1 - HP.lr * HP.weight_decay)).astype(np.float32)
        np.testing.assert_array_equal(t1, want)


def test_constant_gradient_moves_by_lr_per_step():
    S, steps = 512, 20
    hp = AdamW(weight_decay=0.0)
    g = gen.normal_f32(S, 1e-2, 3, gen.STREAM_GRAD)
    th0 = gen.normal_f32(S, 0.02, 3, gen.STREAM_MASTER)
    th, m, v = th0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    for t in range(1, steps + 1):
        th, m, v = _run(g, th, m, v, step=t, hp=hp)
        g64 = g.astype(np.float64)
        want = th0.astype(np.float64) - t * hp.lr * g64 / (np.abs(g64) + hp.eps)
        # theta is rounded to fp32 after every step (half an ulp each) and the
        # stored moments carry a relative error of about t * 2^-24
        atol = t * (2.0 ** -24 * np.abs(th0).max() * 1.5 + hp.lr * t * 2.0 ** -23)
        np.testing.assert_allclose(th, want, rtol=0, atol=atol)
        np.testing.assert_allclose(m, (1 - hp.beta1 ** t) * g64, rtol=1e-6)
        np.testing.assert_allclose(v, (1 - hp.beta2 ** t) * g64 ** 2, rtol=1e-6)


@pytest.mark.parametrize("step,scale", [(1, 1.0), (2, 1e-3), (3, 1.0), (10, 3e-4), (1000, 1e-2)])
def test_matches_torch_adamw_float64(step, scale):
    S = 2000
    g = gen.normal_f32(S, scale, step, gen.STREAM_GRAD)
    th = gen.normal_f32(S, 0.02, step, gen.STREAM_MASTER)
    m = gen.normal_f32(S, scale * 0.3, step, gen.STREAM_EXP_AVG) if step > 1 else np.zeros(S, np.float32)
    v = (gen.normal_f32(S, scale, step, gen.STREAM_EXP_AVG_SQ) ** 2 if step > 1
         else np.zeros(S, np.float32))
    t1, m1, v1 = _run(g, th, m, v, step=step)

    p = torch.nn.Parameter(torch.from_numpy(th.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                            weight_decay=HP.weight_decay, foreach=False)
    if step > 1:
        opt.state[p] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                        "exp_avg": torch.from_numpy(m.astype(np.float64)),
                        "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    p.grad = torch.from_numpy(g.astype(np.float64))
    opt.step()
    st = opt.state[p]
    for got, ref in ((t1, p.detach().numpy()), (m1, st["exp_avg"].numpy()), (v1, st["exp_avg_sq"].numpy())):
        # oracle = one rounding of the fp64 result; torch's fp64 differs by ~1e-16
        assert _ulp_dist(got, ref.astype(np.float32)).max() <= 1
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-9)


def test_skip_leaves_state_untouched():
    S = 300
    g = gen.normal_f32(S, 1.0, 4, gen.STREAM_GRAD)
    th = gen.normal_f32(S, 0.02, 4, gen.STREAM_MASTER)
    m = gen.normal_f32(S, 0.1, 4, gen.STREAM_EXP_AVG)
    v = np.abs(gen.normal_f32(S, 0.1, 4, gen.STREAM_EXP_AVG_SQ))
    t1, m1, v1 = _run(g, th, m, v, step=5, skip=True)
    for a, b in ((t1, th), (m1, m), (v1, v)):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("world", [2, 3, 8])
def test_shardwise_update_equals_whole_buffer_update(world):
    S = 97
    P = world * S
    g = gen.normal_f32(P, 1e-3, 5, gen.STREAM_GRAD)
    th = gen.normal_f32(P, 0.02, 5, gen.STREAM_MASTER)
    m = gen.normal_f32(P, 1e-4, 5, gen.STREAM_EXP_AVG)
    v = gen.normal_f32(P, 1e-3, 5, gen.STREAM_EXP_AVG_SQ) ** 2
    whole = _run(g, th, m, v, step=7)
    parts = [_run(g[r * S:(r + 1) * S].copy(), th[r * S:(r + 1) * S].copy(),
                  m[r * S:(r + 1) * S].copy(), v[r * S:(r + 1) * S].copy(), step=7) for r in range(world)]
    for k in range(3):
        np.testing.assert_array_equal(np.concatenate([p[k] for p in parts]).view(np.uint32),
                                      whole[k].view(np.uint32))
