"""Helpers shared by the GPU parity tests: device buffers from host arrays and
the comparison rules.

Comparison rules:
* integer / byte work (pack, unshard, views) and the fixed-order reduce:
  bitwise, except that non-finite floats compare by class (NaN, +inf,
  -inf), since NaN payloads are not specified;
* AdamW fp32 state: |got - oracle| <= 1e-9 + 1e-6 * |oracle| per element;
* bf16 parameters: at most 1 ulp apart (ordered-integer distance).
"""

from __future__ import annotations

import sys

import numpy as np
import torch

ATOL, RTOL = 1e-9, 1e-6


def say(*args):
    """Print a progress line at once, so that a failing run names its case."""
    print(*args, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev())
    return torch.from_numpy(a).to(dev())


def to_host(t) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        return a.view(np.uint16)
    return a


def f32_class(x: np.ndarray) -> np.ndarray:
    """0 finite, 1 NaN, 2 +inf, 3 -inf."""
    c = np.zeros(x.shape, np.int8)
    c[np.isnan(x)] = 1
    c[np.isposinf(x)] = 2
    c[np.isneginf(x)] = 3
    return c


def assert_f32_bitexact(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    cg, cw = f32_class(got), f32_class(want)
    bad = cg != cw
    fin = (cg == 0) & (cw == 0)
    bad |= fin & (got.view(np.uint32) != want.view(np.uint32))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first at {i}: "
                             f"got {got[i]!r} ({got.view(np.uint32)[i]:#010x}) "
                             f"want {want[i]!r} ({want.view(np.uint32)[i]:#010x})")


def assert_f32_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    cg, cw = f32_class(got), f32_class(want)
    assert np.array_equal(cg, cw), f"{what}: non-finite classes differ"
    fin = cw == 0
    err = np.abs(got[fin].astype(np.float64) - want[fin].astype(np.float64))
    tol = ATOL + RTOL * np.abs(want[fin].astype(np.float64))
    bad = err > tol
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside 1e-6 rel / 1e-9 abs; "
                             f"first: got {got[fin][i]!r} want {want[fin][i]!r}")


def bf16_is_nan(h: np.ndarray) -> np.ndarray:
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def key(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    d = np.abs(key(a) - key(b))
    both_nan = bf16_is_nan(a) & bf16_is_nan(b)
    d[both_nan] = 0
    return d


def assert_bf16_within_1ulp(got: np.ndarray, want: np.ndarray, what: str = ""):
    d = bf16_ulp_distance(np.asarray(got, np.uint16), np.asarray(want, np.uint16))
    if (d > 1).any():
        i = int(np.flatnonzero(d > 1)[0])
        raise AssertionError(f"{what}: {int((d > 1).sum())} bf16 values > 1 ulp apart; "
                             f"first at {i}: got {got[i]:#06x} want {want[i]:#06x}")


def assert_bf16_equal(got: np.ndarray, want: np.ndarray, what: str = ""):
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    bad = (got != want) & ~(bf16_is_nan(got) & bf16_is_nan(want))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} bf16 values differ; "
                             f"first at {i}: got {got[i]:#06x} want {want[i]:#06x}")


def norm_rel_tol(n: int) -> float:
    """Relative tolerance of a GPU sum of n squares against the oracle's serial
    fp64 sum: each order's rounding error is below n * 2^-53 of the sum of
    non-negative terms (recursive summation bound), so the two differ by at
    most twice that (floored at 1e-12)."""
    return max(1e-12, 2.0 * n * 2.0 ** -53)


def hp_kwargs(hp):
    return dict(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay)
