"""Python access to the serial CPU oracle (liboracle.so, built from oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and
by bench.py's CPU-baseline leg, never by the product package.

All arrays are numpy arrays; bf16 values travel as uint16 bit patterns.
Functions that update state work in place on the arrays they are given.
"""

from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np

from . import build as _build

_lib = None
_lock = threading.Lock()

_i32, _i64, _f32, _f64, _vp = C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_void_p


def lib():
    """Load liboracle.so, compiling it first when it is missing or stale."""
    global _lib
    with _lock:
        if _lib is None:
            src_mtime = os.path.getmtime(_build.SRC)
            if (not os.path.exists(_build.LIB)
                    or os.path.getmtime(_build.LIB) < src_mtime):
                _build.build()
            L = C.CDLL(_build.LIB)
            sig = {
                "or_geometry": (None, [_i32, _vp, _i32, _vp, _vp, _vp]),
                "or_pack": (None, [_i32, _vp, _i32, _vp, _i32, _vp]),
                "or_locate_sorted": (None, [_i32, _vp, _i64, _vp, _vp, _vp]),
                "or_views": (_i32, [_i32, _vp, _i32, _i32, _vp, _vp, _vp]),
                "or_bf16_to_f32": (_f32, [C.c_uint16]),
                "or_f32_to_bf16": (C.c_uint16, [_f32]),
                "or_f32_to_bf16_array": (None, [_i64, _vp, _vp]),
                "or_reduce": (None, [_i64, _i32, _vp, _f32, _i32, _vp]),
                "or_reduce_hybrid": (None, [_i64, _i32, _i32, _vp, _f32, _i32, _vp]),
                "or_reshard": (None, [_i64, _i32, _i32, _i32, _i32, _vp, _vp]),
                "or_found_inf": (_i32, [_i64, _vp]),
                "or_sq_norm": (_f64, [_i64, _vp]),
                "or_adamw": (None, [_i64, _f64, _f64, _f64, _f64, _f64, _i64,
                                    _vp, _vp, _vp, _vp, _i32]),
                "or_unshard": (None, [_i64, _i32, _vp, _vp]),
                "or_adamw_coef": (None, [_i64, _f64, _f64, _f64, _f64, _f64, _i64, _f64,
                                         _vp, _vp, _vp, _vp, _i32]),
                "or_local_accumulate": (None, [_i64, _vp, _i32, _vp]),
                "or_local_finish": (None, [_i64, _vp, _i32, _vp, _vp]),
                "or_grad_coef": (_f64, [_f64, _f32, _f64]),
                "or_scaler_update": (None, [_i32, _vp, _vp, _f32, _f32, _i32]),
                "or_state_bytes": (_f64, [_f64, _i32, _f64, _i32]),
                "or_shard0_geometry": (None, [_i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
                "or_shard0_pack": (None, [_i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
                "or_shard0_unpack": (None, [_i32, _vp, _vp, _i32, _i32, _vp, _vp]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"expected C-contiguous {np.dtype(dtype)} array, got {a.dtype}")
    return a


def _ptr_table(arrays):
    return (C.c_void_p * len(arrays))(*[_ptr(a) for a in arrays])


# ---------------------------------------------------------------- geometry
def geometry(numels, world: int):
    n = np.ascontiguousarray(numels, dtype=np.int64)
    t, p, s = _i64(), _i64(), _i64()
    lib().or_geometry(len(n), _ptr(n), world, C.byref(t), C.byref(p), C.byref(s))
    return t.value, p.value, s.value


def pack(tensors, world: int) -> np.ndarray:
    """FlatParameter of the given arrays (all one dtype of 2 or 4 bytes)."""
    srcs = [np.ascontiguousarray(t).reshape(-1) for t in tensors]
    dtype = srcs[0].dtype
    if any(s.dtype != dtype for s in srcs) or dtype.itemsize not in (2, 4):
        raise TypeError("pack needs tensors of one 2- or 4-byte dtype")
    numel = np.array([s.size for s in srcs], dtype=np.int64)
    _, p, _ = geometry(numel, world)
    flat = np.empty(p, dtype=dtype)
    table = _ptr_table(srcs)
    lib().or_pack(len(srcs), _ptr(numel), dtype.itemsize, table, world, _ptr(flat))
    return flat


def locate_sorted(numels, positions):
    n = np.ascontiguousarray(numels, dtype=np.int64)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    if pos.size > 1 and np.any(np.diff(pos) < 0):
        raise ValueError("positions must be ascending")
    tensor = np.empty(pos.size, dtype=np.int32)
    offset = np.empty(pos.size, dtype=np.int64)
    lib().or_locate_sorted(len(n), _ptr(n), pos.size, _ptr(pos), _ptr(tensor), _ptr(offset))
    return tensor, offset


def views(numels, world: int, rank: int):
    """(buf_offset, length, tensor_offset) arrays, one row per tensor."""
    n = np.ascontiguousarray(numels, dtype=np.int64)
    bo = np.empty(len(n), dtype=np.int64)
    ln = np.empty(len(n), dtype=np.int64)
    to = np.empty(len(n), dtype=np.int64)
    lib().or_views(len(n), _ptr(n), world, rank, _ptr(bo), _ptr(ln), _ptr(to))
    return bo, ln, to


# ---------------------------------------------------------------- per-parameter dim-0 shards
def _shape_arrays(shapes):
    nd = np.array([len(s) for s in shapes], dtype=np.int32)
    dims = np.array([d for s in shapes for d in s] or [0], dtype=np.int64)
    return nd, dims


def shard0_geometry(shapes, world: int):
    """(rows c_i, row_elems r_i, offset_i, S) of the per-parameter dim-0 layout."""
    n = len(shapes)
    nd, dims = _shape_arrays(shapes)
    c, r, o = (np.empty(max(n, 1), dtype=np.int64) for _ in range(3))
    S = _i64()
    lib().or_shard0_geometry(n, _ptr(nd), _ptr(dims), world, _ptr(c), _ptr(r), _ptr(o), C.byref(S))
    return c[:n], r[:n], o[:n], S.value


def shard0_pack(tensors, world: int, rank: int) -> np.ndarray:
    """Rank `rank`'s buffer of the group (each parameter's dim-0 chunk, zero-padded)."""
    srcs = [np.ascontiguousarray(t) for t in tensors]
    dtype = srcs[0].dtype
    if any(x.dtype != dtype for x in srcs) or dtype.itemsize not in (2, 4):
        raise TypeError("shard0_pack needs tensors of one 2- or 4-byte dtype")
    shapes = [x.shape for x in srcs]
    _, _, _, S = shard0_geometry(shapes, world)
    nd, dims = _shape_arrays(shapes)
    out = np.empty(max(S, 1), dtype=dtype)
    lib().or_shard0_pack(len(srcs), _ptr(nd), _ptr(dims), world, dtype.itemsize, rank,
                         _ptr_table([x.reshape(-1) if x.size else np.zeros(1, dtype) for x in srcs]),
                         _ptr(out))
    return out[:S]


def shard0_unpack(full: np.ndarray, shapes, world: int):
    """The parameters (global shapes) from the ranks' buffers one after the other."""
    full = np.ascontiguousarray(full)
    nd, dims = _shape_arrays(shapes)
    outs = [np.empty(tuple(s), dtype=full.dtype) for s in shapes]
    lib().or_shard0_unpack(len(shapes), _ptr(nd), _ptr(dims), world, full.dtype.itemsize,
                           _ptr(full if full.size else np.zeros(1, full.dtype)),
                           _ptr_table([o.reshape(-1) if o.size else np.zeros(1, full.dtype) for o in outs]))
    return outs


def reshard(old_shards, numel: int, world_new: int, new_rank: int = -1) -> np.ndarray:
    """The new ranks' shards (new_rank = -1: all, concatenated) of a flat buffer
    of numel elements held as len(old_shards) old shards."""
    rows = [np.ascontiguousarray(x) for x in old_shards]
    dtype = rows[0].dtype
    if dtype.itemsize not in (2, 4) or any(r.dtype != dtype for r in rows):
        raise TypeError("reshard needs shards of one 2- or 4-byte dtype")
    N = len(rows)
    s_new = -(-numel // world_new)
    n_out = s_new * (world_new if new_rank < 0 else 1)
    out = np.empty(max(n_out, 1), dtype=dtype)
    lib().or_reshard(int(numel), N, int(world_new), dtype.itemsize, int(new_rank),
                     _ptr_table([r if r.size else np.zeros(1, dtype) for r in rows]), _ptr(out))
    return out[:n_out]


# ---------------------------------------------------------------- bf16
def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().or_f32_to_bf16_array(x.size, _ptr(x), _ptr(y))
    return y


# ---------------------------------------------------------------- reduce
def reduce(grads, scale: float, acc: np.ndarray = None, accumulate: bool = False) -> np.ndarray:
    """One micro-batch of the reduce: grads is a list of N uint16 arrays of length S."""
    grads = [_c(g, np.uint16) for g in grads]
    S = grads[0].size
    if any(g.size != S for g in grads):
        raise ValueError("rank gradients differ in length")
    if acc is None:
        if accumulate:
            raise ValueError("accumulate needs an accumulator")
        acc = np.empty(S, dtype=np.float32)
    acc = _c(acc, np.float32)
    lib().or_reduce(S, len(grads), _ptr_table(grads), np.float32(scale), int(bool(accumulate)),
                    _ptr(acc))
    return acc


def reduce_hybrid(grads, group: int, scale: float, acc: np.ndarray = None,
                  accumulate: bool = False) -> np.ndarray:
    """Two-level reduce of hybrid sharding: sums inside each group of `group`
    ranks, then across the groups, then one multiply by scale."""
    rows = [_c(g, np.uint16) for g in grads]
    S = rows[0].size
    if len(rows) % group != 0:
        raise ValueError("world must be a multiple of the group size")
    if acc is None:
        acc = np.zeros(S, np.float32)
    _c(acc, np.float32)
    lib().or_reduce_hybrid(S, len(rows), int(group), _ptr_table(rows), np.float32(scale),
                           int(bool(accumulate)), _ptr(acc))
    return acc


def found_inf(acc: np.ndarray) -> int:
    acc = _c(acc, np.float32)
    return int(lib().or_found_inf(acc.size, _ptr(acc)))


def sq_norm(acc: np.ndarray) -> float:
    acc = _c(acc, np.float32)
    return float(lib().or_sq_norm(acc.size, _ptr(acc)))


# ---------------------------------------------------------------- AdamW
def adamw(grad, master, exp_avg, exp_avg_sq, *, lr, beta1, beta2, eps,
          weight_decay, step: int, skip: bool = False, coef: float = None):
    """In-place AdamW on fp32 master / exp_avg / exp_avg_sq (fp64 arithmetic);
    with coef, every gradient element is first multiplied by it in fp64."""
    g = _c(grad, np.float32)
    arrs = [_c(a, np.float32) for a in (master, exp_avg, exp_avg_sq)]
    if any(a.size != g.size for a in arrs):
        raise ValueError("state arrays differ in length")
    if coef is None:
        lib().or_adamw(g.size, float(lr), float(beta1), float(beta2), float(eps),
                       float(weight_decay), int(step), _ptr(g), _ptr(arrs[0]),
                       _ptr(arrs[1]), _ptr(arrs[2]), int(bool(skip)))
    else:
        lib().or_adamw_coef(g.size, float(lr), float(beta1), float(beta2), float(eps),
                            float(weight_decay), int(step), float(coef), _ptr(g), _ptr(arrs[0]),
                            _ptr(arrs[1]), _ptr(arrs[2]), int(bool(skip)))


# ---------------------------------------------------------------- no_sync and the scaler
def local_accumulate(grad, local=None, accumulate: bool = False) -> np.ndarray:
    """A rank's fp32 local gradient sum after one more bf16 micro-batch (no exchange)."""
    g = _c(grad, np.uint16)
    out = np.empty(g.size, np.float32) if local is None else _c(local, np.float32)
    if out.size != g.size:
        raise ValueError("local buffer differs in length")
    lib().or_local_accumulate(g.size, _ptr(g), int(bool(accumulate)), _ptr(out))
    return out


def local_finish(grad, local=None, accumulate: bool = False) -> np.ndarray:
    """The rank's bf16 row for the exchange: bf16(local + grad), or bf16(grad)."""
    g = _c(grad, np.uint16)
    loc = np.zeros(g.size, np.float32) if local is None else _c(local, np.float32)
    out = np.empty(g.size, np.uint16)
    lib().or_local_finish(g.size, _ptr(g), int(bool(accumulate)), _ptr(loc), _ptr(out))
    return out


def grad_coef(sq_norm: float, loss_scale: float, max_norm: float) -> float:
    """fp64 factor for the loss-scaled reduced gradient: unscale, then clip."""
    return float(lib().or_grad_coef(float(sq_norm), np.float32(loss_scale), float(max_norm)))


def scaler_update(found_inf: int, scale: float, clean_steps: int, *, growth_factor: float = 2.0,
                  backoff_factor: float = 0.5, growth_interval: int = 2000):
    """(new fp32 scale, new clean-step count) after one step's overflow decision."""
    sc = np.array([scale], np.float32)
    cs = np.array([clean_steps], np.int32)
    lib().or_scaler_update(int(found_inf), _ptr(sc), _ptr(cs), np.float32(growth_factor),
                           np.float32(backoff_factor), int(growth_interval))
    return float(sc[0]), int(cs[0])


# ---------------------------------------------------------------- unshard
def unshard(shards) -> np.ndarray:
    shards = [_c(s, np.uint16) for s in shards]
    S = shards[0].size
    full = np.empty(S * len(shards), dtype=np.uint16)
    lib().or_unshard(S, len(shards), _ptr_table(shards), _ptr(full))
    return full


# ---------------------------------------------------------------- memory model
def state_bytes(psi: float, world: int, k: float, stage: int) -> float:
    return float(lib().or_state_bytes(float(psi), int(world), float(k), int(stage)))


# ---------------------------------------------------------------- whole step
def shard_step(micro_grads, acc, master, exp_avg, exp_avg_sq, other_shards, rank: int,
               *, hp, step: int):
    """One rank's shard step composed from the routines above.

    micro_grads[m][q]: rank q's bf16 gradient slice for micro-batch m.
    other_shards[q]: rank q's bf16 parameter shard (entry `rank` ignored).
    Updates acc / master / exp_avg / exp_avg_sq in place and returns
    (full bf16 buffer, found_inf, sq_norm).
    """
    n = len(micro_grads)
    world = len(micro_grads[0])
    scale = np.float32(1.0 / (world * n))
    for m, grads in enumerate(micro_grads):
        reduce(grads, scale, acc, accumulate=m > 0)
    flag = found_inf(acc)
    norm = sq_norm(acc)
    adamw(acc, master, exp_avg, exp_avg_sq, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2,
          eps=hp.eps, weight_decay=hp.weight_decay, step=step, skip=bool(flag))
    own = f32_to_bf16(master)
    shards = [own if q == rank else other_shards[q] for q in range(world)]
    return unshard(shards), flag, norm
