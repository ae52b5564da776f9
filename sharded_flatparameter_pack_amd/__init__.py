"""One rank's FSDP / ZeRO shard step on AMD Instinct MI355X (gfx950).

A thin binding of libflatparam.so (include/flatparam.h): it checks and
marshals torch tensors (device memory) and torch's current stream into
the C ABI; every step of the path runs in the library's HIP kernels.

    plan = Plan(shapes, world)            # FlatParameter geometry (host)
    flat = plan.pack(tensors)             # flatten + concatenate + pad (GPU)
    views = plan.views(flat)              # original tensors as views
    reduce_shard(grads, acc, scale=...)   # bf16 -> fp32 reduce, overflow flag
    adamw_shard(acc, master, m, v, ...)   # fp32 AdamW + bf16 cast
    unshard(shards, full)                 # gather the bf16 shards
    shard_step(...)                       # the whole step for the last micro-batch
"""

from __future__ import annotations

import ctypes as C
import math
from typing import Optional, Sequence

from . import _lib
from ._lib import (FP_MAX_WORLD, FP_PATH_NO_SKIP, FP_PATH_NO_SKIP_SPLIT, FP_PATH_ONE_PASS,  # noqa: F401
                   FP_PATH_SPECULATIVE, FP_PATH_SPECULATIVE_ONE_PASS, FP_PATH_SPECULATIVE_SPLIT,
                   FP_PATH_TWO_PHASE, FP_STEP_EXACT_SKIP, FP_STEP_KEEP_GRAD, FP_STEP_NO_COOP,
                   FP_STEP_NO_SKIP, FP_FLAG_OVERFLOW, FP_FLAG_GAVE_UP, FlatParamError, check, lib)

__all__ = ["Plan", "Units", "Shard0Plan", "ReshardPlan", "reduce_shard_hybrid", "local_accumulate", "local_finish", "grad_coef", "scaler_update", "reduce_shard", "adamw_shard", "unshard", "shard_step", "ShardStep", "state_bytes",
           "workspace_bytes", "new_workspace", "workspace_timeouts", "FlatParamError", "FP_STEP_EXACT_SKIP",
           "FP_STEP_NO_SKIP", "FP_STEP_KEEP_GRAD", "FP_STEP_NO_COOP", "FP_PATH_ONE_PASS",
           "FP_PATH_TWO_PHASE", "FP_PATH_NO_SKIP", "FP_PATH_NO_SKIP_SPLIT", "FP_PATH_SPECULATIVE",
           "FP_PATH_SPECULATIVE_SPLIT", "FP_PATH_SPECULATIVE_ONE_PASS", "FP_FLAG_OVERFLOW", "FP_FLAG_GAVE_UP", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


_BF16_DTYPES = None


def _bf16_dtypes():
    global _BF16_DTYPES
    if _BF16_DTYPES is None:
        torch = _torch()
        _BF16_DTYPES = tuple(d for d in (torch.bfloat16, torch.int16, getattr(torch, "uint16", None)) if d)
    return _BF16_DTYPES


def _stream(t):
    device = t if isinstance(t, _torch().device) else t.device
    return C.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _dev_ptr(t, dtypes, n, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, needs {n}")
    return t.data_ptr()


def _one_device(*objs):
    """All tensors of one call (nested lists and [N, S] tensors included) on one device."""
    devs = set()
    todo = list(objs)
    while todo:
        o = todo.pop()
        if o is None:
            continue
        if isinstance(o, (list, tuple)):
            todo.extend(o)
        else:
            devs.add(o.device)
    if len(devs) > 1:
        raise ValueError(f"tensors of one call sit on several devices: {sorted(map(str, devs))}")


def _f32(t, n, name):
    return _dev_ptr(t, (_torch().float32,), n, name)


def _bf16(t, n, name):
    return _dev_ptr(t, _bf16_dtypes(), n, name)


def _rank_ptrs(x, n, name, allow_none=False):
    """Device pointers of N bf16 rows: a list of 1-D tensors or one [N, >=n] tensor."""
    if hasattr(x, "dim") and x.dim() == 2:
        if not x.is_cuda or x.dtype not in _bf16_dtypes() or x.stride(1) != 1 or x.shape[1] < n:
            raise ValueError(f"{name}: need a device bf16 [N, >= {n}] tensor with unit column stride")
        base, step = x.data_ptr(), x.stride(0) * x.element_size()
        return [base + q * step for q in range(x.shape[0])]
    ptrs = []
    for q, t in enumerate(x):
        if t is None:
            if not allow_none:
                raise ValueError(f"{name}[{q}] is None")
            ptrs.append(None)
        else:
            ptrs.append(_bf16(t, n, f"{name}[{q}]"))
    return ptrs


def _ptr_table(ptrs):
    return (C.c_void_p * len(ptrs))(*[p if p is not None else None for p in ptrs])


# ------------------------------------------------------------------ plan
class Plan:
    """FlatParameter geometry of a unit: tensor shapes in order and N_d."""

    def __init__(self, shapes: Sequence[Sequence[int]], world: int):
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.world = int(world)
        ndims = (C.c_int32 * len(self.shapes))(*[len(s) for s in self.shapes])
        flat_dims = [d for s in self.shapes for d in s]
        dims = (C.c_int64 * max(1, len(flat_dims)))(*flat_dims)
        h = C.c_void_p()
        check(lib().fp_plan_create(len(self.shapes), ndims, dims, self.world, C.byref(h)))
        self._h = h
        t, p, s = C.c_int64(), C.c_int64(), C.c_int64()
        check(lib().fp_plan_info(self._h, C.byref(t), C.byref(p), C.byref(s)))
        self.numel, self.padded, self.shard = t.value, p.value, s.value

    def close(self):
        if getattr(self, "_h", None):
            lib().fp_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def view_descriptors(self, rank: int = -1):
        """One dict per tensor: buf_offset, numel, tensor_offset, shape (see fp_unpack_views)."""
        n = len(self.shapes)
        out = (_lib.fp_view * n)()
        n_out = C.c_int32()
        check(lib().fp_unpack_views(self._h, int(rank), out, n, C.byref(n_out)))
        return [{"tensor": v.tensor, "buf_offset": v.buf_offset, "numel": v.numel,
                 "tensor_offset": v.tensor_offset, "shape": tuple(v.shape[:v.ndim])} for v in out]

    def pack(self, tensors, flat=None):
        """FlatParameter of `tensors` (one 2- or 4-byte dtype) on the GPU."""
        return self.packer(tensors, flat)()

    def packer(self, tensors, flat=None):
        """A callable that packs `tensors` into `flat` (allocated here when
        None) and returns it, with the tensors checked and their pointers
        marshalled once -- for repeated packs of the same buffers.  The
        caller keeps the tensors alive and in place."""
        _one_device(tensors, flat)
        torch = _torch()
        if len(tensors) != len(self.shapes):
            raise ValueError("tensor count differs from the plan")
        dtype = tensors[0].dtype
        esize = tensors[0].element_size()
        ptrs = []
        for i, (t, s) in enumerate(zip(tensors, self.shapes)):
            if tuple(t.shape) != s or t.dtype != dtype:
                raise ValueError(f"tensor {i}: shape {tuple(t.shape)} / dtype {t.dtype} differ from the plan")
            ptrs.append(_dev_ptr(t, (dtype,), math.prod(s), f"tensors[{i}]") if t.numel() else None)
        if flat is None:
            flat = torch.empty(self.padded, dtype=dtype, device=tensors[0].device)
        fptr = C.c_void_p(_dev_ptr(flat, (dtype,), self.padded, "flat"))
        table = _ptr_table(ptrs)
        fn, h = lib().fp_pack, self._h

        def run():
            check(fn(h, esize, table, fptr, _stream(flat)))
            return flat
        return run

    def views(self, buf, rank: int = -1):
        """Views of the original tensors on `buf` (aliasing, no copy).

        rank = -1: `buf` is the FlatParameter; each view has its tensor's shape.
        rank = q : `buf` is rank q's shard; each view is a 1-D fragment, empty
                   when the rank holds none of the tensor.
        """
        out = []
        for d in self.view_descriptors(rank):
            v = buf.narrow(0, d["buf_offset"], d["numel"])
            out.append(v.view(d["shape"]) if rank < 0 else v)
        return out


class Shard0Plan:
    """Per-parameter dim-0 layout of a parameter group over N_d ranks: each
    parameter cut into ceil(d0 / N_d)-row chunks (zero rows past d0), a
    rank's chunks back to back in one buffer of S elements."""

    def __init__(self, shapes: Sequence[Sequence[int]], world: int):
        self.shapes = [tuple(int(d) for d in s) for s in shapes]
        self.world = int(world)
        ndims = (C.c_int32 * len(self.shapes))(*[len(s) for s in self.shapes])
        flat_dims = [d for s in self.shapes for d in s]
        dims = (C.c_int64 * max(1, len(flat_dims)))(*flat_dims)
        h = C.c_void_p()
        check(lib().fp_shard0_plan_create(len(self.shapes), ndims, dims, self.world, C.byref(h)))
        self._h = h
        s, t = C.c_int64(), C.c_int64()
        check(lib().fp_shard0_plan_info(self._h, C.byref(s), C.byref(t)))
        self.shard, self.numel = s.value, t.value

    def close(self):
        if getattr(self, "_h", None):
            lib().fp_shard0_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def view_descriptors(self, rank: int):
        """One dict per parameter: buf_offset, numel, tensor_offset, local shape."""
        n = len(self.shapes)
        out = (_lib.fp_view * n)()
        n_out = C.c_int32()
        check(lib().fp_shard0_views(self._h, int(rank), out, n, C.byref(n_out)))
        return [{"tensor": v.tensor, "buf_offset": v.buf_offset, "numel": v.numel,
                 "tensor_offset": v.tensor_offset, "shape": tuple(v.shape[:v.ndim])} for v in out]

    def views(self, buf, rank: int):
        """Rank `rank`'s local piece of every parameter on its buffer `buf`
        (aliasing, no copy), each with its local shape."""
        return [buf.narrow(0, d["buf_offset"], d["numel"]).view(d["shape"])
                for d in self.view_descriptors(rank)]

    def _params(self, params):
        if len(params) != len(self.shapes):
            raise ValueError("parameter count differs from the plan")
        dtype = params[0].dtype
        ptrs = []
        for i, (t, s) in enumerate(zip(params, self.shapes)):
            if tuple(t.shape) != s or t.dtype != dtype:
                raise ValueError(f"parameter {i}: shape {tuple(t.shape)} / dtype {t.dtype} differ from the plan")
            ptrs.append(_dev_ptr(t, (dtype,), math.prod(s), f"params[{i}]") if t.numel() else None)
        return dtype, params[0].element_size(), ptrs

    def packer(self, params, dst=None, rank: int = -1):
        """A callable writing rank `rank`'s buffer (rank = -1: every rank's,
        the gathered layout) of `params` into `dst` (allocated here when
        None) and returning it; pointers are marshalled once."""
        _one_device(params, dst)
        torch = _torch()
        dtype, esize, ptrs = self._params(params)
        n = self.shard * (self.world if rank < 0 else 1)
        if dst is None:
            dst = torch.empty(n, dtype=dtype, device=params[0].device)
        dptr = C.c_void_p(_dev_ptr(dst, (dtype,), n, "dst"))
        table = _ptr_table(ptrs)
        fn, h, r = lib().fp_shard0_pack, self._h, int(rank)

        def run():
            check(fn(h, esize, r, table, dptr, _stream(dst)))
            return dst
        return run

    def pack(self, params, dst=None, rank: int = -1):
        return self.packer(params, dst, rank)()

    def unpacker(self, full, params=None):
        """A callable writing every parameter (global shape) from the gathered
        buffer `full` into `params` (allocated here when None) and returning
        them."""
        _one_device(full, params)
        torch = _torch()
        if params is None:
            params = [torch.empty(s, dtype=full.dtype, device=full.device) for s in self.shapes]
        dtype, esize, ptrs = self._params(params)
        fptr = C.c_void_p(_dev_ptr(full, (dtype,), self.shard * self.world, "full"))
        table = _ptr_table(ptrs)
        fn, h = lib().fp_shard0_unpack, self._h

        def run():
            check(fn(h, esize, fptr, table, _stream(full)))
            return params
        return run

    def unpack(self, full, params=None):
        return self.unpacker(full, params)()


class ReshardPlan:
    """A flat buffer of `numel` elements cut into world_old shards, to be cut
    into world_new shards (a sharded checkpoint loaded into another rank
    count): shard sizes ceil(numel / world), zeros past numel."""

    def __init__(self, numel: int, world_old: int, world_new: int):
        self.numel, self.world_old, self.world_new = int(numel), int(world_old), int(world_new)
        h = C.c_void_p()
        check(lib().fp_reshard_plan_create(self.numel, self.world_old, self.world_new, C.byref(h)))
        self._h = h
        so, sn = C.c_int64(), C.c_int64()
        check(lib().fp_reshard_plan_info(self._h, C.byref(so), C.byref(sn)))
        self.shard_old, self.shard_new = so.value, sn.value

    def close(self):
        if getattr(self, "_h", None):
            lib().fp_reshard_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def resharder(self, old_shards, dst=None, rank: int = -1):
        """A callable writing new rank `rank`'s shard (rank = -1: every new
        rank's, one after the other) from the old shards into dst (allocated
        here when None) and returning it; pointers are marshalled once."""
        _one_device(old_shards, dst)
        torch = _torch()
        if len(old_shards) != self.world_old:
            raise ValueError(f"need {self.world_old} old shards")
        given = [t for t in old_shards if t is not None] + ([dst] if dst is not None else [])
        if not given:
            raise ValueError("need at least one old shard or dst to know the dtype and device")
        dtype = given[0].dtype
        esize = torch.empty(0, dtype=dtype).element_size()
        ptrs = []
        for q, t in enumerate(old_shards):
            if t is None:
                ptrs.append(None)
                continue
            if t.dtype != dtype:
                raise TypeError("old shards differ in dtype")
            ptrs.append(_dev_ptr(t, (dtype,), self.shard_old, f"old_shards[{q}]"))
        n = self.shard_new * (self.world_new if rank < 0 else 1)
        if dst is None:
            dst = torch.empty(n, dtype=dtype, device=given[0].device)
        dptr = C.c_void_p(_dev_ptr(dst, (dtype,), n, "dst"))
        table = _ptr_table(ptrs)
        fn, h, r = lib().fp_reshard, self._h, int(rank)

        def run():
            check(fn(h, esize, r, table, dptr, _stream(dst)))
            return dst
        return run

    def reshard(self, old_shards, dst=None, rank: int = -1):
        return self.resharder(old_shards, dst, rank)()


# ------------------------------------------------------------------ reduce
def workspace_bytes(shard: int) -> int:
    return int(lib().fp_workspace_bytes(int(shard)))


def new_workspace(device, shard: int):
    """Zero-filled device workspace for shards of up to `shard` elements."""
    torch = _torch()
    return torch.zeros(workspace_bytes(shard), dtype=torch.uint8, device=device)


def workspace_timeouts(workspace) -> int:
    """Grid-barrier waits of the one-pass step that gave up (0 in correct operation)."""
    off = _lib.FP_WORKSPACE_TIMEOUTS_OFFSET
    return int(workspace[off:off + 4].view(_torch().int32).item())


def reduce_shard(grads, acc, *, scale: float, accumulate: bool = False, found_inf=None,
                 sq_norm=None, workspace=None):
    """acc (= or +=) scale * sum of the ranks' bf16 gradients, fixed rank order."""
    _one_device(grads, acc, found_inf, sq_norm, workspace)
    torch = _torch()
    S = acc.numel()
    ptrs = _rank_ptrs(grads, S, "grads")
    fi = _dev_ptr(found_inf, (torch.int32,), 1, "found_inf") if found_inf is not None else None
    sq = _dev_ptr(sq_norm, (torch.float64,), 1, "sq_norm") if sq_norm is not None else None
    ws = _dev_ptr(workspace, (torch.uint8,), workspace_bytes(S), "workspace") if workspace is not None else None
    check(lib().fp_reduce_shard(S, len(ptrs), _ptr_table(ptrs), float(scale), int(bool(accumulate)),
                                C.c_void_p(_f32(acc, S, "acc")), fi, sq, ws, _stream(acc)))
    return acc


def reduce_shard_hybrid(grads, acc, *, group: int, scale: float, accumulate: bool = False, found_inf=None,
                        sq_norm=None, workspace=None):
    """acc (= or +=) scale * two-level sum of the W ranks' bf16 gradients: inside
    each group of `group` consecutive ranks, then across the groups."""
    _one_device(grads, acc, found_inf, sq_norm, workspace)
    torch = _torch()
    S = acc.numel()
    ptrs = _rank_ptrs(grads, S, "grads")
    fi = _dev_ptr(found_inf, (torch.int32,), 1, "found_inf") if found_inf is not None else None
    sq = _dev_ptr(sq_norm, (torch.float64,), 1, "sq_norm") if sq_norm is not None else None
    ws = _dev_ptr(workspace, (torch.uint8,), workspace_bytes(S), "workspace") if workspace is not None else None
    check(lib().fp_reduce_shard_hybrid(S, len(ptrs), int(group), _ptr_table(ptrs), float(scale),
                                       int(bool(accumulate)), C.c_void_p(_f32(acc, S, "acc")), fi, sq, ws,
                                       _stream(acc)))
    return acc


# ------------------------------------------------------------------ adamw
def _hparams(lr, beta1, beta2, eps, weight_decay, step):
    return _lib.fp_adamw_hparams(float(lr), float(beta1), float(beta2), float(eps),
                                 float(weight_decay), int(step))


def _coef_ptr(grad_coef):
    return _dev_ptr(grad_coef, (_torch().float64,), 1, "grad_coef") if grad_coef is not None else None


def adamw_shard(grad, master, exp_avg, exp_avg_sq, *, lr, beta1, beta2, eps, weight_decay,
                step: int, found_inf=None, param_bf16=None, grad_coef=None):
    """In-place AdamW on fp32 master / exp_avg / exp_avg_sq; bf16 copy to param_bf16.
    grad_coef: optional device float64 factor applied to the gradient (see grad_coef())."""
    _one_device(grad, master, exp_avg, exp_avg_sq, found_inf, param_bf16, grad_coef)
    torch = _torch()
    S = master.numel()
    hp = _hparams(lr, beta1, beta2, eps, weight_decay, step)
    fi = _dev_ptr(found_inf, (torch.int32,), 1, "found_inf") if found_inf is not None else None
    out = _bf16(param_bf16, S, "param_bf16") if param_bf16 is not None else None
    check(lib().fp_adamw_shard(S, C.byref(hp), _f32(grad, S, "grad"), _f32(master, S, "master"),
                               _f32(exp_avg, S, "exp_avg"), _f32(exp_avg_sq, S, "exp_avg_sq"),
                               fi, out, _coef_ptr(grad_coef), _stream(master)))


# ------------------------------------------------------------------ no_sync and the loss scaler
def local_accumulate(grad, local, *, accumulate: bool):
    """local (fp32) = (local if accumulate else 0) + grad (bf16): one micro-batch
    accumulated without communication."""
    _one_device(grad, local)
    n = local.numel()
    check(lib().fp_local_accumulate(n, _bf16(grad, n, "grad"), int(bool(accumulate)),
                                    _f32(local, n, "local"), _stream(local)))
    return local


def local_finish(grad, out, local=None, *, accumulate: bool):
    """out (bf16) = bf16(local + grad), or bf16(grad) when not accumulating: the
    row this rank contributes to the reduce-scatter."""
    _one_device(grad, out, local)
    n = out.numel()
    lp = _f32(local, n, "local") if local is not None else None
    check(lib().fp_local_finish(n, _bf16(grad, n, "grad"), int(bool(accumulate)), lp, _bf16(out, n, "out"),
                                _stream(out)))
    return out


def grad_coef(coef, *, sq_norm=None, loss_scale=None, max_norm: float = 0.0):
    """coef (device float64[1]) = 1 / loss_scale, times the global-norm clip
    factor min(1, max_norm / (||g|| + 1e-6)) when max_norm > 0."""
    _one_device(coef, sq_norm, loss_scale)
    torch = _torch()
    sq = _dev_ptr(sq_norm, (torch.float64,), 1, "sq_norm") if sq_norm is not None else None
    ls = _dev_ptr(loss_scale, (torch.float32,), 1, "loss_scale") if loss_scale is not None else None
    check(lib().fp_grad_coef(sq, ls, float(max_norm), _dev_ptr(coef, (torch.float64,), 1, "coef"),
                             _stream(coef)))
    return coef


def scaler_update(found_inf, scale, clean_steps, *, growth_factor: float = 2.0, backoff_factor: float = 0.5,
                  growth_interval: int = 2000):
    """Dynamic loss scaling on device values after a step's overflow decision."""
    _one_device(found_inf, scale, clean_steps)
    torch = _torch()
    check(lib().fp_scaler_update(_dev_ptr(found_inf, (torch.int32,), 1, "found_inf"),
                                 _dev_ptr(scale, (torch.float32,), 1, "scale"),
                                 _dev_ptr(clean_steps, (torch.int32,), 1, "clean_steps"),
                                 float(growth_factor), float(backoff_factor), int(growth_interval),
                                 _stream(scale)))


# ------------------------------------------------------------------ unshard
def unshard(shards, full):
    """full[q*S:(q+1)*S] = shards[q]; a None entry leaves that range untouched."""
    _one_device(shards, full)
    world = len(shards) if not hasattr(shards, "dim") else shards.shape[0]
    S = full.numel() // world
    if S * world != full.numel():
        raise ValueError("full is not world * S elements")
    ptrs = _rank_ptrs(shards, S, "shards", allow_none=True)
    check(lib().fp_unshard(S, world, _ptr_table(ptrs), C.c_void_p(_bf16(full, S * world, "full")),
                           _stream(full)))
    return full


# ------------------------------------------------------------------ step
def shard_step(grads, acc, master, exp_avg, exp_avg_sq, shards, full, rank: int, *, scale: float,
               lr, beta1, beta2, eps, weight_decay, step: int, found_inf, accumulate: bool = False,
               sq_norm=None, workspace=None, flags: int = FP_STEP_EXACT_SKIP, profile_events=None,
               grad_coef=None, out=None):
    """Reduce (last micro-batch) + AdamW + bf16 cast + unshard for this rank."""
    ShardStep(grads, acc, master, exp_avg, exp_avg_sq, shards, full, rank, scale=scale, lr=lr,
              beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay, found_inf=found_inf,
              accumulate=accumulate, sq_norm=sq_norm, workspace=workspace,
              flags=flags, grad_coef=grad_coef, out=out)(step, profile_events)


class ShardStep:
    """shard_step with its arguments marshalled once, for tight step loops.

    The tensors are checked and their pointers captured at construction;
    each call only sets the step count (and the optional profile events)
    and makes one library call on the current stream of master's device.
    The caller keeps the tensors alive and unchanged in size.

    out: None (the state is updated in place) or (master_out, exp_avg_out,
    exp_avg_sq_out), three fp32 buffers of the shard's size that receive
    the new state while master / exp_avg / exp_avg_sq are only read (the
    speculative step; the caller alternates two ShardStep objects whose
    input and output buffers are swapped).

    library_scratch: call fp_shard_step_noalloc, whose scratch is an array
    inside the library (workspace must then be None); for callers that
    cannot allocate device memory.
    """

    def __init__(self, grads, acc, master, exp_avg, exp_avg_sq, shards, full, rank: int, *,
                 scale: float, lr, beta1, beta2, eps, weight_decay, found_inf,
                 accumulate: bool = False, sq_norm=None, workspace=None,
                 flags: int = FP_STEP_EXACT_SKIP, grad_coef=None, out=None, library_scratch: bool = False):
        _one_device(grads, acc, master, exp_avg, exp_avg_sq, shards, full, found_inf, sq_norm, workspace,
                    grad_coef, out)
        if library_scratch and workspace is not None:
            raise ValueError("library_scratch uses the library's own scratch: pass no workspace")
        if out is not None and len(out) != 3:
            raise ValueError("out is (master_out, exp_avg_out, exp_avg_sq_out)")
        torch = _torch()
        S = master.numel()
        gptr = _rank_ptrs(grads, S, "grads")
        sptr = _rank_ptrs(shards, S, "shards", allow_none=True)
        if len(sptr) != len(gptr):
            raise ValueError("shards and grads differ in length")
        self._tables = (_ptr_table(gptr), _ptr_table(sptr))
        self._events = (C.c_void_p * _lib.FP_STEP_EVENTS)()
        a = _lib.fp_step_args()
        a.shard, a.world, a.rank = S, len(gptr), int(rank)
        a.grads = C.cast(self._tables[0], C.c_void_p)
        a.shards = C.cast(self._tables[1], C.c_void_p)
        a.scale, a.accumulate = float(scale), int(bool(accumulate))
        a.acc, a.master = _f32(acc, S, "acc"), _f32(master, S, "master")
        a.exp_avg, a.exp_avg_sq = _f32(exp_avg, S, "exp_avg"), _f32(exp_avg_sq, S, "exp_avg_sq")
        a.hp = _hparams(lr, beta1, beta2, eps, weight_decay, 1)
        a.full = _bf16(full, S * len(gptr), "full")
        a.found_inf = _dev_ptr(found_inf, (torch.int32,), 1, "found_inf")
        a.sq_norm = _dev_ptr(sq_norm, (torch.float64,), 1, "sq_norm") if sq_norm is not None else None
        a.workspace = (_dev_ptr(workspace, (torch.uint8,), workspace_bytes(S), "workspace")
                       if workspace is not None else None)
        a.flags = int(flags)
        a.grad_coef = _coef_ptr(grad_coef)
        if out is not None:
            a.master_out = _f32(out[0], S, "master_out")
            a.exp_avg_out = _f32(out[1], S, "exp_avg_out")
            a.exp_avg_sq_out = _f32(out[2], S, "exp_avg_sq_out")
        self._args = a
        self._device = master.device
        self._fn = lib().fp_shard_step_noalloc if library_scratch else lib().fp_shard_step

    def __call__(self, step: int, profile_events=None):
        a = self._args
        a.hp.step = int(step)
        if profile_events is None:
            a.profile_events = None
        else:
            if len(profile_events) != _lib.FP_STEP_EVENTS:
                raise ValueError(f"profile_events needs {_lib.FP_STEP_EVENTS} hipEvent_t handles")
            for i, e in enumerate(profile_events):
                self._events[i] = e
            a.profile_events = C.cast(self._events, C.c_void_p)
        check(self._fn(C.byref(a), _stream(self._device)))

    def test_give_up(self, step: int):
        """fp_step_test_give_up with these arguments: the one-pass kernel with a
        barrier that always gives up (for tests of that path; the workspace must
        be zero-filled again afterwards)."""
        a = self._args
        a.hp.step = int(step)
        a.profile_events = None
        check(lib().fp_step_test_give_up(C.byref(a), _stream(self._device)))

    def path(self) -> int:
        """One of the FP_PATH_* values: the kernels a call launches on this device."""
        torch = _torch()
        out = C.c_int32(-1)
        with torch.cuda.device(self._device):
            check(lib().fp_step_path(C.byref(self._args), C.byref(out)))
        return out.value


# ------------------------------------------------------------------ units
class Units:
    """Many units (DDP buckets, FSDP units) of one rank stepped together:
    one launch per stage for all of them (fp_units_*).

    grads: per unit, the world ranks' bf16 gradients over this rank's shard
    of that unit (a list of 1-D tensors or a [world, S_u] tensor).
    shards / full: per unit, the ranks' bf16 shards (entry `rank` None) and
    the gathered bf16 [world * S_u] buffer; both None for a reduce-only plan.
    The rank's fp32 state is one partition of `partition` elements holding
    unit u at `offsets[u]`.  The tensors must stay alive and in place for
    the plan's life; the plan is bound to the device current at creation.
    """

    def __init__(self, grads, rank: int, shards=None, full=None):
        _one_device(grads, shards, full)
        torch = _torch()
        n = len(grads)
        if n < 1:
            raise ValueError("need at least one unit")
        if (shards is None) != (full is None):
            raise ValueError("shards and full go together")
        sizes, gtab, stab, ftab = [], [], [], []
        world = None
        for u in range(n):
            g = grads[u]
            S = g.shape[1] if hasattr(g, "dim") and g.dim() == 2 else g[0].numel()
            p = _rank_ptrs(g, S, f"grads[{u}]")
            world = len(p) if world is None else world
            if len(p) != world:
                raise ValueError(f"grads[{u}] has {len(p)} ranks, expected {world}")
            sizes.append(S)
            gtab += p
            if shards is not None:
                sp = _rank_ptrs(shards[u], S, f"shards[{u}]", allow_none=True)
                if len(sp) != world:
                    raise ValueError(f"shards[{u}] has {len(sp)} ranks, expected {world}")
                stab += sp
                ftab.append(_bf16(full[u], S * world, f"full[{u}]"))
        self.world, self.rank, self.n_units, self.sizes = world, int(rank), n, sizes
        self._keep = (grads, shards, full)
        self._device = (grads[0] if hasattr(grads[0], "device") else grads[0][0]).device
        out = C.c_void_p()
        with torch.cuda.device(self._device):
            check(lib().fp_units_create(
                n, world, int(rank), (C.c_int64 * n)(*sizes), _ptr_table(gtab),
                _ptr_table(stab) if shards is not None else None,
                _ptr_table(ftab) if shards is not None else None, C.byref(out)))
        self._h = out
        part, ws = C.c_int64(), C.c_int64()
        check(lib().fp_units_info(self._h, C.byref(part), C.byref(ws)))
        self.partition, self.workspace_bytes = part.value, ws.value
        offs = (C.c_int64 * n)()
        check(lib().fp_units_offsets(self._h, offs))
        self.offsets = list(offs)

    def close(self):
        if getattr(self, "_h", None):
            lib().fp_units_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_workspace(self):
        torch = _torch()
        return torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=self._device)

    def unit_slice(self, buf, u: int):
        """Unit u's shard inside a partition-sized tensor."""
        return buf.narrow(0, self.offsets[u], self.sizes[u])

    def _opt(self, t, dtype, n, name):
        return _dev_ptr(t, (dtype,), n, name) if t is not None else None

    def reduce(self, acc, *, scale: float, accumulate: bool = False, found_inf=None, sq_norm=None,
               workspace=None):
        _one_device(acc, found_inf, sq_norm, workspace)
        torch = _torch()
        check(lib().fp_units_reduce(
            self._h, float(scale), int(bool(accumulate)), C.c_void_p(_f32(acc, self.partition, "acc")),
            self._opt(found_inf, torch.int32, 1, "found_inf"), self._opt(sq_norm, torch.float64, 1, "sq_norm"),
            self._opt(workspace, torch.uint8, self.workspace_bytes, "workspace"), _stream(acc)))
        return acc

    def _step_args(self, acc, master, exp_avg, exp_avg_sq, *, scale, lr, beta1, beta2, eps, weight_decay,
                   step, found_inf, accumulate, sq_norm, workspace, flags, profile_events, grad_coef, out):
        _one_device(acc, master, exp_avg, exp_avg_sq, found_inf, sq_norm, workspace, grad_coef, out)
        if out is not None and len(out) != 3:
            raise ValueError("out is (master_out, exp_avg_out, exp_avg_sq_out)")
        torch = _torch()
        P = self.partition
        a = _lib.fp_units_step_args()
        a.scale, a.accumulate = float(scale), int(bool(accumulate))
        a.acc, a.master = _f32(acc, P, "acc"), _f32(master, P, "master")
        a.exp_avg, a.exp_avg_sq = _f32(exp_avg, P, "exp_avg"), _f32(exp_avg_sq, P, "exp_avg_sq")
        a.hp = _hparams(lr, beta1, beta2, eps, weight_decay, step)
        a.found_inf = _dev_ptr(found_inf, (torch.int32,), 1, "found_inf")
        a.sq_norm = self._opt(sq_norm, torch.float64, 1, "sq_norm")
        a.workspace = self._opt(workspace, torch.uint8, self.workspace_bytes, "workspace")
        a.flags = int(flags)
        a.grad_coef = _coef_ptr(grad_coef)
        if out is not None:
            a.master_out = _f32(out[0], P, "master_out")
            a.exp_avg_out = _f32(out[1], P, "exp_avg_out")
            a.exp_avg_sq_out = _f32(out[2], P, "exp_avg_sq_out")
        ev = None
        if profile_events is not None:
            if len(profile_events) != _lib.FP_STEP_EVENTS:
                raise ValueError(f"profile_events needs {_lib.FP_STEP_EVENTS} hipEvent_t handles")
            ev = (C.c_void_p * _lib.FP_STEP_EVENTS)(*profile_events)
            a.profile_events = C.cast(ev, C.c_void_p)
        return a, ev

    def step(self, acc, master, exp_avg, exp_avg_sq, *, scale: float, lr, beta1, beta2, eps,
             weight_decay, step: int, found_inf, accumulate: bool = False, sq_norm=None,
             workspace=None, flags: int = FP_STEP_EXACT_SKIP, profile_events=None, grad_coef=None,
             out=None):
        """The last micro-batch's step over all units.  out: None (in place) or
        (master_out, exp_avg_out, exp_avg_sq_out) partitions that receive the new
        state while master / exp_avg / exp_avg_sq are only read (the speculative
        step; the caller swaps the partitions after each step)."""
        a, _ev = self._step_args(acc, master, exp_avg, exp_avg_sq, scale=scale, lr=lr, beta1=beta1, beta2=beta2,
                                 eps=eps, weight_decay=weight_decay, step=step, found_inf=found_inf,
                                 accumulate=accumulate, sq_norm=sq_norm, workspace=workspace, flags=flags,
                                 profile_events=profile_events, grad_coef=grad_coef, out=out)
        check(lib().fp_units_step(self._h, C.byref(a), _stream(master)))

    def step_path(self, acc, master, exp_avg, exp_avg_sq, *, found_inf, flags: int = FP_STEP_EXACT_SKIP,
                  out=None, sq_norm=None, workspace=None):
        """One of the FP_PATH_* values: the launches step() makes with these buffers."""
        a, _ev = self._step_args(acc, master, exp_avg, exp_avg_sq, scale=1.0, lr=1e-3, beta1=0.9, beta2=0.999,
                                 eps=1e-8, weight_decay=0.0, step=1, found_inf=found_inf, accumulate=False,
                                 sq_norm=sq_norm, workspace=workspace, flags=flags, profile_events=None,
                                 grad_coef=None, out=out)
        path = C.c_int32(-1)
        check(lib().fp_units_step_path(self._h, C.byref(a), C.byref(path)))
        return path.value


# ------------------------------------------------------------------ helpers
def state_bytes(psi: float, world: int, k: float = 12.0, stage: int = 3) -> float:
    """Model-state bytes per GPU for ZeRO stage 0..3 (fp_state_bytes)."""
    out = C.c_double()
    check(lib().fp_state_bytes(float(psi), int(world), float(k), int(stage), C.byref(out)))
    return out.value
