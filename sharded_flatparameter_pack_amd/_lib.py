"""ctypes declarations of libflatparam.so (include/flatparam.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflatparam.so")

FP_OK = 0
FP_ERR_INVALID = -1
FP_ERR_RANGE = -2
FP_ERR_ALIGN = -3
FP_ERR_DEVICE = -4
FP_MAX_WORLD = 128
FP_MAX_NDIM = 8
FP_STEP_EXACT_SKIP = 0
FP_STEP_NO_SKIP = 1
FP_STEP_KEEP_GRAD = 2
FP_STEP_NO_COOP = 4
FP_STEP_EVENTS = 3
FP_PATH_ONE_PASS = 0
FP_PATH_TWO_PHASE = 1
FP_PATH_NO_SKIP = 2
FP_PATH_NO_SKIP_SPLIT = 3
FP_PATH_SPECULATIVE = 4
FP_PATH_SPECULATIVE_SPLIT = 5
FP_PATH_SPECULATIVE_ONE_PASS = 6
FP_WORKSPACE_TIMEOUTS_OFFSET = 8320
FP_FLAG_OVERFLOW = 1
FP_FLAG_GAVE_UP = 2

_i32, _i64, _f32, _f64, _vp = C.c_int32, C.c_int64, C.c_float, C.c_double, C.c_void_p


class fp_view(C.Structure):
    _fields_ = [("tensor", _i32), ("ndim", _i32), ("buf_offset", _i64), ("numel", _i64),
                ("tensor_offset", _i64), ("shape", _i64 * FP_MAX_NDIM)]


class fp_adamw_hparams(C.Structure):
    _fields_ = [("lr", _f64), ("beta1", _f64), ("beta2", _f64), ("eps", _f64),
                ("weight_decay", _f64), ("step", _i64)]


class fp_step_args(C.Structure):
    _fields_ = [("shard", _i64), ("world", _i32), ("rank", _i32), ("grads", _vp),
                ("scale", _f32), ("accumulate", _i32), ("acc", _vp), ("master", _vp),
                ("exp_avg", _vp), ("exp_avg_sq", _vp), ("hp", fp_adamw_hparams),
                ("shards", _vp), ("full", _vp), ("found_inf", _vp), ("sq_norm", _vp),
                ("workspace", _vp), ("flags", _i32), ("profile_events", _vp), ("grad_coef", _vp),
                ("master_out", _vp), ("exp_avg_out", _vp), ("exp_avg_sq_out", _vp)]


class fp_units_step_args(C.Structure):
    _fields_ = [("scale", _f32), ("accumulate", _i32), ("acc", _vp), ("master", _vp),
                ("exp_avg", _vp), ("exp_avg_sq", _vp), ("hp", fp_adamw_hparams),
                ("found_inf", _vp), ("sq_norm", _vp), ("workspace", _vp), ("flags", _i32),
                ("profile_events", _vp), ("grad_coef", _vp), ("master_out", _vp), ("exp_avg_out", _vp),
                ("exp_avg_sq_out", _vp)]


# name -> (restype, argtypes); the export test compares this table with the header
SIGNATURES = {
    "fp_plan_create": (_i32, [_i32, _vp, _vp, _i32, C.POINTER(_vp)]),
    "fp_plan_destroy": (None, [_vp]),
    "fp_plan_info": (_i32, [_vp, _vp, _vp, _vp]),
    "fp_pack": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "fp_unpack_views": (_i32, [_vp, _i32, _vp, _i32, _vp]),
    "fp_workspace_bytes": (_i64, [_i64]),
    "fp_reduce_shard": (_i32, [_i64, _i32, _vp, _f32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "fp_reduce_shard_hybrid": (_i32, [_i64, _i32, _i32, _vp, _f32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "fp_adamw_shard": (_i32, [_i64, C.POINTER(fp_adamw_hparams), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp_unshard": (_i32, [_i64, _i32, _vp, _vp, _vp]),
    "fp_shard_step": (_i32, [C.POINTER(fp_step_args), _vp]),
    "fp_step_path": (_i32, [C.POINTER(fp_step_args), C.POINTER(C.c_int32)]),
    "fp_step_test_give_up": (_i32, [C.POINTER(fp_step_args), _vp]),
    "fp_shard_step_noalloc": (_i32, [C.POINTER(fp_step_args), _vp]),
    "fp_units_create": (_i32, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, C.POINTER(_vp)]),
    "fp_units_destroy": (None, [_vp]),
    "fp_units_info": (_i32, [_vp, _vp, _vp]),
    "fp_units_offsets": (_i32, [_vp, _vp]),
    "fp_units_reduce": (_i32, [_vp, _f32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "fp_units_step": (_i32, [_vp, C.POINTER(fp_units_step_args), _vp]),
    "fp_units_step_path": (_i32, [_vp, C.POINTER(fp_units_step_args), C.POINTER(C.c_int32)]),
    "fp_shard0_plan_create": (_i32, [_i32, _vp, _vp, _i32, C.POINTER(_vp)]),
    "fp_shard0_plan_destroy": (None, [_vp]),
    "fp_shard0_plan_info": (_i32, [_vp, _vp, _vp]),
    "fp_shard0_views": (_i32, [_vp, _i32, _vp, _i32, _vp]),
    "fp_shard0_pack": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "fp_shard0_unpack": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "fp_reshard_plan_create": (_i32, [_i64, _i32, _i32, C.POINTER(_vp)]),
    "fp_reshard_plan_destroy": (None, [_vp]),
    "fp_reshard_plan_info": (_i32, [_vp, _vp, _vp]),
    "fp_reshard": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp]),
    "fp_local_accumulate": (_i32, [_i64, _vp, _i32, _vp, _vp]),
    "fp_local_finish": (_i32, [_i64, _vp, _i32, _vp, _vp, _vp]),
    "fp_grad_coef": (_i32, [_vp, _vp, _f64, _vp, _vp]),
    "fp_scaler_update": (_i32, [_vp, _vp, _vp, _f32, _f32, _i32, _vp]),
    "fp_state_bytes": (_i32, [_f64, _i32, _f64, _i32, C.POINTER(_f64)]),
    "fp_status_string": (C.c_char_p, [_i32]),
    "fp_last_error": (C.c_char_p, []),
}

_lib = None


class FlatParamError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -c \"import __graft_entry__; "
                f"__graft_entry__.build()\"` (hipcc, gfx950). There is no fallback.")
        try:  # share torch's HIP runtime (same SONAME) when torch is present
            import torch  # noqa: F401
        except ImportError:
            pass
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != FP_OK:
        msg = lib().fp_last_error().decode(errors="replace")
        raise FlatParamError(status, msg)
