"""Host-side checks of the C ABI (no GPU needed).

* libflatparam.so loads and exports every function include/flatparam.h
  declares, and the binding's ctypes table declares the same set;
* the host-only entry points (plan geometry, views, memory model) agree
  with the CPU oracle;
* argument validation rejects bad calls before anything is enqueued --
  every call below fails validation, so no kernel is ever launched.
"""

import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT
from workloads import CONFIGS

HEADER = os.path.join(ROOT, "include", "flatparam.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("fp_pack", "fp_reduce_shard", "fp_adamw_shard", "fp_unshard", "fp_unpack_views",
                     "fp_shard_step", "fp_plan_create", "fp_state_bytes"):
        assert required in names


def test_library_exports_every_declared_function(fp):
    L = C.CDLL(fp.library_path())
    missing = [n for n in header_functions() if not hasattr(L, n)]
    assert missing == []
    from sharded_flatparameter_pack_amd import _lib
    assert sorted(_lib.SIGNATURES) == header_functions()


def test_struct_layouts_match_the_header(fp):
    from sharded_flatparameter_pack_amd import _lib
    assert C.sizeof(_lib.fp_view) == 4 + 4 + 8 * 3 + 8 * 8
    assert C.sizeof(_lib.fp_adamw_hparams) == 6 * 8
    # fp_step_args: offsets follow the C layout rules of the header's field order
    assert _lib.fp_step_args.grads.offset == 16
    assert _lib.fp_step_args.hp.offset == 64
    assert _lib.fp_step_args.flags.offset == 152
    assert _lib.fp_step_args.grad_coef.offset == 64 + 48 + 5 * 8 + 8 + 8
    assert _lib.fp_step_args.master_out.offset == 64 + 48 + 5 * 8 + 8 + 8 + 8
    assert _lib.fp_step_args.exp_avg_sq_out.offset == 64 + 48 + 5 * 8 + 8 + 8 + 8 + 16
    assert C.sizeof(_lib.fp_step_args) == 64 + 48 + 5 * 8 + 8 + 8 + 8 + 24
    assert _lib.fp_units_step_args.hp.offset == 40
    assert _lib.fp_units_step_args.grad_coef.offset == 128
    assert _lib.fp_units_step_args.exp_avg_sq_out.offset == 152
    assert C.sizeof(_lib.fp_units_step_args) == 160


def test_struct_layouts_match_a_c_compiler(fp, tmp_path):
    """Every field offset and struct size of the ctypes declarations equals what
    a C compiler makes of include/flatparam.h."""
    import shutil
    import subprocess
    from sharded_flatparameter_pack_amd import _lib
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = [_lib.fp_view, _lib.fp_adamw_hparams, _lib.fp_step_args, _lib.fp_units_step_args]
    lines = ['#include <stddef.h>', '#include <stdio.h>', f'#include "{HEADER}"', "int main(void) {"]
    want = []
    for st in structs:
        name = st.__name__
        lines.append(f'  printf("%zu\\n", sizeof({name}));')
        want.append(C.sizeof(st))
        for field, *_ in st._fields_:
            lines.append(f'  printf("%zu\\n", offsetof({name}, {field}));')
            want.append(getattr(st, field).offset)
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-o", str(exe), str(src)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got == want


def _random_shapes(r):
    n = int(r.integers(1, 12))
    return [tuple(int(d) for d in r.integers(0 if r.random() < 0.1 else 1, 7, size=int(r.integers(0, 4))))
            for _ in range(n)]


@pytest.mark.parametrize("seed", range(30))
def test_plan_geometry_and_views_match_oracle(fp, seed):
    r = np.random.default_rng(seed)
    shapes = _random_shapes(r)
    world = int(r.choice([1, 2, 3, 4, 7, 8, 64, 1000]))
    numel = [math.prod(s) for s in shapes]
    plan = fp.Plan(shapes, world)
    assert (plan.numel, plan.padded, plan.shard) == oracle.geometry(numel, world)
    for rank in [-1] + sorted(set(int(x) for x in r.integers(0, world, size=4))):
        got = plan.view_descriptors(rank)
        bo, ln, to = oracle.views(numel, world, rank)
        for i, d in enumerate(got):
            assert d["tensor"] == i
            assert d["numel"] == ln[i]
            if ln[i] > 0:
                assert (d["buf_offset"], d["tensor_offset"]) == (bo[i], to[i])
            if rank < 0:
                assert d["shape"] == shapes[i]
            else:
                assert d["shape"] == (int(ln[i]),)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_plan_of_each_workload(fp, name):
    cfg = CONFIGS[name]
    for T in cfg.units()[:2]:
        shapes = cfg.shapes if cfg.shapes is not None else [(T,)]
        plan = fp.Plan(shapes, cfg.world)
        numel = [math.prod(s) for s in shapes]
        assert (plan.numel, plan.padded, plan.shard) == oracle.geometry(numel, cfg.world)
        for rank in cfg.ranks:
            bo, ln, to = oracle.views(numel, cfg.world, rank)
            got = plan.view_descriptors(rank)
            assert [d["numel"] for d in got] == list(ln)
            assert [d["buf_offset"] for d in got if d["numel"]] == [b for b, n in zip(bo, ln) if n]


def test_state_bytes_match_oracle(fp):
    for psi in (7e9, 1.3e8, 611e6):
        for world in (1, 2, 8, 512):
            for stage in range(4):
                assert fp.state_bytes(psi, world, 12, stage) == pytest.approx(
                    oracle.state_bytes(psi, world, 12, stage), rel=1e-15)
    with pytest.raises(fp.FlatParamError):
        fp.state_bytes(1e9, 8, 12, 4)
    with pytest.raises(fp.FlatParamError):
        fp.state_bytes(1e9, 0, 12, 1)


def _status(fn, *args):
    return int(fn(*args))


def test_plan_validation(fp):
    L = fp.lib()
    h = C.c_void_p()
    nd = (C.c_int32 * 1)(2)
    dims = (C.c_int64 * 2)(4, 2)
    assert _status(L.fp_plan_create, 0, nd, dims, 2, C.byref(h)) == -2
    assert _status(L.fp_plan_create, 1, nd, dims, 0, C.byref(h)) == -2
    assert _status(L.fp_plan_create, 1, None, dims, 2, C.byref(h)) == -1
    bad = (C.c_int64 * 2)(4, -2)
    assert _status(L.fp_plan_create, 1, nd, bad, 2, C.byref(h)) == -2
    nd9 = (C.c_int32 * 1)(9)
    assert _status(L.fp_plan_create, 1, nd9, dims, 2, C.byref(h)) == -2
    huge = (C.c_int64 * 2)(1 << 40, 1 << 30)
    assert _status(L.fp_plan_create, 1, nd, huge, 2, C.byref(h)) == -2
    assert b"too many" in L.fp_last_error() or b"2^62" in L.fp_last_error()
    plan = fp.Plan([(4, 2)] * 3, 2)
    out = (fp._lib.fp_view * 2)()
    n = C.c_int32()
    assert _status(L.fp_unpack_views, plan._h, 0, out, 2, C.byref(n)) == -2 and n.value == 3
    assert _status(L.fp_unpack_views, plan._h, 2, out, 3, C.byref(n)) == -2
    assert _status(L.fp_pack, plan._h, 3, (C.c_void_p * 3)(), C.c_void_p(256), None) == -1
    assert _status(L.fp_pack, plan._h, 4, (C.c_void_p * 3)(256, 512, 768), C.c_void_p(1028), None) == -3
    assert _status(L.fp_pack, plan._h, 4, (C.c_void_p * 3)(256, 0, 768), C.c_void_p(4096), None) == -1


def test_device_entry_points_reject_bad_arguments(fp):
    """Every call here fails validation; fake addresses are never dereferenced."""
    from sharded_flatparameter_pack_amd import _lib
    L = fp.lib()
    g = (C.c_void_p * 2)(0x10000, 0x20000)
    # world out of range
    assert _status(L.fp_reduce_shard, 16, 0, g, 1.0, 0, C.c_void_p(0x30000), None, None, None, None) == -2
    assert _status(L.fp_reduce_shard, 16, 129, g, 1.0, 0, C.c_void_p(0x30000), None, None, None, None) == -2
    # misaligned fp32 accumulator / bf16 gradient
    assert _status(L.fp_reduce_shard, 16, 2, g, 1.0, 0, C.c_void_p(0x30004), None, None, None, None) == -3
    g_odd = (C.c_void_p * 2)(0x10001, 0x20000)
    assert _status(L.fp_reduce_shard, 16, 2, g_odd, 1.0, 0, C.c_void_p(0x30000), None, None, None, None) == -3
    # missing gradient pointer, negative size, norm without workspace
    g_null = (C.c_void_p * 2)(0x10000, None)
    assert _status(L.fp_reduce_shard, 16, 2, g_null, 1.0, 0, C.c_void_p(0x30000), None, None, None, None) == -1
    assert _status(L.fp_reduce_shard, -1, 2, g, 1.0, 0, C.c_void_p(0x30000), None, None, None, None) == -2
    assert _status(L.fp_reduce_shard, 16, 2, g, 1.0, 0, C.c_void_p(0x30000), None,
                   C.c_void_p(0x40000), None, None) == -1
    # gradient overlapping the accumulator
    g_ov = (C.c_void_p * 2)(0x30010, 0x20000)
    assert _status(L.fp_reduce_shard, 16, 2, g_ov, 1.0, 0, C.c_void_p(0x30000), None, None, None, None) == -1

    hp = _lib.fp_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 0)
    ptr = [C.c_void_p(0x100000 * (i + 1)) for i in range(4)]
    assert _status(L.fp_adamw_shard, 64, C.byref(hp), *ptr, None, None, None, None) == -2  # step 0
    hp.step, hp.beta2 = 1, 1.0
    assert _status(L.fp_adamw_shard, 64, C.byref(hp), *ptr, None, None, None, None) == -2  # beta2 = 1
    hp.beta2 = 0.999
    assert _status(L.fp_adamw_shard, 64, C.byref(hp), ptr[0], ptr[1], ptr[1], ptr[3], None, None, None,
                   None) == -1
    assert _status(L.fp_adamw_shard, 64, C.byref(hp), ptr[0], C.c_void_p(0x200008), ptr[2], ptr[3],
                   None, None, None, None) == -3
    assert _status(L.fp_adamw_shard, 64, None, *ptr, None, None, None, None) == -1
    assert _status(L.fp_adamw_shard, 64, C.byref(hp), *ptr, None, None, C.c_void_p(0x300004), None) == -3

    sh = (C.c_void_p * 2)(0x10000, 0x20000)
    assert _status(L.fp_unshard, 16, 2, sh, C.c_void_p(0x10010), None) == -1   # source inside full
    assert _status(L.fp_unshard, 16, 2, sh, C.c_void_p(0x30001), None) == -3

    a = _lib.fp_step_args()
    a.shard, a.world, a.rank = 16, 2, 2
    assert _status(L.fp_shard_step, C.byref(a), None) == -2                      # rank out of range
    a.rank, a.flags = 0, 8
    assert _status(L.fp_shard_step, C.byref(a), None) == -1                      # unknown flag
    assert L.fp_workspace_bytes(0) >= 256 + 8
    assert L.fp_workspace_bytes(1 << 30) == 16384 + 8 * ((1 << 30) // 4 // 256 + 1)
    assert _status(L.fp_shard_step, None, None) == -1
    assert L.fp_status_string(-3) == b"misaligned pointer"


# One dispatch carries a 32-bit work-item count: at most (2^32 - 1) // 256
# workgroups of 256 lanes.  Each streaming kernel covers 1024 elements per
# workgroup, each copy 2048 (one 16-byte word per lane).
MAX_GROUPS = (2 ** 32 - 1) // 256


def test_launch_size_limit_without_a_device(fp):
    """Sizes whose grid would not fit one dispatch are refused with
    FP_ERR_RANGE before any launch, with a message naming the limit;
    otherwise valid fake addresses are never dereferenced."""
    from sharded_flatparameter_pack_amd import _lib
    L = fp.lib()
    over = MAX_GROUPS * 1024 + 4                 # one streaming tile too many
    step = 1 << 40                                # keeps the fake buffers apart
    g = (C.c_void_p * 2)(step, 2 * step)
    acc = C.c_void_p(3 * step)

    def refused(status):
        return status == -2 and b"more than one launch holds" in L.fp_last_error()

    assert refused(_status(L.fp_reduce_shard, over, 2, g, 1.0, 0, acc, None, None, None, None))
    assert refused(_status(L.fp_reduce_shard_hybrid, over, 2, 1, g, 1.0, 0, acc, None, None, None, None))
    hp = _lib.fp_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    ptr = [C.c_void_p(step * (i + 1)) for i in range(4)]
    assert refused(_status(L.fp_adamw_shard, over, C.byref(hp), *ptr, None, None, None, None))
    assert refused(_status(L.fp_local_accumulate, over, g[0], 0, acc, None))
    assert refused(_status(L.fp_local_finish, over, g[0], 0, None, acc, None))
    # the unshard: (S / 8 + 1) words per shard, 256 per workgroup
    sh = (C.c_void_p * 2)(step, 2 * step)
    s_copy = (MAX_GROUPS * 256 - 1) * 8 + 8
    assert refused(_status(L.fp_unshard, s_copy, 2, sh, C.c_void_p(4 * step), None))
    # the two-phase step's first launch holds the reduce tiles and the copy
    # tiles of the N - 1 other shards: 1 + 7/2 workgroups per 1024 elements
    # at N = 8, so shards of about 3.8e9 elements (48 bytes each, 180 GB of
    # HBM) are already too large for it
    grads = (C.c_void_p * 8)(*[step * (i + 1) for i in range(8)])
    shards = (C.c_void_p * 8)(None, *[step * (i + 9) for i in range(7)])
    a = _lib.fp_step_args()
    a.world, a.rank, a.scale = 8, 0, 0.125
    a.grads, a.shards = C.cast(grads, C.c_void_p), C.cast(shards, C.c_void_p)
    a.acc, a.master, a.exp_avg, a.exp_avg_sq = 17 * step, 18 * step, 19 * step, 20 * step
    a.hp = _lib.fp_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    a.full, a.found_inf = 21 * step, 29 * step
    a.flags = _lib.FP_STEP_NO_SKIP
    path = C.c_int32(-1)
    a.shard = 3_000_000_000
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
    a.shard = 3_900_000_000
    assert refused(_status(L.fp_step_path, C.byref(a), C.byref(path)))
    assert refused(_status(L.fp_shard_step, C.byref(a), None))


def test_step_path_without_a_device(fp):
    """fp_step_path validates like fp_shard_step and launches nothing; the
    paths that need no occupancy query are decided on the host (fake,
    never-dereferenced addresses)."""
    from sharded_flatparameter_pack_amd import _lib
    L = fp.lib()
    grads = (C.c_void_p * 2)(0x1000000, 0x2000000)
    shards = (C.c_void_p * 2)(None, 0x3000000)
    a = _lib.fp_step_args()
    a.shard, a.world, a.rank, a.scale = 16, 2, 0, 0.5
    a.grads, a.shards = C.cast(grads, C.c_void_p), C.cast(shards, C.c_void_p)
    a.acc, a.master, a.exp_avg, a.exp_avg_sq = 0x4000000, 0x5000000, 0x6000000, 0x7000000
    a.hp = _lib.fp_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    a.full, a.found_inf = 0x8000000, 0x9000000
    path = C.c_int32(-1)
    a.flags = _lib.FP_STEP_NO_SKIP
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
    assert path.value == _lib.FP_PATH_NO_SKIP
    a.flags = _lib.FP_STEP_EXACT_SKIP          # no workspace: no grid barrier
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
    assert path.value == _lib.FP_PATH_TWO_PHASE
    a.workspace, a.flags = 0xA000000, _lib.FP_STEP_NO_COOP
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
    assert path.value == _lib.FP_PATH_TWO_PHASE
    # the test entry of the one-pass give-up refuses arguments of another path
    assert _status(L.fp_step_test_give_up, C.byref(a), None) == -1
    assert b"one-pass" in L.fp_last_error()
    # a kept gradient into an accumulator that is also an input: never one pass
    a.flags, a.accumulate = _lib.FP_STEP_KEEP_GRAD, 1
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
    assert path.value == _lib.FP_PATH_TWO_PHASE
    a.accumulate = 0
    # the entry point without allocation takes no workspace, and refuses a norm
    # over more partials than its array holds, both before touching a device
    assert _status(L.fp_shard_step_noalloc, C.byref(a), None) == -1
    assert b"workspace must be NULL" in L.fp_last_error()
    a.workspace, a.sq_norm, a.shard = None, 0xB000000, 266_337_284
    assert L.fp_workspace_bytes(266_337_283) == 2 << 20 < L.fp_workspace_bytes(266_337_284)
    assert _status(L.fp_shard_step_noalloc, C.byref(a), None) == -2
    assert b"266337283" in L.fp_last_error()
    assert _status(L.fp_shard_step_noalloc, None, None) == -1
    a.sq_norm, a.shard = None, 16
    a.master = 0x4000010                       # overlaps acc
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == -1
    assert _status(L.fp_step_path, C.byref(a), None) == -1
    # shards of 2^24 elements and more: the no-skip step splits off the copies
    step = 1 << 40
    grads2 = (C.c_void_p * 2)(step, 2 * step)
    shards2 = (C.c_void_p * 2)(None, 3 * step)
    a.grads, a.shards = C.cast(grads2, C.c_void_p), C.cast(shards2, C.c_void_p)
    a.acc, a.master, a.exp_avg, a.exp_avg_sq = 4 * step, 5 * step, 6 * step, 7 * step
    a.full, a.found_inf, a.workspace = 8 * step, 9 * step, None
    for S, want in ((1 << 24, _lib.FP_PATH_NO_SKIP_SPLIT), ((1 << 24) - 4, _lib.FP_PATH_NO_SKIP)):
        a.shard, a.flags = S, _lib.FP_STEP_NO_SKIP
        assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
        assert path.value == want
        a.flags = _lib.FP_STEP_EXACT_SKIP
        assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
        assert path.value == _lib.FP_PATH_TWO_PHASE


def test_speculative_step_path_and_checks(fp):
    """With output state buffers and no workspace (so no one-pass kernel, whose
    choice needs the device's occupancy), the exact-skip step takes the
    speculative paths (split from 2^24 elements on) and the no-skip step
    writes the outputs; the output buffers come as all three or none, and
    may overlap no other buffer of the call."""
    from sharded_flatparameter_pack_amd import _lib
    L = fp.lib()
    step = 1 << 40
    grads = (C.c_void_p * 2)(step, 2 * step)
    shards = (C.c_void_p * 2)(None, 3 * step)
    a = _lib.fp_step_args()
    a.world, a.rank, a.scale = 2, 0, 0.5
    a.grads, a.shards = C.cast(grads, C.c_void_p), C.cast(shards, C.c_void_p)
    a.acc, a.master, a.exp_avg, a.exp_avg_sq = 4 * step, 5 * step, 6 * step, 7 * step
    a.hp = _lib.fp_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    a.full, a.found_inf, a.workspace = 8 * step, 9 * step, None
    a.master_out, a.exp_avg_out, a.exp_avg_sq_out = 11 * step, 12 * step, 13 * step
    path = C.c_int32(-1)
    for S, spec, nsk in ((1 << 24, _lib.FP_PATH_SPECULATIVE_SPLIT, _lib.FP_PATH_NO_SKIP_SPLIT),
                         ((1 << 24) - 1, _lib.FP_PATH_SPECULATIVE, _lib.FP_PATH_NO_SKIP),
                         (5, _lib.FP_PATH_SPECULATIVE, _lib.FP_PATH_NO_SKIP)):
        a.shard = S
        for flags, want in ((_lib.FP_STEP_EXACT_SKIP, spec), (_lib.FP_STEP_NO_COOP, spec),
                            (_lib.FP_STEP_KEEP_GRAD, spec), (_lib.FP_STEP_NO_SKIP, nsk)):
            a.flags = flags
            assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0
            assert path.value == want, (S, flags)
    a.flags = _lib.FP_STEP_EXACT_SKIP
    a.exp_avg_out = None                       # two of three
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == -1
    a.exp_avg_out = 12 * step + 2              # misaligned
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == -3
    for alias in (5 * step + 16, 4 * step, 11 * step + 16, 8 * step, step):
        a.exp_avg_out = alias                  # overlaps master, acc, master_out, full, a gradient row
        assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == -1, hex(alias)
        assert _status(L.fp_shard_step, C.byref(a), None) == -1
    a.exp_avg_out = 12 * step
    assert _status(L.fp_step_path, C.byref(a), C.byref(path)) == 0


def test_units_validation_without_a_device(fp):
    """fp_units_create rejects bad arguments before any device call."""
    L = fp.lib()
    out = C.c_void_p()
    sizes = (C.c_int64 * 2)(16, 8)
    g = (C.c_void_p * 4)(0x1000000, 0x2000000, 0x3000000, 0x4000000)
    assert _status(L.fp_units_create, 0, 2, 0, sizes, g, None, None, C.byref(out)) == -2   # no units
    assert _status(L.fp_units_create, 2, 0, 0, sizes, g, None, None, C.byref(out)) == -2   # world 0
    assert _status(L.fp_units_create, 2, 2, 2, sizes, g, None, None, C.byref(out)) == -2   # rank
    assert _status(L.fp_units_create, 2, 2, 0, None, g, None, None, C.byref(out)) == -1
    assert _status(L.fp_units_create, 2, 2, 0, sizes, None, None, None, C.byref(out)) == -1
    full = (C.c_void_p * 2)(0x5000000, 0x6000000)
    assert _status(L.fp_units_create, 2, 2, 0, sizes, g, None, full, C.byref(out)) == -1  # shards missing
    g_odd = (C.c_void_p * 4)(0x1000000, 0x2000001, 0x3000000, 0x4000000)
    assert _status(L.fp_units_create, 2, 2, 0, sizes, g_odd, None, None, C.byref(out)) == -3
    g_null = (C.c_void_p * 4)(0x1000000, None, 0x3000000, 0x4000000)
    assert _status(L.fp_units_create, 2, 2, 0, sizes, g_null, None, None, C.byref(out)) == -1
    neg = (C.c_int64 * 2)(16, -1)
    assert _status(L.fp_units_create, 2, 2, 0, neg, g, None, None, C.byref(out)) == -2
    # a gradient row inside its unit's full buffer
    sh = (C.c_void_p * 4)(None, 0x7000000, None, 0x8000000)
    g_in = (C.c_void_p * 4)(0x5000000, 0x2000000, 0x3000000, 0x4000000)
    assert _status(L.fp_units_create, 2, 2, 0, sizes, g_in, sh, full, C.byref(out)) == -1
    assert out.value is None
    assert _status(L.fp_units_info, None, None, None) == -1
    assert _status(L.fp_units_reduce, None, 1.0, 0, None, None, None, None, None) == -1
    assert _status(L.fp_units_step, None, None, None) == -1
    L.fp_units_destroy(None)


@pytest.mark.parametrize("seed", range(20))
def test_shard0_geometry_and_views_match_oracle(fp, seed):
    r = np.random.default_rng(100 + seed)
    shapes = _random_shapes(r)
    world = int(r.choice([1, 2, 3, 4, 7, 8, 64]))
    plan = fp.Shard0Plan(shapes, world)
    c, rows_elems, off, S = oracle.shard0_geometry(shapes, world)
    assert plan.shard == S
    assert plan.numel == sum(math.prod(s) for s in shapes)
    for rank in sorted(set(int(x) for x in r.integers(0, world, size=4))):
        for i, d in enumerate(plan.view_descriptors(rank)):
            d0 = shapes[i][0] if shapes[i] else 1
            real = max(0, min(c[i], d0 - rank * c[i]))
            assert d["tensor"] == i
            assert d["buf_offset"] == off[i]
            assert d["numel"] == real * rows_elems[i]
            assert d["tensor_offset"] == (rank * c[i] * rows_elems[i] if d["numel"] else 0)
            assert d["shape"] == (real,) + tuple(shapes[i][1:])


def test_shard0_validation_without_a_device(fp):
    """The dim-0 entry points reject bad arguments before any device call
    (fake, never-dereferenced addresses)."""
    L = fp.lib()
    h = C.c_void_p()
    nd = (C.c_int32 * 2)(2, 0)
    dims = (C.c_int64 * 2)(4, 2)
    assert _status(L.fp_shard0_plan_create, 0, nd, dims, 2, C.byref(h)) == -2
    assert _status(L.fp_shard0_plan_create, 2, nd, dims, 0, C.byref(h)) == -2
    assert _status(L.fp_shard0_plan_create, 2, None, dims, 2, C.byref(h)) == -1
    assert _status(L.fp_shard0_plan_create, 2, nd, None, 2, C.byref(h)) == -1
    bad = (C.c_int64 * 2)(4, -2)
    assert _status(L.fp_shard0_plan_create, 2, nd, bad, 2, C.byref(h)) == -2
    huge = (C.c_int64 * 2)(1 << 40, 1 << 30)
    assert _status(L.fp_shard0_plan_create, 2, nd, huge, 2, C.byref(h)) == -2
    plan = fp.Shard0Plan([(4, 2), ()], 2)
    assert plan.shard == 2 * 2 + 1
    out = (fp._lib.fp_view * 2)()
    n = C.c_int32()
    assert _status(L.fp_shard0_views, plan._h, 0, out, 1, C.byref(n)) == -2 and n.value == 2
    assert _status(L.fp_shard0_views, plan._h, 2, out, 2, C.byref(n)) == -2
    assert _status(L.fp_shard0_views, plan._h, -1, out, 2, C.byref(n)) == -2
    p = (C.c_void_p * 2)(0x100000, 0x200000)
    dst = C.c_void_p(0x300000)
    assert _status(L.fp_shard0_pack, plan._h, 3, 0, p, dst, None) == -1        # elem_size
    assert _status(L.fp_shard0_pack, plan._h, 2, 2, p, dst, None) == -2        # rank
    assert _status(L.fp_shard0_pack, plan._h, 2, -2, p, dst, None) == -2
    assert _status(L.fp_shard0_pack, plan._h, 2, 0, None, dst, None) == -1
    assert _status(L.fp_shard0_pack, plan._h, 2, 0, p, None, None) == -1
    assert _status(L.fp_shard0_pack, plan._h, 4, 0, p, C.c_void_p(0x300002), None) == -3
    assert _status(L.fp_shard0_pack, plan._h, 2, 0, (C.c_void_p * 2)(0x100001, 0x200000), dst, None) == -3
    assert _status(L.fp_shard0_pack, plan._h, 2, 0, (C.c_void_p * 2)(None, 0x200000), dst, None) == -1
    assert _status(L.fp_shard0_pack, plan._h, 2, -1, (C.c_void_p * 2)(0x300004, 0x200000), dst, None) == -1
    assert _status(L.fp_shard0_unpack, plan._h, 2, None, p, None) == -1
    assert _status(L.fp_shard0_unpack, plan._h, 2, dst, (C.c_void_p * 2)(0x300004, 0x200000), None) == -1
    assert _status(L.fp_shard0_unpack, plan._h, 2, dst, (C.c_void_p * 2)(0x100000, 0x100002), None) == -1
    assert _status(L.fp_shard0_unpack, None, 2, dst, p, None) == -1
    assert _status(L.fp_shard0_plan_info, None, None, None) == -1
    L.fp_shard0_plan_destroy(None)


def test_local_and_scaler_validation_without_a_device(fp):
    """no_sync accumulation, the gradient factor and the loss-scale update
    reject bad arguments before any launch (fake addresses)."""
    L = fp.lib()
    g, loc, out = C.c_void_p(0x100000), C.c_void_p(0x200000), C.c_void_p(0x300000)
    assert _status(L.fp_local_accumulate, -1, g, 0, loc, None) == -2
    assert _status(L.fp_local_accumulate, 0, None, 0, None, None) == 0          # nothing to do
    assert _status(L.fp_local_accumulate, 16, None, 0, loc, None) == -1
    assert _status(L.fp_local_accumulate, 16, C.c_void_p(0x100001), 0, loc, None) == -3
    assert _status(L.fp_local_accumulate, 16, g, 1, C.c_void_p(0x200008), None) == -3
    assert _status(L.fp_local_accumulate, 16, g, 1, None, None) == -1
    assert _status(L.fp_local_accumulate, 16, C.c_void_p(0x200010), 1, loc, None) == -1   # grad inside local
    assert _status(L.fp_local_finish, 16, g, 1, loc, None, None) == -1
    assert _status(L.fp_local_finish, 16, g, 1, None, out, None) == -1                      # accumulate needs local
    assert _status(L.fp_local_finish, 16, g, 0, None, C.c_void_p(0x300001), None) == -3
    assert _status(L.fp_local_finish, 16, g, 0, None, C.c_void_p(0x100008), None) == -1     # out overlaps grad
    assert _status(L.fp_local_finish, 16, g, 1, loc, C.c_void_p(0x200010), None) == -1      # out overlaps local
    coef, sq, ls = C.c_void_p(0x400000), C.c_void_p(0x500000), C.c_void_p(0x600000)
    assert _status(L.fp_grad_coef, sq, ls, 1.0, None, None) == -1
    assert _status(L.fp_grad_coef, sq, ls, 1.0, C.c_void_p(0x400004), None) == -3
    assert _status(L.fp_grad_coef, None, ls, 1.0, coef, None) == -1                # clipping needs the norm
    assert _status(L.fp_grad_coef, C.c_void_p(0x500004), ls, 1.0, coef, None) == -3
    assert _status(L.fp_grad_coef, None, C.c_void_p(0x600002), 0.0, coef, None) == -3
    assert _status(L.fp_grad_coef, None, None, float("nan"), coef, None) == -1
    fi, sc, cs = C.c_void_p(0x700000), C.c_void_p(0x700010), C.c_void_p(0x700020)
    assert _status(L.fp_scaler_update, None, sc, cs, 2.0, 0.5, 2000, None) == -1
    assert _status(L.fp_scaler_update, fi, sc, cs, 2.0, 0.5, 0, None) == -2
    assert _status(L.fp_scaler_update, fi, sc, cs, 0.0, 0.5, 10, None) == -2
    assert _status(L.fp_scaler_update, fi, C.c_void_p(0x700011), cs, 2.0, 0.5, 10, None) == -3


def test_hybrid_validation_without_a_device(fp):
    L = fp.lib()
    g = (C.c_void_p * 4)(0x10000, 0x20000, 0x30000, 0x40000)
    acc = C.c_void_p(0x50000)
    assert _status(L.fp_reduce_shard_hybrid, 16, 4, 3, g, 1.0, 0, acc, None, None, None, None) == -2
    assert _status(L.fp_reduce_shard_hybrid, 16, 4, 0, g, 1.0, 0, acc, None, None, None, None) == -2
    assert _status(L.fp_reduce_shard_hybrid, 16, 4, 8, g, 1.0, 0, acc, None, None, None, None) == -2
    assert _status(L.fp_reduce_shard_hybrid, 16, 4, 2, g, 1.0, 0, C.c_void_p(0x50004), None, None, None,
                   None) == -3
    g_null = (C.c_void_p * 4)(0x10000, None, 0x30000, 0x40000)
    assert _status(L.fp_reduce_shard_hybrid, 16, 4, 2, g_null, 1.0, 0, acc, None, None, None, None) == -1


def test_reshard_plan_and_validation_without_a_device(fp):
    L = fp.lib()
    h = C.c_void_p()
    assert _status(L.fp_reshard_plan_create, -1, 2, 3, C.byref(h)) == -2
    assert _status(L.fp_reshard_plan_create, 10, 0, 3, C.byref(h)) == -2
    assert _status(L.fp_reshard_plan_create, 10, 2, 0, C.byref(h)) == -2
    plan = fp.ReshardPlan(10, 4, 3)
    assert (plan.shard_old, plan.shard_new) == (3, 4)
    assert fp.ReshardPlan(0, 4, 3).shard_new == 0
    old = (C.c_void_p * 4)(0x100000, 0x200000, 0x300000, None)   # rank 3 holds only padding
    dst = C.c_void_p(0x400000)
    assert _status(L.fp_reshard, plan._h, 3, -1, old, dst, None) == -1
    assert _status(L.fp_reshard, plan._h, 2, 3, old, dst, None) == -2
    assert _status(L.fp_reshard, plan._h, 2, -2, old, dst, None) == -2
    assert _status(L.fp_reshard, plan._h, 2, -1, None, dst, None) == -1
    assert _status(L.fp_reshard, plan._h, 2, -1, old, None, None) == -1
    assert _status(L.fp_reshard, plan._h, 4, -1, old, C.c_void_p(0x400002), None) == -3
    bad = (C.c_void_p * 4)(0x100000, None, 0x300000, None)
    assert _status(L.fp_reshard, plan._h, 2, -1, bad, dst, None) == -1
    ov = (C.c_void_p * 4)(0x100000, 0x400004, 0x300000, None)
    assert _status(L.fp_reshard, plan._h, 2, -1, ov, dst, None) == -1
    assert _status(L.fp_reshard_plan_info, None, None, None) == -1
    L.fp_reshard_plan_destroy(None)


def test_binding_rejects_tensors_on_several_devices(fp):
    """The binding checks that one call's tensors share a device before it
    marshals anything (a CPU and a meta tensor stand in for two devices)."""
    import torch
    from sharded_flatparameter_pack_amd import _one_device
    a, b = torch.empty(8), torch.empty(8, device="meta")
    _one_device(a, [a, None], None, [[a], (a,)])
    with pytest.raises(ValueError, match="several devices"):
        _one_device(a, [[a, b]])
    with pytest.raises(ValueError, match="several devices"):
        fp.unshard([a, b], a)
    with pytest.raises(ValueError, match="several devices"):
        fp.reduce_shard(torch.empty(2, 8, dtype=torch.int16), b, scale=0.5)
