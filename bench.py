"""Throughput of one rank's shard step (reduce + AdamW + bf16 cast + unshard).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--mode speculative|exact|twophase|noskip] [--timing auto|graph|eager]

A step is the whole per-step hot path for rank r's shard: the fixed-order
reduce of the N_d ranks' bf16 gradients for every micro-batch, the AdamW
update of the fp32 master / moments with the overflow gate, the bf16 cast
of the own shard into the full buffer and the copy of the other N_d - 1
shards into it.  Single-unit workloads run fp_shard_step; the bucketed
workload runs the multi-unit entry points, one launch per micro-batch over
all buckets.  Pack and views are one-time set-up per unit and are not part
of a step; pack throughput is reported on its own.

With no flags the line is the d=12288 layer unit (226.5M-element shard,
N_d = 8, the largest workload that is one unit on one GPU) with the exact
overflow skip in its speculative form (separate output state, swapped each
step); `configs` carries the 10k-tensor group at 64 ranks and the bucketed
611M model the same way.

All inputs are synthetic and resident in HBM before timing starts.  The
step rotates over enough buffer sets (>= 1.5 GB) that no step finds its
data in the 256 MB Infinity Cache left behind by the previous ones.
Exactly K steps are timed.

Output: one JSON line.  `value` is algorithmic GB/s of the whole step,
B = 2*N*n + 8*(n-1) + 24 + 2 + 4*(N-1) bytes per shard element; `roofline`
takes the dominant kernel's average duration from HIP events that the
library records around its kernels on its stream; `cpu_baseline` times the
serial CPU oracle on a bounded sample of the same workload on one host core.
"""

from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "shard-step GB/s and params/s (reduce+AdamW+unshard), % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
ROTATE_BYTES = 1.5e9           # buffer-set rotation span, > 256 MB Infinity Cache
KERNEL_SOURCES = ["sharded_flatparameter_pack_amd/csrc/step_kernels.hip",
                  "sharded_flatparameter_pack_amd/csrc/unit_kernels.hip",
                  "sharded_flatparameter_pack_amd/csrc/step_ops.h",
                  "sharded_flatparameter_pack_amd/csrc/fp_device.h",
                  "sharded_flatparameter_pack_amd/csrc/fp_internal.h"]
MODE_FLAGS = {"speculative": "FP_STEP_EXACT_SKIP", "exact": "FP_STEP_EXACT_SKIP", "twophase": "FP_STEP_NO_COOP",
              "noskip": "FP_STEP_NO_SKIP"}
# modes that give the step separate output state buffers
OUT_OF_PLACE_MODES = {"speculative"}
DEFAULT_WORKLOAD = "c4_layer_d12288_nd8"
SIDE_WORKLOADS = ("c5_ragged10k_nd64", "c3_611m_buckets_nd16")
EAGER_MIN_MS = 0.2             # auto timing: steps this long are timed eagerly with per-kernel events


def step_bytes_per_elem(world: int, n_micro: int) -> int:
    """Algorithmic bytes per shard element of one shard step."""
    return 2 * world * n_micro + 8 * (n_micro - 1) + 24 + 2 + 4 * (world - 1)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    # Timing-only events: no system-scope fence (cache write-back and
    # invalidate) when an event is recorded, which would otherwise land inside
    # the kernel spans that the events bracket.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.L = C.CDLL("libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.L.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventSynchronize.argtypes = [C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = C.c_void_p()
        if self.L.hipEventCreateWithFlags(C.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value

    def record(self, e, stream):
        if self.L.hipEventRecord(C.c_void_p(e), C.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        if self.L.hipEventSynchronize(C.c_void_p(b)) != 0 or \
                self.L.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(C.c_void_p(e))


# ------------------------------------------------------------------ workloads
def row_stride(S: int) -> int:
    """Elements between consecutive simulated ranks' rows of S bf16 elements
    cut from one tensor: S rounded up to 64, so that every row starts on a
    128-byte cache line, as a separate allocation would (the torch allocator
    aligns blocks to 512 bytes)."""
    return -(-S // 64) * 64


class SingleUnit:
    """Buffer sets of one rank's step on one unit (fp_shard_step)."""

    def __init__(self, cfg, rank, dev, flags, out_of_place=False, n_sets=None):
        import torch
        import sharded_flatparameter_pack_amd as fp
        from workloads import gen
        self.cfg, self.rank, self.world, self.n_micro = cfg, rank, cfg.world, cfg.n_micro
        self.dev = dev
        self.S = S = -(-cfg.units()[0] // cfg.world)
        world = self.world
        per_set = S * (2 * world + 16 + 2 * (world - 1) + 2 * world)
        self.n_sets = n_sets or max(2, math.ceil(ROTATE_BYTES / per_set))
        self.sets = []
        Sp = row_stride(S)
        for k in range(self.n_sets):
            key = lambda stream, q=0: (stream, k, 0, q)  # noqa: E731
            grads = gen.torch_bf16_normal(world * Sp, cfg.grad_sigma, cfg.seed, key(gen.STREAM_GRAD), dev)
            others = gen.torch_bf16_normal(world * Sp, cfg.master_sigma, cfg.seed, key(gen.STREAM_SHARD), dev)
            s = dict(grads=grads.view(world, Sp)[:, :S],
                     shards=[None if q == rank else others[q * Sp:q * Sp + S] for q in range(world)],
                     master=gen.torch_normal_f32(S, cfg.master_sigma, cfg.seed, key(gen.STREAM_MASTER), dev),
                     exp_avg=torch.zeros(S, dtype=torch.float32, device=dev),
                     exp_avg_sq=torch.zeros(S, dtype=torch.float32, device=dev),
                     acc=torch.zeros(S, dtype=torch.float32, device=dev),
                     full=torch.zeros(world * S, dtype=torch.int16, device=dev),
                     found_inf=torch.zeros(1, dtype=torch.int32, device=dev),
                     workspace=fp.new_workspace(dev, S))
            self.sets.append(s)
        self.set_flags(flags, out_of_place)

    def set_flags(self, flags, out_of_place=False):
        """Calls of every set with these flags.  out_of_place: each set also
        gets output state buffers; the step alternates two calls whose input
        and output buffers are swapped (a graph of one step per set replays
        the first of them, which moves the same bytes)."""
        import torch
        import sharded_flatparameter_pack_amd as fp
        hp, world = self.cfg.hp, self.world

        def call(s, state, out):
            return fp.ShardStep(s["grads"], s["acc"], *state, s["shards"], s["full"], self.rank,
                                scale=1.0 / world, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                                weight_decay=hp.weight_decay, found_inf=s["found_inf"],
                                workspace=s["workspace"], flags=flags, out=out)

        self.out_of_place = out_of_place
        self.calls = []
        for s in self.sets:
            state = [s["master"], s["exp_avg"], s["exp_avg_sq"]]
            if not out_of_place:
                s.pop("out", None)
                self.calls.append([call(s, state, None)])
                continue
            if "out" not in s:
                s["out"] = [torch.zeros(self.S, dtype=torch.float32, device=self.dev) for _ in range(3)]
            self.calls.append([call(s, state, s["out"]), call(s, s["out"], state)])
        self.path = self.calls[0][0].path()

    def n_events(self):
        return 3

    def state_io(self, i):
        """(input state, output state or None) of step i on its set."""
        s = self.sets[i % self.n_sets]
        state = [s["master"], s["exp_avg"], s["exp_avg_sq"]]
        if not self.out_of_place:
            return state, None
        return (state, s["out"]) if (i // self.n_sets) % 2 == 0 else (s["out"], state)

    def step(self, i, events=None):
        calls = self.calls[i % self.n_sets]
        k = i // self.n_sets
        calls[k % len(calls)](k + 1, events)

    def kernels(self, ev_ms):
        """(name, rocprof id, ms per launch, algorithmic bytes per launch, launches per step),
        durations from the mean event offsets of a step (the library's events)."""
        import sharded_flatparameter_pack_amd as fp
        S, N = self.S, self.world
        B = step_bytes_per_elem(N, 1)
        k1, k2 = ev_ms[1] - ev_ms[0], ev_ms[2] - ev_ms[1]
        if self.path in (fp.FP_PATH_NO_SKIP, fp.FP_PATH_SPECULATIVE):
            # (the speculative step's restore kernel runs between the second and third
            # event and returns at once without overflow)
            return [("step_phase1_kernel<true>", "step_phase1_fused", k1, S * B, 1)]
        if self.path in (fp.FP_PATH_ONE_PASS, fp.FP_PATH_SPECULATIVE_ONE_PASS):
            return [("step_coop_kernel", "step_coop", k1, S * B, 1)]
        if self.path in (fp.FP_PATH_NO_SKIP_SPLIT, fp.FP_PATH_SPECULATIVE_SPLIT):
            # fused reduce + AdamW + cast, then the copies (and the restore kernel)
            return [("step_phase1_kernel<true>", "step_phase1_fused", k1, S * (B - 4 * (N - 1)), 1),
                    ("unshard_kernel", "unshard", k2, S * 4 * (N - 1), 1)]
        return [("step_phase1_kernel<false>", "step_phase1", k1, S * (2 * N + 4 * (N - 1)), 1),
                ("adamw_kernel", "adamw", k2, S * 26, 1)]

    def flagged(self):
        import sharded_flatparameter_pack_amd as fp
        if any(int(s["found_inf"].item()) for s in self.sets):
            return "unexpected overflow flag in a finite workload"
        if any(fp.workspace_timeouts(s["workspace"]) for s in self.sets):
            return "grid barrier wait gave up"
        return None


class Bucketed:
    """Buffer sets of one rank's step on all buckets of a bucketed model: one
    multi-unit reduce launch per earlier micro-batch, then fp_units_step."""

    def __init__(self, cfg, rank, dev, flags, out_of_place=False, n_sets=None):
        import torch
        import sharded_flatparameter_pack_amd as fp
        from workloads import gen
        self.cfg, self.rank, self.world, self.n_micro = cfg, rank, cfg.world, cfg.n_micro
        self.dev = dev
        N, n = cfg.world, cfg.n_micro
        sizes = [-(-T // N) for T in cfg.units()]
        self.sizes = sizes
        self.S = sum(sizes)
        per_set = self.S * (2 * N * n + 16 + 4 * N)
        self.n_sets = n_sets or max(2, math.ceil(ROTATE_BYTES / per_set))
        offs = [0]
        for S in sizes[:-1]:
            offs.append(offs[-1] + S)
        self.offsets = offs
        self.sets = []
        for k in range(self.n_sets):
            # rank q's gradient (and shard) rows of bucket b are slices of one
            # buffer per set and micro-batch; rank q's row starts a cache line
            Rp = row_stride(self.S)
            grads = [gen.torch_bf16_normal(N * Rp, cfg.grad_sigma, cfg.seed, (gen.STREAM_GRAD, k, m), dev)
                     .view(N, Rp) for m in range(n)]
            others = gen.torch_bf16_normal(N * Rp, cfg.master_sigma, cfg.seed, (gen.STREAM_SHARD, k),
                                           dev).view(N, Rp)
            full = [torch.zeros(N * S, dtype=torch.int16, device=dev) for S in sizes]
            g_rows = [[[grads[m][q, o:o + S] for q in range(N)] for o, S in zip(offs, sizes)]
                      for m in range(n)]
            sh_rows = [[None if q == rank else others[q, o:o + S] for q in range(N)]
                       for o, S in zip(offs, sizes)]
            plans = [fp.Units(g_rows[m], rank, shards=sh_rows, full=full) for m in range(n)]
            P = plans[0].partition
            self.sets.append(dict(plans=plans, grads=grads, others=others, full=full,
                                  master=gen.torch_normal_f32(P, cfg.master_sigma, cfg.seed,
                                                              (gen.STREAM_MASTER, k), dev),
                                  exp_avg=torch.zeros(P, dtype=torch.float32, device=dev),
                                  exp_avg_sq=torch.zeros(P, dtype=torch.float32, device=dev),
                                  acc=torch.zeros(P, dtype=torch.float32, device=dev),
                                  found_inf=torch.zeros(1, dtype=torch.int32, device=dev)))
        self.ev = HipEvents()
        self.set_flags(flags, out_of_place)

    def set_flags(self, flags, out_of_place=False):
        """Flags of the last micro-batch's call; out_of_place: each set also gets
        output partitions, and successive steps on a set swap input and output
        (as the single-unit workload does)."""
        import torch
        import sharded_flatparameter_pack_amd as fp
        self.flags = flags & fp.FP_STEP_NO_SKIP       # the multi-unit step has no one-pass form
        self.out_of_place = out_of_place
        for s in self.sets:
            if not out_of_place:
                s.pop("out", None)
            elif "out" not in s:
                P = s["plans"][0].partition
                s["out"] = [torch.zeros(P, dtype=torch.float32, device=self.dev) for _ in range(3)]
        s0 = self.sets[0]
        self.path = s0["plans"][-1].step_path(s0["acc"], s0["master"], s0["exp_avg"], s0["exp_avg_sq"],
                                              found_inf=s0["found_inf"], flags=self.flags,
                                              out=s0.get("out"))

    def n_events(self):
        return self.n_micro + 2

    def state_io(self, i):
        """(input state, output state or None) of step i on its set."""
        s = self.sets[i % self.n_sets]
        state = [s["master"], s["exp_avg"], s["exp_avg_sq"]]
        if not self.out_of_place:
            return state, None
        return (state, s["out"]) if (i // self.n_sets) % 2 == 0 else (s["out"], state)

    def step(self, i, events=None):
        import torch
        s = self.sets[i % self.n_sets]
        hp, n = self.cfg.hp, self.n_micro
        scale = 1.0 / (self.world * n)
        stream = torch.cuda.current_stream().cuda_stream
        for m in range(n - 1):
            if events is not None:
                self.ev.record(events[m], stream)
            s["plans"][m].reduce(s["acc"], scale=scale, accumulate=m > 0, found_inf=s["found_inf"])
        state, out = self.state_io(i)
        s["plans"][n - 1].step(s["acc"], *state, scale=scale,
                               accumulate=n > 1, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                               weight_decay=hp.weight_decay, step=i // self.n_sets + 1,
                               found_inf=s["found_inf"], flags=self.flags, out=out,
                               profile_events=None if events is None else events[n - 1:n + 2])

    def kernels(self, ev_ms):
        import sharded_flatparameter_pack_amd as fp
        S, N, n = self.S, self.world, self.n_micro
        d = [ev_ms[i + 1] - ev_ms[i] for i in range(n + 1)]
        out = []
        acc_in = 4 if n > 1 else 0
        if n > 1:
            t_red = sum(d[:n - 1])
            alg_red = S * (2 * N * (n - 1) + 4 + 8 * (n - 2))   # the first writes acc, later ones read + write
            out.append(("units_reduce_kernel", "units_reduce", t_red / (n - 1), alg_red / (n - 1), n - 1))
        if self.path in (fp.FP_PATH_NO_SKIP_SPLIT, fp.FP_PATH_SPECULATIVE_SPLIT):
            # fused reduce + AdamW + casts, then the copies (and the restore kernel,
            # which returns at once without overflow)
            out.append(("units_phase1_kernel<true>", "units_phase1_fused", d[n - 1],
                        S * (2 * N + acc_in + 26), 1))
            out.append(("units_copy_kernel", "units_copy", d[n], S * 4 * (N - 1), 1))
        elif self.path != fp.FP_PATH_TWO_PHASE:
            # fused reduce + AdamW + casts + copies; the restore kernel (speculative)
            # follows between the last two events and returns at once without overflow
            out.append(("units_phase1_kernel<true>", "units_phase1_fused", d[n - 1],
                        S * (2 * N + acc_in + 26 + 4 * (N - 1)), 1))
        else:
            out.append(("units_phase1_kernel<false>", "units_phase1", d[n - 1],
                        S * (2 * N + acc_in + 4 * (N - 1)), 1))
            out.append(("units_adamw_kernel", "units_adamw", d[n], S * 26, 1))
        return out

    def flagged(self):
        if any(int(s["found_inf"].item()) for s in self.sets):
            return "unexpected overflow flag in a finite workload"
        return None


def make_workload(cfg, rank, dev, flags, out_of_place=False, n_sets=None):
    if cfg.shapes is None:
        return Bucketed(cfg, rank, dev, flags, out_of_place, n_sets)
    if cfg.n_micro == 1:
        return SingleUnit(cfg, rank, dev, flags, out_of_place, n_sets)
    raise ValueError("single-unit workloads with several micro-batches are not benchmarked")


# ------------------------------------------------------------------ timing
def time_steps(w, K, W, timing, ev):
    """Time exactly K steps after W warm-up steps.

    Returns (step ms, mean event offsets of a step in ms, how).  timing:
    "eager" launches every step from Python with the library's per-kernel
    events recorded inside the timed region; "graph" replays HIP graphs of
    one step per buffer set (plus a graph of the K mod sets remaining steps),
    then takes the per-kernel split from an eager pass with events; "auto"
    picks eager for steps of EAGER_MIN_MS and more (not launch-bound), else
    graph."""
    import torch
    for i in range(W):
        w.step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    if timing == "auto":
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(2):
            w.step(W + i)
        b.record()
        torch.cuda.synchronize()
        timing = "eager" if a.elapsed_time(b) / 2 >= EAGER_MIN_MS else "graph"
        W += 2

    def eager_pass(first, count):
        evs = [[ev.create() for _ in range(w.n_events())] for _ in range(count)]
        marks = [ev.create(), ev.create()]
        torch.cuda.synchronize()
        ev.record(marks[0], stream)
        for k in range(count):
            w.step(first + k, evs[k])
        ev.record(marks[1], stream)
        torch.cuda.synchronize()
        total = ev.elapsed_ms(marks[0], marks[1])
        mean = [0.0] * w.n_events()
        # each step from its first event to the next step's (the last one to the end mark)
        per_step = [ev.elapsed_ms(evs[k][0], evs[k + 1][0] if k + 1 < count else marks[1])
                    for k in range(count)]
        for e in evs:
            for j in range(1, len(e)):
                mean[j] += ev.elapsed_ms(e[0], e[j]) / count
            for x in e:
                ev.destroy(x)
        for x in marks:
            ev.destroy(x)
        return total / count, mean, sorted(per_step)

    time_steps.spread = None
    if timing == "eager":
        step_ms, ev_ms, per_step = eager_pass(W, K)
        time_steps.spread = {"median_ms_per_step": round(per_step[len(per_step) // 2], 5),
                             "min_ms_per_step": round(per_step[0], 5),
                             "max_ms_per_step": round(per_step[-1], 5), "steps": K,
                             "how": "each step from the library's first event of the step to the next step's"}
        return step_ms, ev_ms, ("eager launches from Python, exactly K steps; step time from hipEvents around "
                                "the region, per-kernel times from the hipEvents the library records around "
                                "its kernels on its stream inside the same region")
    n = w.n_sets
    reps, rem = divmod(K, n)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            w.step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for count in (n if reps else 0, rem):
        if count == 0:
            graphs.append(None)
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                w.step(i)
        graphs.append(g)
    main, tail = graphs
    for _ in range(max(1, W // n)):
        (main or tail).replay()
    torch.cuda.synchronize()
    # an event between replays as well, for the spread over replays (one replay = n steps)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
    marks[0].record()
    for r in range(reps):
        main.replay()
        marks[r + 1].record()
    if tail is not None:
        tail.replay()
    marks[-1].record()
    torch.cuda.synchronize()
    step_ms = marks[0].elapsed_time(marks[-1]) / K
    if reps:
        per_replay = sorted(marks[r].elapsed_time(marks[r + 1]) / n for r in range(reps))
        time_steps.spread = {"median_ms_per_step": round(per_replay[len(per_replay) // 2], 5),
                             "min_ms_per_step": round(per_replay[0], 5),
                             "max_ms_per_step": round(per_replay[-1], 5), "replays": reps,
                             "steps_per_replay": n, "tail_steps": rem}
    del graphs, main, tail
    _, ev_ms, _ = eager_pass(W + K, min(K, 200))
    # An eager step of a short shard is host-bound: the GPU waits between the
    # library's events, so the eager per-kernel split is scaled to the graph's
    # step time (for a one-kernel step, its kernel time is the step time).
    span = ev_ms[-1]
    if span > 0:
        ev_ms = [x * step_ms / span for x in ev_ms]
    return step_ms, ev_ms, ("HIP graphs of one step per buffer set (and of the K mod sets remaining steps), "
                            "replayed for exactly K steps; span timed by hipEvents on the replay stream; "
                            "per-kernel split from the library's hipEvents in an eager pass of min(K, 200) "
                            "steps, scaled to the graph's step time")


def measure(w, K, W, timing, ev, B):
    """One timed run of workload w: the step and its kernels."""
    step_ms, ev_ms, how = time_steps(w, K, W, timing, ev)
    kernels = w.kernels(ev_ms)
    name, kernel_id, dur_ms, alg, _ = max(kernels, key=lambda x: x[2] * x[4])
    gbs = w.S * B / (step_ms * 1e-3) / 1e9
    return dict(step_ms=step_ms, gbs=gbs, kernels=kernels, dominant=(name, kernel_id, dur_ms, alg), how=how,
                spread=time_steps.spread)


def pack_bench(cfg, dev, reps: int):
    """fp_pack of the workload's FlatParameter (fp32 tensors): elements/s and GB/s."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    plan = fp.Plan(cfg.shapes, cfg.world)
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    tensors = [torch.randn(s, generator=g, device=dev, dtype=torch.float32) for s in cfg.shapes]
    flat = torch.empty(plan.padded, dtype=torch.float32, device=dev)
    pack = plan.packer(tensors, flat)
    pack()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pack()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    alg = 4 * plan.numel + 4 * plan.padded
    gbs = alg / (ms * 1e-3) / 1e9
    out = {"workload": cfg.name, "tensors": len(cfg.shapes), "elements": plan.numel, "padded": plan.padded,
           "dtype": "fp32", "us_per_pack": round(ms * 1e3, 2), "elements_per_s": round(plan.numel / (ms * 1e-3), 1),
           "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "timing": f"hipEvents around {reps} back-to-back fp_pack calls on one stream (tensors "
                     f"marshalled beforehand; the pointer table is uploaded once), mean"}
    plan.close()
    return out


def shard0_bench(cfg, dev, reps: int):
    """The per-parameter dim-0 layout of the workload's parameter group in
    bf16: fp_shard0_pack of every rank's rows (full-shape gradients to the
    rank-major reduce-scatter input) and fp_shard0_unpack (the gathered
    buffer back to full-shape parameters).  The parameters (and the unpack's
    outputs) are consecutive views of one allocation each."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    from workloads import gen
    plan = fp.Shard0Plan(cfg.shapes, cfg.world)
    T, N, S = plan.numel, cfg.world, plan.shard

    def split(flat):          # consecutive views of one allocation, one per parameter
        out, o = [], 0
        for s in cfg.shapes:
            n = math.prod(s)
            out.append(flat[o:o + n].view(s))
            o += n
        return out
    params = split(gen.torch_bf16_normal(T, 1e-3, cfg.seed, (gen.STREAM_TENSOR,), dev))
    full = torch.empty(N * S, dtype=torch.int16, device=dev)
    outs = split(torch.empty(T, dtype=torch.int16, device=dev))
    legs = {"pack_all_ranks": (plan.packer(params, full), 2 * T + 2 * N * S),
            "unpack": (plan.unpacker(full, outs), 4 * T)}
    out = {"workload": cfg.name, "params": len(cfg.shapes), "elements": T, "N_d": N,
           "shard_elems": S, "dtype": "bf16"}
    for name, (run, alg) in legs.items():
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = alg / (ms * 1e-3) / 1e9
        out[name] = {"us_per_call": round(ms * 1e3, 2), "alg_bytes": alg, "GBps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    out["timing"] = (f"hipEvents around {reps} back-to-back calls on one stream (pointer-table upload + "
                     f"kernel), mean; pack moves 2T + 2*N_d*S bytes (padding rows written), "
                     f"unpack 4T")
    plan.close()
    return out


def nosync_bench(cfg, dev, reps: int):
    """Accumulation without communication over the rank's whole unit (T
    elements of the workload, bf16 gradients, fp32 local buffer):
    fp_local_accumulate of a later micro-batch (reads 2 + 4, writes 4 bytes
    per element) and fp_local_finish (reads 2 + 4, writes 2)."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    from workloads import gen
    T = sum(cfg.units())
    grad = gen.torch_bf16_normal(T, 1e-3, cfg.seed, (gen.STREAM_GRAD,), dev)
    local = torch.zeros(T, dtype=torch.float32, device=dev)
    out = torch.empty(T, dtype=torch.int16, device=dev)
    legs = {"local_accumulate": (lambda: fp.local_accumulate(grad, local, accumulate=True), 10 * T),
            "local_finish": (lambda: fp.local_finish(grad, out, local, accumulate=True), 8 * T)}
    res = {"workload": cfg.name, "elements": T, "n_micro": cfg.n_micro}
    for name, (run, alg) in legs.items():
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = alg / (ms * 1e-3) / 1e9
        res[name] = {"us_per_call": round(ms * 1e3, 2), "alg_bytes": alg, "GBps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    res["per_step"] = (f"a no_sync step of {cfg.n_micro} micro-batches runs {cfg.n_micro - 1} local "
                       f"accumulations (the first without the fp32 read) and one finish per rank before "
                       f"the shard step")
    return res


def hybrid_bench(cfg, dev, reps: int, replicas: int = 2):
    """The hybrid-sharding reduce of the workload's unit with sharding factor
    F = N_d and W = replicas * F ranks (groups of F, e.g. one 8-GPU node per
    group): one micro-batch's fp_reduce_shard_hybrid over the W ranks' bf16
    rows of this rank's slice, against fp_reduce_shard over the same rows
    (the flat order)."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    from workloads import gen
    F = cfg.world
    W = replicas * F
    S = fp.Plan(cfg.shapes, F).shard if cfg.shapes is not None else cfg.units()[0] // F
    Sp = row_stride(S)
    rows = gen.torch_bf16_normal(W * Sp, 1e-3, cfg.seed, (gen.STREAM_GRAD,), dev).view(W, Sp)[:, :S]
    acc = torch.zeros(S, dtype=torch.float32, device=dev)
    legs = {"hybrid": lambda: fp.reduce_shard_hybrid(rows, acc, group=F, scale=1.0 / W),
            "flat_same_rows": lambda: fp.reduce_shard(rows, acc, scale=1.0 / W)}
    alg = (2 * W + 4) * S
    res = {"workload": cfg.name, "W": W, "F": F, "shard_elems": S, "alg_bytes": alg}
    for name, run in legs.items():
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = alg / (ms * 1e-3) / 1e9
        res[name] = {"us_per_call": round(ms * 1e3, 2), "GBps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def reshard_bench(cfg, dev, reps: int):
    """Resharding the workload's fp32 flat state (one of master / exp_avg /
    exp_avg_sq: T elements) from N_d to 2 N_d and to N_d / 2 ranks, every new
    rank's shard in one call: reads 4T, writes 4 N' S' bytes."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    from workloads import gen
    T = sum(cfg.units())
    N = cfg.world
    res = {"workload": cfg.name, "elements": T, "N_d": N, "dtype": "fp32"}
    for N2 in (2 * N, max(1, N // 2)):
        plan = fp.ReshardPlan(T, N, N2)
        S = plan.shard_old
        flat = torch.zeros(N * S, dtype=torch.float32, device=dev)
        flat[:T] = gen.torch_normal_f32(T, 0.02, cfg.seed, (gen.STREAM_MASTER,), dev)
        run = plan.resharder([flat[q * S:(q + 1) * S] for q in range(N)])
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        alg = 4 * T + 4 * N2 * plan.shard_new
        gbs = alg / (ms * 1e-3) / 1e9
        res[f"to_{N2}"] = {"us_per_call": round(ms * 1e3, 2), "alg_bytes": alg, "GBps": round(gbs, 1),
                           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del flat, run
        plan.close()
        torch.cuda.empty_cache()
    return res


COPY_REFERENCE_SHARD = 64 * 1024 * 1024   # 16 shards: 2 GiB read and 2 GiB written per copy


def copy_reference(fp, dev, reps: int = 20):
    """Measured plain-copy bandwidth (fp_unshard of 16 x 64M bf16 shards, 2 GiB each
    way: large enough that launch and drain cost under 1 % of a copy)."""
    import torch
    world, S = 16, COPY_REFERENCE_SHARD
    src = torch.ones(world * S, dtype=torch.int16, device=dev)
    full = torch.zeros(world * S, dtype=torch.int16, device=dev)
    shards = [src[q * S:(q + 1) * S] for q in range(world)]
    fp.unshard(shards, full)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fp.unshard(shards, full)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return round(4 * world * S / (ms * 1e-3) / 1e9, 1)


def copy_calibration(fp, dev, launches: int) -> int:
    """fp_unshard of 16 aligned shards of 8M bf16 elements: 256 MiB read and
    256 MiB written per launch, the reference for scaling HBM byte counters."""
    import torch
    world, S = 16, 8 * 1024 * 1024
    src = torch.ones(world * S, dtype=torch.int16, device=dev)
    full = torch.zeros(world * S, dtype=torch.int16, device=dev)
    shards = [src[q * S:(q + 1) * S] for q in range(world)]
    for _ in range(max(1, launches)):
        fp.unshard(shards, full)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "unshard_kernel", "launches": max(1, launches),
                      "read_bytes_per_launch": 2 * world * S, "write_bytes_per_launch": 2 * world * S}))
    return 0


def cpu_model_from_lscpu(text: str) -> str:
    """The model name in lscpu's output.  A name without a model number (a
    virtual machine's "AMD EPYC") gets lscpu's family / model / stepping and the
    hypervisor, which identify the part."""
    fields = {}
    for line in text.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    name = fields.get("Model name", "")
    if name and not any(c.isdigit() for c in name):
        ids = [f"{k.lower()} {fields[k]}" for k in ("CPU family", "Model", "Stepping") if fields.get(k)]
        if fields.get("Hypervisor vendor"):
            ids.append(f"{fields['Hypervisor vendor']} guest")
        if ids:
            name = f"{name} ({', '.join(ids)})"
    return name


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it, else /proc/cpuinfo's, else
    the machine type."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        name = cpu_model_from_lscpu(out)
        if name:
            return name
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(cfg, rank, budget_s: float):
    """The serial CPU oracle on a bounded sample of the workload, on one host core:
    whole shard steps (all micro-batches) of a shard of at most 2M elements with
    the workload's N_d and micro-batch count."""
    import numpy as np
    import oracle
    from workloads import gen
    world, n = cfg.world, cfg.n_micro
    S_full = -(-cfg.units()[0] // world)
    S = min(S_full, 2_000_000)
    micro = [[gen.bf16_normal(S, cfg.grad_sigma, cfg.seed, gen.STREAM_GRAD, 0, m, q) for q in range(world)]
             for m in range(n)]
    others = [gen.bf16_normal(S, cfg.master_sigma, cfg.seed, gen.STREAM_SHARD, 0, 0, q) for q in range(world)]
    master = gen.normal_f32(S, cfg.master_sigma, cfg.seed, gen.STREAM_MASTER)
    m_, v_, acc = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.float32)
    old = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(old)})
    try:
        oracle.lib()
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.shard_step(micro, acc, master, m_, v_, others, rank, hp=cfg.hp, step=reps + 1)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, old)
    B = step_bytes_per_elem(world, n)
    what = "the whole shard" if S == S_full else f"the first {S} elements of a {S_full}-element shard"
    if len(cfg.units()) > 1:
        what += f" of unit 0 (of {len(cfg.units())})"
    return {"value": round(S * reps * B / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "params_per_s": round(S * reps / dt, 1), "seconds": round(dt, 2),
            "host_cores_available": len(old), "cpu": cpu_model(),
            "sample": f"{reps} shard steps of {what} of the {cfg.name} workload (rank {rank}, N_d={world}, "
                      f"{n} micro-batch(es)) by the serial oracle: reduce, AdamW, bf16 cast, unshard"}


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ main
PATH_NAMES = {0: "one-pass", 1: "two-phase", 2: "fused-no-skip", 3: "fused-no-skip-split", 4: "speculative",
              5: "speculative-split", 6: "speculative-one-pass"}


def kernel_lines(kernels):
    return [{"name": nm, "avg_us": round(d * 1e3, 3), "launches_per_step": c, "alg_bytes": a,
             "alg_GBps": round(a / (d * 1e-3) / 1e9, 1)} for nm, _, d, a, c in kernels]


def summary(cfg, w, mode, r, B):
    """The figures of one timed run, for the `configs` and `modes` entries."""
    name, kernel_id, dur_ms, alg = r["dominant"]
    kgbs = alg / (dur_ms * 1e-3) / 1e9
    return {"mode": mode, "path": PATH_NAMES[w.path], "ms_per_step": round(r["step_ms"], 5),
            "GBps": round(r["gbs"], 2), "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
            "params_per_s": round(w.S / (r["step_ms"] * 1e-3), 1),
            "dominant_kernel": {"name": name, "avg_us": round(dur_ms * 1e3, 3), "alg_bytes": alg,
                                "alg_GBps": round(kgbs, 1), "frac": round(kgbs / HBM_PEAK_GBS, 4),
                                "traffic": load_traffic(cfg.name, kernel_id)}}


def side_config(name, K, W, timing, ev, dev):
    """A workload of the `configs` entry: its default (speculative) mode and the
    in-place exact skip, exactly K steps each."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    from workloads import CONFIGS
    cfg = CONFIGS[name]
    rank = cfg.ranks[0]
    B = step_bytes_per_elem(cfg.world, cfg.n_micro)
    w = make_workload(cfg, rank, dev, fp.FP_STEP_EXACT_SKIP, True)
    out = {"workload": name, "N_d": cfg.world, "rank": rank, "shard_elems": w.S, "units": len(cfg.units()),
           "n_micro": cfg.n_micro, "alg_bytes_per_elem": B, "buffer_sets": w.n_sets, "steps": K}
    r = measure(w, K, W, timing, ev, B)
    bad = w.flagged()
    if bad:
        raise RuntimeError(f"{name}: {bad}")
    out.update(summary(cfg, w, "speculative", r, B))
    out["kernels"] = kernel_lines(r["kernels"])
    out["timing"] = r["how"]
    out["spread"] = r["spread"]
    w.set_flags(fp.FP_STEP_EXACT_SKIP, False)
    r = measure(w, K, W, timing, ev, B)
    out["in_place_exact"] = summary(cfg, w, "exact", r, B)
    del w
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", choices=list(MODE_FLAGS), default="speculative",
                    help="speculative: exact overflow skip with separate output state (the fused pass, "
                         "then a restore kernel that acts only on overflow); exact: exact skip in place "
                         "(one-pass kernel when the shard fits the co-resident grid, else two kernels); "
                         "twophase: exact skip in place with two kernels; noskip: one pass, no gate")
    ap.add_argument("--timing", choices=("auto", "graph", "eager"), default="auto",
                    help="auto: eager launches with per-kernel events for steps of 0.2 ms and more, "
                         "HIP graph replays for shorter (launch-bound) steps")
    ap.add_argument("--eager", action="store_true", help="same as --timing eager")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other modes, the pack, layout and copy legs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (the `configs` entry of the default line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run fp_unshard (a plain copy of known size) for counter calibration")
    ap.add_argument("--dim0-only", action="store_true",
                    help="only time the per-parameter dim-0 layout's pack and unpack of the workload")
    ap.add_argument("--nosync-only", action="store_true",
                    help="only time the no_sync local accumulation kernels over the workload's unit")
    ap.add_argument("--hybrid-only", action="store_true",
                    help="only time the hybrid-sharding reduce (F = N_d, W = 2F) against the flat one")
    ap.add_argument("--reshard-only", action="store_true",
                    help="only time resharding the workload's fp32 flat state to 2 N_d and N_d / 2 ranks")
    ap.add_argument("--pack-only", action="store_true",
                    help="only time fp_pack of the workload's FlatParameter (fp32 tensors)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)
    timing = "eager" if args.eager else args.timing

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the N_d ranks of the shard "
              f"step are buffers on that GPU, and the library has no multi-GPU path.", file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        return 2

    import torch
    import __graft_entry__
    __graft_entry__._ensure_built()
    import sharded_flatparameter_pack_amd as fp
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        return copy_calibration(fp, dev, args.steps)
    cfg = CONFIGS[args.workload]
    if args.dim0_only:
        if cfg.shapes is None:
            print(f"{cfg.name} has no parameter shapes", file=sys.stderr)
            return 2
        print(json.dumps(shard0_bench(cfg, dev, max(1, args.steps))), flush=True)
        return 0
    if args.pack_only:
        if cfg.shapes is None:
            print(f"{cfg.name} has no tensor shapes", file=sys.stderr)
            return 2
        print(json.dumps(pack_bench(cfg, dev, max(1, args.steps))), flush=True)
        return 0
    if args.reshard_only:
        print(json.dumps(reshard_bench(cfg, dev, max(1, args.steps))), flush=True)
        return 0
    if args.hybrid_only:
        print(json.dumps(hybrid_bench(cfg, dev, max(1, args.steps))), flush=True)
        return 0
    if args.nosync_only:
        print(json.dumps(nosync_bench(cfg, dev, max(1, args.steps))), flush=True)
        return 0
    rank = cfg.ranks[0]
    world, n = cfg.world, cfg.n_micro
    B = step_bytes_per_elem(world, n)
    ev = HipEvents()
    K = args.steps

    w = make_workload(cfg, rank, dev, getattr(fp, MODE_FLAGS[args.mode]), args.mode in OUT_OF_PLACE_MODES)
    S = w.S
    r = measure(w, K, args.warmup, timing, ev, B)
    bad = w.flagged()
    if bad:
        print(bad, file=sys.stderr)
        return 1
    step_ms, gbs = r["step_ms"], r["gbs"]
    name, kernel_id, dur_ms, alg = r["dominant"]
    achieved = alg / (dur_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32/f64", "data": "synthetic",
        "config": {"workload": cfg.name, "N_d": world, "rank": rank, "shard_elems": S,
                   "units": len(cfg.units()), "n_micro": n, "mode": args.mode,
                   "path": PATH_NAMES[w.path], "alg_bytes_per_elem": B, "buffer_sets": w.n_sets},
        "params_per_s": round(S / (step_ms * 1e-3), 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "kernels": kernel_lines(r["kernels"]),
        "roofline": {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(cfg.name, kernel_id)},
        "timing": r["how"],
        "spread": r["spread"],
        "source_hash": kernel_source_hash(),
    }
    print(f"# main line done: {cfg.name} {args.mode} {step_ms:.4f} ms/step", file=sys.stderr, flush=True)
    if not args.no_extras:
        modes, seen = {}, {w.path: args.mode}
        for mode in MODE_FLAGS:
            if mode == args.mode:
                continue
            w.set_flags(getattr(fp, MODE_FLAGS[mode]), mode in OUT_OF_PLACE_MODES)
            if w.path in seen:
                modes[mode] = {"path": PATH_NAMES[w.path], "same_path_as": seen[w.path]}
                continue
            seen[w.path] = mode
            rm = measure(w, K, min(args.warmup, 20), timing, ev, B)
            modes[mode] = summary(cfg, w, mode, rm, B)
        result["modes"] = modes
    del w
    torch.cuda.empty_cache()
    if args.workload == DEFAULT_WORKLOAD and not args.no_configs:
        configs = {}
        for name2 in SIDE_WORKLOADS:
            configs[name2] = side_config(name2, K, args.warmup, timing, ev, dev)
            print(f"# config done: {name2}", file=sys.stderr, flush=True)
        result["configs"] = configs
    if not args.no_extras:
        copy_gbs = copy_reference(fp, dev)
        torch.cuda.empty_cache()
        result["copy_reference"] = {"GBps": copy_gbs, "what": "fp_unshard of 16 x 64M bf16 shards "
                                    "(2 GiB read + 2 GiB written): the plain-copy rate on this GPU",
                                    "value_over_copy": round(gbs / copy_gbs, 4)}
        if cfg.shapes is not None:
            result["pack"] = pack_bench(cfg, dev, 20)
            torch.cuda.empty_cache()
            result["dim0_layout"] = shard0_bench(cfg, dev, 20)
            torch.cuda.empty_cache()
            result["hybrid_reduce"] = hybrid_bench(cfg, dev, 20)
        torch.cuda.empty_cache()
        result["reshard"] = reshard_bench(cfg, dev, 10)
        if cfg.n_micro > 1:
            torch.cuda.empty_cache()
            result["no_sync"] = nosync_bench(cfg, dev, 10)
        print("# extras done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, rank, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
