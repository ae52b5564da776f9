"""Throughput of one rank's shard step (reduce + AdamW + bf16 cast + unshard).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode exact|noskip]

A step is the whole per-step hot path for rank r's shard of one unit: the
fixed-order reduce of the N_d ranks' bf16 gradients (last micro-batch),
the AdamW update of the fp32 master / moments with the overflow gate, the
bf16 cast of the own shard into the full buffer and the copy of the other
N_d - 1 shards into it (fp_shard_step).  Pack and views are one-time set-up
per unit and are not part of a step.

All inputs are synthetic and resident in HBM before timing starts.  The
step rotates over enough buffer sets (>= 1.5 GB) that no step finds its
data in the 256 MB Infinity Cache left behind by the previous ones.

Output: one JSON line.  `value` is algorithmic GB/s of the whole step,
B = 2*N*n + 8*(n-1) + 24 + 2 + 4*(N-1) bytes per shard element; `roofline`
times the dominant kernel with HIP events recorded around it on the
library's stream inside the timed region; `cpu_baseline` times the serial
CPU oracle on the same workload on one host core.
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
                  "sharded_flatparameter_pack_amd/csrc/fp_device.h",
                  "sharded_flatparameter_pack_amd/csrc/fp_internal.h"]


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

    def __init__(self):
        self.L = C.CDLL("libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.L.hipEventSynchronize.argtypes = [C.c_void_p]
        self.L.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = C.c_void_p()
        if self.L.hipEventCreate(C.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        if self.L.hipEventSynchronize(C.c_void_p(b)) != 0 or \
                self.L.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.L.hipEventDestroy(C.c_void_p(e))


def make_sets(cfg, rank, n_sets, dev):
    """n_sets independent buffer sets of one rank's shard step, all on the GPU."""
    import torch
    import sharded_flatparameter_pack_amd as fp
    from workloads import gen
    world = cfg.world
    T = cfg.units()[0]
    S = -(-T // world)
    sets = []
    for k in range(n_sets):
        key = lambda stream, q=0: (stream, k, 0, q)  # noqa: E731
        grads = gen.torch_bf16_normal(world * S, cfg.grad_sigma, cfg.seed, key(gen.STREAM_GRAD), dev)
        others = gen.torch_bf16_normal(world * S, cfg.master_sigma, cfg.seed, key(gen.STREAM_SHARD), dev)
        sets.append(dict(
            grads=grads.view(world, S),
            shards=[None if q == rank else others[q * S:(q + 1) * S] for q in range(world)],
            master=gen.torch_normal_f32(S, cfg.master_sigma, cfg.seed, key(gen.STREAM_MASTER), dev),
            exp_avg=torch.zeros(S, dtype=torch.float32, device=dev),
            exp_avg_sq=torch.zeros(S, dtype=torch.float32, device=dev),
            acc=torch.zeros(S, dtype=torch.float32, device=dev),
            full=torch.zeros(world * S, dtype=torch.int16, device=dev),
            found_inf=torch.zeros(1, dtype=torch.int32, device=dev),
            workspace=fp.new_workspace(dev, S)))
    return S, sets


def cpu_baseline(cfg, rank, budget_s: float):
    """The serial CPU oracle on the same workload, on one host core."""
    import numpy as np
    import oracle
    from workloads import gen
    world = cfg.world
    S = -(-cfg.units()[0] // world)
    grads = [gen.bf16_normal(S, cfg.grad_sigma, cfg.seed, gen.STREAM_GRAD, 0, 0, q) for q in range(world)]
    others = [gen.bf16_normal(S, cfg.master_sigma, cfg.seed, gen.STREAM_SHARD, 0, 0, q) for q in range(world)]
    master = gen.normal_f32(S, cfg.master_sigma, cfg.seed, gen.STREAM_MASTER)
    m, v, acc = np.zeros(S, np.float32), np.zeros(S, np.float32), np.zeros(S, np.float32)
    old = os.sched_getaffinity(0)
    core = min(old)
    os.sched_setaffinity(0, {core})
    try:
        oracle.lib()
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.shard_step([grads], acc, master, m, v, others, rank, hp=cfg.hp, step=reps + 1)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, old)
    B = step_bytes_per_elem(world, 1)
    return {"value": round(S * reps * B / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "params_per_s": round(S * reps / dt, 1), "seconds": round(dt, 2),
            "host_cores_available": len(old), "cpu": platform.processor() or platform.machine(),
            "sample": f"{reps} whole shard steps of the {cfg.name} workload (rank {rank}, S={S}, "
                      f"N_d={world}) by the serial oracle: reduce, AdamW, bf16 cast, unshard"}


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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="c2_layer_d1024_nd8")
    ap.add_argument("--mode", choices=["exact", "twophase", "noskip"], default="exact",
                    help="exact: exact overflow skip (one-pass cooperative kernel when the shard "
                         "fits); twophase: exact skip with two kernels; noskip: one pass, no gate")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python with per-kernel events (launch-bound for "
                         "small shards) instead of replaying a captured HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run fp_unshard (a plain copy of known size) for counter calibration")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the N_d ranks of the shard "
              f"step are buffers on that GPU; there is no multi-GPU path in this build.", file=sys.stderr)
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
    if cfg.shapes is None or cfg.n_micro != 1:
        print("bench.py times single-unit, single-micro-batch workloads", file=sys.stderr)
        return 2
    rank = cfg.ranks[0]
    world = cfg.world
    B = step_bytes_per_elem(world, 1)
    T = cfg.units()[0]
    S = -(-T // world)
    n_sets = max(2, math.ceil(ROTATE_BYTES / (S * (2 * world + 16 + 2 * (world - 1) + 2 * world))))
    S, sets = make_sets(cfg, rank, n_sets, dev)
    flags = {"exact": fp.FP_STEP_EXACT_SKIP, "twophase": fp.FP_STEP_NO_COOP,
             "noskip": fp.FP_STEP_NO_SKIP}[args.mode]
    hp = cfg.hp
    ev = HipEvents()
    K, W = args.steps, args.warmup

    calls = [fp.ShardStep(s["grads"], s["acc"], s["master"], s["exp_avg"], s["exp_avg_sq"],
                          s["shards"], s["full"], rank, scale=1.0 / world, lr=hp.lr, beta1=hp.beta1,
                          beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay,
                          found_inf=s["found_inf"], workspace=s["workspace"], flags=flags)
             for s in sets]

    def step(i, profile=None):
        calls[i % n_sets](i // n_sets + 1, profile)

    def eager_pass(first, count):
        evs = [[ev.create() for _ in range(3)] for _ in range(count)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(count):
            step(first + k, evs[k])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        k1 = [ev.elapsed_ms(e[0], e[1]) for e in evs]
        k2 = [ev.elapsed_ms(e[1], e[2]) for e in evs]
        for e in evs:
            for x in e:
                ev.destroy(x)
        return dt, sum(k1) / count, sum(k2) / count

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    if args.eager:
        elapsed, k1_ms, k2_ms = eager_pass(W, K)
        timing = "eager launches from Python; kernel times from hipEvents recorded by the library " \
                 "around its kernels"
    else:
        # One step per buffer set captured into a graph; replays run the steps
        # back to back on torch's current stream, timed by events on it.
        reps = max(1, -(-K // n_sets))
        K = reps * n_sets
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(n_sets):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_sets):
                step(i)
        for _ in range(max(1, W // n_sets)):
            graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        span_ms = e0.elapsed_time(e1)
        # per-kernel split of the step from a short eager pass with events
        _, k1_ms, k2_ms = eager_pass(W + K, min(K, 200))
        timing = "HIP graph of one step per buffer set, replayed; span timed by hipEvents on the " \
                 "replay stream; per-kernel split from library-recorded hipEvents in an eager pass"
    if any(int(s["found_inf"].item()) for s in sets):
        print("unexpected overflow flag in a finite workload", file=sys.stderr)
        return 1
    if any(fp.workspace_timeouts(s["workspace"]) for s in sets):
        print("grid barrier wait gave up", file=sys.stderr)
        return 1
    path = calls[0].path()
    step_ms = (span_ms / K) if not args.eager else (k1_ms + k2_ms)
    ms_step = elapsed * 1e3 / K
    gbs = S * B * K / elapsed / 1e9
    if path in (fp.FP_PATH_NO_SKIP, fp.FP_PATH_ONE_PASS):
        # one kernel per step: its average duration is the step's (graph span / steps)
        nm = "step_phase1_kernel<true>" if path == fp.FP_PATH_NO_SKIP else "step_coop_kernel"
        kid = "step_phase1_fused" if path == fp.FP_PATH_NO_SKIP else "step_coop"
        kernels = [(nm, kid, step_ms, S * B)]
    else:
        frac1 = k1_ms / (k1_ms + k2_ms)
        kernels = [("step_phase1_kernel<false>", "step_phase1", step_ms * frac1,
                    S * (2 * world + 4 * (world - 1))),
                   ("adamw_kernel", "adamw", step_ms * (1 - frac1), S * 26)]
    name, kernel_id, dur_ms, alg = max(kernels, key=lambda x: x[2])
    achieved = alg / (dur_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32/f64", "data": "synthetic",
        "config": {"workload": cfg.name, "N_d": world, "rank": rank, "shard_elems": S,
                   "unit_elems": T, "n_micro": 1, "mode": args.mode,
                   "alg_bytes_per_elem": B, "buffer_sets": n_sets,
                   "path": {fp.FP_PATH_ONE_PASS: "one-pass", fp.FP_PATH_TWO_PHASE: "two-phase",
                            fp.FP_PATH_NO_SKIP: "fused-no-skip"}[path]},
        "params_per_s": round(S * K / elapsed, 1),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "kernels": [{"name": n, "avg_us": round(d * 1e3, 3), "alg_bytes": a,
                     "alg_GBps": round(a / (d * 1e-3) / 1e9, 1)} for n, _, d, a in kernels],
        "roofline": {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(cfg.name, kernel_id)},
        "timing": timing,
        "eager_kernel_us": [round(k1_ms * 1e3, 3), round(k2_ms * 1e3, 3)],
        "source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, rank, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
