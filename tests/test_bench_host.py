"""Host-side checks of bench.py's bookkeeping (no GPU needed).

* every step mode of the default line's mode loop can be applied to both
  workload classes (single unit and bucketed): set_flags takes the
  out-of-place argument and picks the path the library would take;
* the algorithmic bytes of a step's kernels add up to B(N, n) bytes per
  shard element on every path, so the roofline entry and the step figure
  count the same bytes;
* the speculative modes alternate input and output state from step to step
  on each buffer set;
* --gpus above 1 is refused with a message;
* the CPU baseline names the host CPU: lscpu's model name, with family /
  model / stepping where the name carries no model number;
* the roofline's traffic comes only from a counter summary taken on the
  current kernel sources, and every timed path's dominant kernel has one.
"""

import types

import pytest

import bench
import sharded_flatparameter_pack_amd as fp
from workloads import CONFIGS


class _StubStep:
    def __init__(self, *args, flags=0, out=None, **kw):
        self.flags, self.out = flags, out

    def path(self):
        if self.flags & fp.FP_STEP_NO_SKIP:
            return fp.FP_PATH_NO_SKIP_SPLIT
        if self.out is not None:
            return fp.FP_PATH_SPECULATIVE_SPLIT
        return fp.FP_PATH_TWO_PHASE


def _single_unit(monkeypatch, n_sets=2):
    import torch
    monkeypatch.setattr(fp, "ShardStep", _StubStep)
    cfg = CONFIGS["c4_layer_d12288_nd8"]
    w = bench.SingleUnit.__new__(bench.SingleUnit)
    w.cfg, w.rank, w.world, w.n_micro, w.dev = cfg, 0, cfg.world, 1, "cpu"
    w.S, w.n_sets = 64, n_sets
    w.sets = [dict(grads=None, shards=None, acc=None, full=None, found_inf=None, workspace=None,
                   master=torch.zeros(64), exp_avg=torch.zeros(64), exp_avg_sq=torch.zeros(64))
              for _ in range(n_sets)]
    return w


def _bucketed(n_sets=2):
    import torch
    cfg = CONFIGS["c3_611m_buckets_nd16"]
    w = bench.Bucketed.__new__(bench.Bucketed)
    w.cfg, w.rank, w.world, w.n_micro, w.dev = cfg, 0, cfg.world, cfg.n_micro, "cpu"
    w.S, w.n_sets = 64, n_sets
    def step_path(*args, flags=0, out=None, **kw):
        if flags & fp.FP_STEP_NO_SKIP:
            return fp.FP_PATH_NO_SKIP_SPLIT
        return fp.FP_PATH_SPECULATIVE_SPLIT if out is not None else fp.FP_PATH_TWO_PHASE

    plan = types.SimpleNamespace(partition=64, step_path=step_path)
    w.sets = [dict(plans=[plan] * cfg.n_micro, master=torch.zeros(64), exp_avg=torch.zeros(64),
                   exp_avg_sq=torch.zeros(64), acc=None, found_inf=None) for _ in range(n_sets)]
    return w


@pytest.mark.parametrize("kind", ["single", "bucketed"])
def test_every_mode_applies_to_both_workload_classes(monkeypatch, kind):
    w = _single_unit(monkeypatch) if kind == "single" else _bucketed()
    for mode, flag_name in bench.MODE_FLAGS.items():
        w.set_flags(getattr(fp, flag_name), mode in bench.OUT_OF_PLACE_MODES)
        if mode == "speculative":
            assert w.path in (fp.FP_PATH_SPECULATIVE, fp.FP_PATH_SPECULATIVE_SPLIT)
        elif mode == "noskip":
            assert w.path in (fp.FP_PATH_NO_SKIP, fp.FP_PATH_NO_SKIP_SPLIT)
        else:
            assert w.path == fp.FP_PATH_TWO_PHASE


@pytest.mark.parametrize("kind", ["single", "bucketed"])
def test_speculative_steps_alternate_state(monkeypatch, kind):
    w = _single_unit(monkeypatch) if kind == "single" else _bucketed()
    w.set_flags(fp.FP_STEP_EXACT_SKIP, True)
    n = w.n_sets
    for i in range(4 * n):
        state_in, state_out = w.state_io(i)
        s = w.sets[i % n]
        even = (i // n) % 2 == 0
        assert (state_in[0] is s["master"]) == even and (state_out[0] is s["master"]) == (not even)
        assert all(a is not b for a, b in zip(state_in, state_out))
    w.set_flags(fp.FP_STEP_EXACT_SKIP, False)
    assert w.state_io(3)[1] is None


def _ev(durations):
    out, t = [0.0], 0.0
    for d in durations:
        t += d
        out.append(t)
    return out


@pytest.mark.parametrize("path", [fp.FP_PATH_ONE_PASS, fp.FP_PATH_TWO_PHASE, fp.FP_PATH_NO_SKIP,
                                  fp.FP_PATH_NO_SKIP_SPLIT, fp.FP_PATH_SPECULATIVE,
                                  fp.FP_PATH_SPECULATIVE_SPLIT])
def test_single_unit_kernel_bytes_add_up(monkeypatch, path):
    w = _single_unit(monkeypatch)
    w.path = path
    ks = w.kernels(_ev([1.0, 0.5]))
    B = bench.step_bytes_per_elem(w.world, 1)
    assert sum(alg * launches for _, _, _, alg, launches in ks) == w.S * B
    assert ks[0][2] == 1.0


@pytest.mark.parametrize("path", [fp.FP_PATH_TWO_PHASE, fp.FP_PATH_NO_SKIP, fp.FP_PATH_NO_SKIP_SPLIT,
                                  fp.FP_PATH_SPECULATIVE, fp.FP_PATH_SPECULATIVE_SPLIT])
def test_bucketed_kernel_bytes_add_up(path):
    w = _bucketed()
    w.set_flags(0, path in (fp.FP_PATH_SPECULATIVE, fp.FP_PATH_SPECULATIVE_SPLIT))
    w.path = path
    n = w.n_micro
    ks = w.kernels(_ev([0.25] * (n - 1) + [0.6, 0.2]))
    B = bench.step_bytes_per_elem(w.world, n)
    assert sum(alg * launches for _, _, _, alg, launches in ks) == w.S * B


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


_LSCPU_VM = """Architecture:                            x86_64
Vendor ID:                               AuthenticAMD
Model name:                              AMD EPYC
CPU family:                              26
Model:                                   2
Thread(s) per core:                      1
Stepping:                                1
Hypervisor vendor:                       KVM
"""

_LSCPU_HOST = """Architecture:            x86_64
Model name:              Intel(R) Xeon(R) Processor @ 2.70GHz
CPU family:              6
Model:                   143
Stepping:                8
"""


def test_cpu_model_names_the_part():
    assert bench.cpu_model_from_lscpu(_LSCPU_VM) == "AMD EPYC (cpu family 26, model 2, stepping 1, KVM guest)"
    assert bench.cpu_model_from_lscpu(_LSCPU_HOST) == "Intel(R) Xeon(R) Processor @ 2.70GHz"
    assert bench.cpu_model_from_lscpu("") == ""


def test_traffic_comes_only_from_counters_of_the_current_sources(tmp_path, monkeypatch):
    import json
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "f" * 16)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / "counters_k_w.json"
    assert bench.load_traffic("w", "k") is None                      # no summary
    f.write_text(json.dumps({"source_hash": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("w", "k") is None                      # taken on other sources
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("w", "k") == 123


def test_every_timed_kernel_has_a_counter_summary():
    """The default line's and the configs' dominant kernels each have a committed
    counter summary (profiles/counters_<kernel>_<workload>.json) with the
    calibrated HBM bytes and the commands that produced them."""
    import json
    import os
    names = [("step_phase1_fused", "c4_layer_d12288_nd8"), ("unshard", "c4_layer_d12288_nd8"),
             ("step_phase1_fused", "c5_ragged10k_nd64"), ("unshard", "c5_ragged10k_nd64"),
             ("units_reduce", "c3_611m_buckets_nd16"), ("units_phase1_fused", "c3_611m_buckets_nd16"),
             ("units_copy", "c3_611m_buckets_nd16"), ("step_coop", "c2_layer_d1024_nd8")]
    for kernel, workload in names:
        path = os.path.join(bench.ROOT, "profiles", f"counters_{kernel}_{workload}.json")
        with open(path) as f:
            d = json.load(f)
        assert d["hbm_bytes_per_launch"] > 0 and d["algorithmic_bytes_per_launch"] > 0, path
        assert set(d["commands"]) == {"FETCH_SIZE", "WRITE_SIZE", "calibration"}, path
        assert 0.9 < d["traffic_over_algorithmic"] < 1.2, path
