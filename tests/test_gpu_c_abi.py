"""The library from C, through include/flatparam.h alone.

tests/c/step_abi.c (built into tests/c/libstep_abi.so by
__graft_entry__.build()) allocates device buffers with hipMalloc and runs two
micro-batches of one rank's shard step (8 ranks, an odd 1,000,003-element
shard) in the one-pass, two-phase and speculative forms, with and without an
overflow, comparing every element with the serial oracle on the same input
bytes ("Infra: Data Parallel", ZeRO-1 / ZeRO-2 paragraphs; "PyTorch FSDP"
section 3.5).  No Python or torch sits between the C caller and the library.
"""

import ctypes
import os

import pytest

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "libstep_abi.so")


@pytest.mark.gpu
def test_step_from_c_matches_the_oracle(capfd):
    if not os.path.exists(LIB):
        raise AssertionError(f"{LIB} is not built: run __graft_entry__.build() first")
    import torch
    torch.cuda.init()                       # the C caller runs on the current device, cuda:0
    lib = ctypes.CDLL(LIB)
    lib.step_abi_run.restype = ctypes.c_int
    print("step_abi_run: 6 cases, S = 1000003, N_d = 8, rank 3", flush=True)
    failed = lib.step_abi_run()
    out = capfd.readouterr().out
    print(out)
    assert failed != 100, "no GPU visible to the C caller"
    assert failed == 0, out
    cases = [line for line in out.splitlines() if " form=" in line]
    assert len(cases) == 6 and all(line.startswith("ok ") for line in cases), out
