"""Compile step_abi.c, a C consumer of include/flatparam.h (test infrastructure),
into libstep_abi.so.

gcc in C11: the header must parse as C.  The library links the HIP library
(libflatparam.so), the CPU oracle (liboracle.so, to check results) and the HIP
runtime, with run paths relative to its own location.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "step_abi.c")
LIB = os.path.join(HERE, "libstep_abi.so")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "sharded_flatparameter_pack_amd")
    orc = os.path.join(ROOT, "oracle")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC,
           "-o", tmp, f"-L{pkg}", "-lflatparam", f"-L{orc}", "-loracle", f"-L{ROCM}/lib", "-lamdhip64",
           "-lm", "-Wl,-rpath,$ORIGIN/../../sharded_flatparameter_pack_amd:$ORIGIN/../../oracle:" + f"{ROCM}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
