"""Build the plain-C consumer of the C ABI (abi_example.c) next to this file.

It links libdtcoll.so (build the library first) and, as test
infrastructure, the CPU oracle it compares against.  gcc only: the program
is host code that calls the HIP runtime and the library.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "collective_communication_primitives_amd")
SOURCE = os.path.join(HERE, "abi_example.c")
BINARY = os.path.join(HERE, "abi_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           SOURCE, os.path.join(ROOT, "oracle", "oracle.c"), "-o", BINARY + ".tmp",
           "-L", PKG, "-ldtcoll", "-Wl,-rpath,$ORIGIN/../../collective_communication_primitives_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building {SOURCE} failed:\n{res.stderr}")
    os.replace(BINARY + ".tmp", BINARY)
    return BINARY


if __name__ == "__main__":
    print(build())
