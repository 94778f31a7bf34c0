"""Compile the C boundary check (c_abi_check.c) with gcc: a host program that
links the HIP library (gqa_mqa_kv_amd/_lib/libgqa_decode.so), the HIP runtime
and the C oracle (oracle/_build/liboracle.so), into tests/c_abi/_build/.
Run by __graft_entry__.build() after the library and the oracle are built."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "c_abi_check.c")
OUT = os.path.join(HERE, "_build", "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = OUT) -> list:
    lib_dir = os.path.join(ROOT, "gqa_mqa_kv_amd", "_lib")
    oracle_dir = os.path.join(ROOT, "oracle", "_build")
    rel = lambda p: os.path.relpath(p, os.path.dirname(out))
    rpath = ":".join(["$ORIGIN/" + rel(lib_dir), "$ORIGIN/" + rel(oracle_dir), os.path.join(ROCM, "lib")])
    # __HIP_PLATFORM_AMD__ selects the AMD runtime API in the HIP headers
    # when they are read by a compiler other than hipcc
    return ["gcc", "-std=c11", "-pthread", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SOURCE, "-o", out,
            "-L", lib_dir, "-lgqa_decode", "-L", oracle_dir, "-loracle", "-L", os.path.join(ROCM, "lib"),
            "-lamdhip64", "-lm", "-pthread", "-Wl,-rpath," + rpath]


def build(out: str = OUT) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(command(tmp), check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
