"""Builds tests/c_abi_consumer: a plain C program (gcc, C11) that uses libtk through
include/tk.h alone and checks its results with the C oracle.  Linked against
bulk_fills_amd/libtk.so and oracle/liboracle.so, found next to the tree at run time."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
EXE = os.path.join(HERE, "c_abi_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           "-I", os.path.join(ROCM, "include"),
           "-o", tmp, os.path.join(HERE, "c_abi_consumer.c"),
           "-L", os.path.join(ROOT, "bulk_fills_amd"), "-ltk", "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../bulk_fills_amd:$ORIGIN/../oracle:" + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"gcc failed with status {res.returncode}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
