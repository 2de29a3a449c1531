"""Builds libtk.so (the HIP library behind include/tk.h) for gfx950 with hipcc.

Flags:
  --offload-arch=gfx950           MI355X only
  -ffp-contract=off               no fused multiply-add where the source has two
                                  operations (the ziggurat and the uniform transforms
                                  must round exactly like a plain CPU evaluation)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  no packed fp32 instructions
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtk.so")
SOURCES = ["tk_runtime.hip", "tk_fills.hip", "tk_ziggurat.hip", "tk_choice.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out=LIB):
    return [
        HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # host pass does not know the device feature
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
