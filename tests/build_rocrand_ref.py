"""Builds tests/librocrand_ref.so: rocRAND's Philox4x32-10 engine (its installed header, host
code) behind one C function, the independent reference for the oracle's Philox words.
Skipped, with a message, where rocRAND's headers are not installed."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "librocrand_ref.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HEADER = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


def build():
    if not os.path.exists(HEADER):
        print(f"build_rocrand_ref: {HEADER} not found; the rocRAND pin will be skipped", file=sys.stderr)
        return None
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-o", tmp, os.path.join(HERE, "rocrand_ref.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
