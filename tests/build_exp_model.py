"""Builds tests/libexp_f64_model.so: the host model of the f64 exponential's logarithm
(tests/exp_f64_model.c, library form), for the GPU test that the fill computes exactly the
modelled operations.  Plain gcc, no contraction beyond the model's explicit fma calls."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libexp_f64_model.so")


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-DTK_MODEL_LIB",
           "-I", os.path.join(ROOT, "bulk_fills_amd", "csrc"), "-o", tmp, os.path.join(HERE, "exp_f64_model.c"), "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"gcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
