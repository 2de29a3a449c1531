"""The C ABI used from plain C: include/tk.h compiles as C11, and a C program
(tests/c_abi_consumer.c, built by build()) fills device buffers through it and matches the
C oracle (u32 at a misaligned address, u64 below 1000, the f64 ziggurat, choice through an
alias table), with the documented status for refused calls."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
EXE = os.path.join(HERE, "c_abi_consumer")


def test_header_is_c11():
    src = '#include "tk.h"\nint main(void) { return tk_status_string(TK_OK) ? 0 : 1; }\n'
    res = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                          "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                          "-isystem", "/opt/rocm/include", "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


@pytest.mark.gpu
def test_c_program_matches_the_oracle():
    if not os.path.exists(EXE):
        import build_c_consumer
        build_c_consumer.build()
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c_abi_consumer: ok" in res.stdout
