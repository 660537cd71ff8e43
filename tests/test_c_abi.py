"""The C ABI from plain C: the header parses as strict C99 (CPU), and a C
program (tests/c_abi/abi_check.c, built by the build step) drives the
library with closed-form checks (GPU)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "abi_check")


def test_header_is_strict_c99(tmp_path):
    src = tmp_path / "use_header.c"
    src.write_text('#include "cp_attn.h"\nint f(void) { return (int)CP_OK + cp_abi_version(); }\n')
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.gpu
def test_c_program_drives_the_abi():
    assert os.path.exists(BIN), "tests/c_abi/abi_check is built by __graft_entry__.build()"
    print("running tests/c_abi/abi_check", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all C ABI checks passed" in r.stdout
