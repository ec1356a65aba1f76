"""The ABI from plain C: the public headers are C99, and a C program with no
Python or torch in its process drives every kernel family through
pa_decode_plan / pa_decode_ex and checks the results against the oracle, then
the checked mode (PA_CHECK=1 / pa_config.check): bad inputs are rejected with
PA_ERR_DEVICE_CHECK before any attention kernel runs and pa_get_device_error
reports them once (tests/c_abi/decode_from_c.c, built by the package build
step)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "decode_from_c")


def test_headers_are_c99():
    src = "".join(f'#include "{h}"\n' for h in sorted(os.listdir(os.path.join(ROOT, "include")))
                  if h.endswith(".h")) + "int main(void) { return 0; }\n"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-fsyntax-only", "-I", os.path.join(ROOT, "include"), "-x", "c", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.gpu
def test_decode_from_plain_c():
    print("case: plain-C driver of the decode ABI", flush=True)
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(": max rel err") == 7 and "FAIL" not in r.stdout
    assert "waves 2:" in r.stdout and "waves 4:" in r.stdout
    # checked mode: rejected before any attention kernel, reported once
    assert r.stdout.count(": ok") == 4
