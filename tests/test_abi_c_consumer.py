"""The C ABI from a plain C99 program (tests/host/abi_consumer.c): include/solattn.h compiles
as C with -pedantic -Werror, the program links against libsolattn.so, and the host-side entry
points (argument checks, workspace sizing and layout, the argument errors every call returns
before it launches anything) behave as the header states.  No device is touched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_attention_tok_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_caller(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libsolattn.so")):
        pytest.skip("libsolattn.so not built")
    exe = tmp_path / "abi_consumer"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host", "abi_consumer.c"), "-L", PKG, "-lsolattn",
                    f"-Wl,-rpath,{PKG}", "-lm", "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    lines = res.stdout.strip().splitlines()
    assert lines[-1] == "0 failures", res.stdout
    assert len([x for x in lines if x.startswith("ok ")]) == 21, res.stdout
