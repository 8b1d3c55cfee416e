"""The C ABI from a C caller: tests/c/abi_consumer.c compiles against include/fa.h as
strict C11, links against the built libfa.so and runs the host-side entry points
(status strings, version, workspace sizing, argument validation). No GPU needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "exact_attention_48_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_consumer_compiles_links_and_runs(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libfa.so")):
        pytest.fail("libfa.so is not built (python -m exact_attention_48_amd.build)")
    exe = str(tmp_path / "abi_consumer")
    cmd = ["gcc", "-std=c11", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-L", LIBDIR, "-lfa", f"-Wl,-rpath,{LIBDIR}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "abi consumer ok" in r.stdout, r.stdout + r.stderr
