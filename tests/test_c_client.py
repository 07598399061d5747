"""include/ga.h is a plain C header and libga.so a plain C library: a C99
client (tests/c_abi_client.c) compiles with strict warnings, links against
the library and runs its host-only checks (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

import gated_activation_amd as ga

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_client_builds_links_and_runs(tmp_path):
    lib_dir = os.path.dirname(ga.library_path)
    exe = tmp_path / "c_abi_client"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_client.c"),
           "-o", str(exe), "-L", lib_dir, "-lga", "-lm", f"-Wl,-rpath,{lib_dir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout + res.stderr
