"""The C ABI from a plain C11 program (no GPU, no Python in the loop): the
header compiles as C with warnings as errors, the program links against
libq4adamw.so and its host-only calls behave as the header states."""
import os
import shutil
import subprocess

import pytest

from bit_adamw_update_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_c_client_builds_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(build.LIB_PATH):
        pytest.fail(f"{build.LIB_PATH} is not built")
    exe = tmp_path / "abi_c_client"
    libdir = os.path.dirname(build.LIB_PATH)
    rocm = "/opt/rocm/lib"
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "abi_c_client.c"), "-o", str(exe), f"-L{libdir}", "-lq4adamw",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath-link,{rocm}", f"-Wl,-rpath,{rocm}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
