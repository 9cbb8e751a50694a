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


def _hash32(x: int) -> int:
    x &= 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def _unit(h, scale):
    import numpy as np
    return (np.float32(h >> 8) * np.float32(1.0 / 16777216.0) - np.float32(0.5)) * np.float32(scale)


@pytest.mark.gpu
def test_c_gpu_client_matches_the_oracle(tmp_path):
    """abi_c_gpu_client.c: init + three ZIP-SR steps through the C ABI on its
    own hipMalloc buffers and the null stream; codes and scales bit for bit
    and weights within 1e-6 of the oracle stepped on the same bytes."""
    import numpy as np

    from oracle import oracle as O
    from tests import parity
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_c_gpu_client"
    libdir = os.path.dirname(build.LIB_PATH)
    rocm = "/opt/rocm"
    cmd = [cc, "-std=c11", "-O2", "-ffp-contract=off", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", f"{rocm}/include", os.path.join(HERE, "abi_c_gpu_client.c"),
           "-o", str(exe), f"-L{libdir}", "-lq4adamw", f"-L{rocm}/lib", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out_path = tmp_path / "state.bin"
    run = subprocess.run([str(exe), str(out_path)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr

    n, nb, nc = 1000, (1000 + 127) // 128, 500
    raw = open(out_path, "rb").read()
    assert len(raw) == 4 * n + nc + 4 * nb + nc + 4 * nb
    p_gpu = np.frombuffer(raw, np.float32, n, 0)
    o = 4 * n
    mc = np.frombuffer(raw, np.uint8, nc, o); o += nc
    ms = np.frombuffer(raw, np.uint32, nb, o); o += 4 * nb
    vc = np.frombuffer(raw, np.uint8, nc, o); o += nc
    vs = np.frombuffer(raw, np.uint32, nb, o)

    param = np.array([_unit(_hash32(i), 0.04) for i in range(n)], np.float32)
    st = O.TensorState(parity.oracle_config("zip_sr"), (n,), 3, 0)
    for s in range(3):
        g = np.array([_unit(_hash32(i + 7919 * (s + 1)), 2e-3) for i in range(n)], np.float32)
        gb = (g.view(np.uint32) >> 16).astype(np.uint16)
        st.step(O.HParams(step=s + 1, seed=5), param, gb)
    assert np.array_equal(mc, st.m_codes) and np.array_equal(vc, st.v_codes)
    assert np.array_equal(ms, st.m_scales.view(np.uint32)) and np.array_equal(vs, st.v_scales.view(np.uint32))
    scale = np.maximum(np.abs(param), np.sqrt(np.mean(param.astype(np.float64) ** 2)))
    assert (np.abs(p_gpu - param) / scale).max() <= parity.W_TOL
