"""Host-side logic of bench.py (no GPU): the algorithmic bytes behind the
roofline figure, the source hash that ties the committed counter profiles to
the kernels, the warm-up rule and the one-GPU refusal."""
import os
import subprocess
import sys

import pytest

import bench
from bit_adamw_update_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_per_parameter():
    w = inputs.gpt_2_7b()
    n = w.numel
    # param 4R+4W, grad 2R, two 4-bit code buffers 0.5R+0.5W each, four
    # FP32 scales per 128 elements (every tensor here is a multiple of 128)
    assert bench.alg_bytes(w, "zip_sr") == n * 12.125
    assert bench.alg_bytes(w, "ze_eden") == n * 12.125
    assert bench.alg_bytes(w, "block8") == n * 14.125
    assert bench.alg_bytes(w, "fp32") == n * 26
    q = inputs.WORKLOADS["qwen3-0.6b-factored"]()
    per = bench.alg_bytes(q, "factored") / q.numel
    assert 11.0 < per < 11.2   # matrices: one packed moment plus R/C; vectors: both moments


def test_algorithmic_bytes_skip_tensors_without_elements():
    w = inputs.custom([(0,), (0, 5), (256,)])
    assert bench.alg_bytes(w, "factored") == bench.alg_bytes(inputs.custom([(256,)]), "factored")


def _write(path, text):
    with open(path, "w") as f:
        f.write(text)


def test_kernel_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    from bit_adamw_update_amd import profiling
    a, b = tmp_path / "a.hip", tmp_path / "b.hip"
    _write(a, "int f(int x) {\n    return x + 1;  // one more\n}\n")
    monkeypatch.setattr(profiling, "KERNEL_SRC", [str(a)])
    h0 = bench.kernel_hash()
    _write(a, "// a new comment line\nint f(int x)   {\n\n    return x + 1;\n}\n")
    assert bench.kernel_hash() == h0
    _write(a, "int f(int x) {\n    return x + 2;\n}\n")
    assert bench.kernel_hash() != h0
    _write(b, "int g();\n")
    monkeypatch.setattr(profiling, "KERNEL_SRC", [str(a), str(b)])
    assert bench.kernel_hash() != h0


def test_traffic_is_read_only_for_the_current_kernels(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    assert bench.read_traffic("gpt-2.7b", "zip_sr") is None          # no summary
    f = tmp_path / "profiles" / "k_fused_step_gpt-2.7b_zip_sr_counters.txt"
    _write(f, f"# header\nkernel_source_sha256_16: {bench.kernel_hash()}\ntraffic_bytes_per_launch: 123.0\n")
    assert bench.read_traffic("gpt-2.7b", "zip_sr") == 123.0
    _write(f, "kernel_source_sha256_16: 0000000000000000\ntraffic_bytes_per_launch: 123.0\n")
    assert bench.read_traffic("gpt-2.7b", "zip_sr") is None          # another kernel source
    g = tmp_path / "profiles" / "k_step8_gpt-2.7b_block8_counters.txt"
    _write(g, f"kernel_source_sha256_16: {bench.kernel_hash()}\ntraffic_bytes_per_launch: 7.5\n")
    assert bench.read_traffic("gpt-2.7b", "block8") == 7.5            # the 8-bit kernel's own file


@pytest.mark.parametrize("warmup", [0, 3])
def test_warm_up_runs_w_steps_then_until_the_minimum_time(warmup, monkeypatch):
    import time
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(bench, "WARMUP_MIN_S", 0.05)
    calls = []

    def one():
        calls.append(1)
        time.sleep(0.002)

    done = bench.warm_up(one, warmup)
    assert done == len(calls) >= warmup
    assert done * 0.002 >= 0.05 * 0.9
    assert done <= bench.WARMUP_CAP


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
