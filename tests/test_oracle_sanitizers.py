"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C is built with ``-fsanitize=address,undefined`` (gcc, host code
only) and every oracle pin runs against that build in a child process: no
out-of-bounds access, use after free, signed overflow, bad shift or other
undefined behaviour may show.  Two controls plant such a mistake in a copy of
the oracle and check that the sanitized run reports it, so a silent run means
a clean oracle, not a sanitizer that never looked.
"""
import glob
import os
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_decode_pins.py", "tests/test_oracle_pins.py", "tests/test_oracle_nonfinite.py"]
SAN_FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _build(tmp, name, src):
    c, so = os.path.join(tmp, f"{name}.c"), os.path.join(tmp, f"{name}.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", *SAN_FLAGS, "-o", so, c, "-lm"])
    return so


def _run(so, tmp, tag, select=None):
    """Runs the pins against `so` with the sanitizer runtime preloaded;
    returns (exit code, the sanitizers' reports)."""
    logs = os.path.join(tmp, f"log_{tag}")
    env = dict(os.environ, Q4_ORACLE_LIB=so, LD_PRELOAD=_runtime(), PYTHONDONTWRITEBYTECODE="1",
               ASAN_OPTIONS=f"detect_leaks=0:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    # -s: a report written to stderr just before the child exits must not
    # sit in pytest's capture buffer
    args = [sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", *PIN_FILES]
    if select:
        args += ["-k", select]
    r = subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    reports += "".join(line + "\n" for line in r.stderr.splitlines()
                       if "Sanitizer" in line or "runtime error" in line)
    return r.returncode, reports, r.stdout[-2000:]


pytestmark = pytest.mark.skipif(_runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")


def test_oracle_pins_clean_under_asan_and_ubsan(tmp_path):
    with open(O.SRC) as f:
        so = _build(str(tmp_path), "oracle", f.read())
    rc, reports, out = _run(so, str(tmp_path), "clean")
    assert reports == "", reports[:4000]
    assert rc == 0, out


def test_sanitizers_report_planted_mistakes(tmp_path):
    with open(O.SRC) as f:
        src = f.read()
    # a read one block scale past the end of the window's scales
    old = "m_out[j] = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[blk];"
    assert src.count(old) == 1
    so = _build(str(tmp_path), "oob", src.replace(old, old.replace("[blk]", "[blk + 1]")))
    rc, reports, _ = _run(so, str(tmp_path), "oob", select="dequant_equals")
    assert rc != 0 and "AddressSanitizer: heap-buffer-overflow" in reports
    # a left shift that overflows int (15 << 28)
    old = "codes[j >> 1] = (uint8_t)((codes[j >> 1] & 0x0F) | (code << 4));"
    assert src.count(old) == 1
    so = _build(str(tmp_path), "shift", src.replace(old, old.replace("code << 4", "code << 28")))
    rc, reports, _ = _run(so, str(tmp_path), "shift", select="steps_from_crafted")
    assert rc != 0 and "runtime error" in reports and "shift" in reports
