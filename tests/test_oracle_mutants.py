"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/q4_oracle.c`` (a swapped
nibble order, a decode without its block scale, a dropped term, a wrong sign,
a transposed operand, a wrong Philox word, NaN handled another way ...), builds that copy with the
oracle's own flags, and runs the pin suites against it in a child process
(the oracle loads the library that Q4_ORACLE_LIB names).  The pins must fail
for every mutant.  The mistakes are planted in the CPU oracle only.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_decode_pins.py", "tests/test_oracle_pins.py", "tests/test_oracle_nonfinite.py"]

# (name, text in q4_oracle.c, replacement); the first occurrence is replaced
MUTANTS = [
    ("nibble read swapped", "return (j & 1) ? (codes[j >> 1] >> 4) : (codes[j >> 1] & 0x0F);",
     "return (j & 1) ? (codes[j >> 1] & 0x0F) : (codes[j >> 1] >> 4);"),
    ("nibble write swapped", "if (j & 1) codes[j >> 1] = (uint8_t)((codes[j >> 1] & 0x0F) | (code << 4));",
     "if (!(j & 1)) codes[j >> 1] = (uint8_t)((codes[j >> 1] & 0x0F) | (code << 4));"),
    ("step: m decoded without its scale", "m0 = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[blk];",
     "m0 = Lm[or_get_nibble(w->m_codes, j)];"),
    ("step: v decoded without its scale", "v0 = Lv[or_get_nibble(w->v_codes, j)] * w->v_scales[blk];",
     "v0 = Lv[or_get_nibble(w->v_codes, j)];"),
    ("step: m decoded with the first block's scale", "m0 = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[blk];",
     "m0 = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[0];"),
    ("dequant: m without its scale", "m_out[j] = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[blk];",
     "m_out[j] = Lm[or_get_nibble(w->m_codes, j)];"),
    ("dequant: v without its scale", "v_out[j] = Lv[or_get_nibble(w->v_codes, j)] * w->v_scales[blk];",
     "v_out[j] = Lv[or_get_nibble(w->v_codes, j)];"),
    ("8-bit step: m decoded without its scale", "float m0 = Lm[w->m_codes[j]] * w->m_scales[blk];",
     "float m0 = Lm[w->m_codes[j]];"),
    ("8-bit dequant: v without its scale", "v_out[j] = Lv[w->v_codes[j]] * w->v_scales[j / OR_BLOCK];",
     "v_out[j] = Lv[w->v_codes[j]];"),
    ("weight decay dropped", "w->param[j] = fmaf(-step_size, mm / denom, w->param[j] * decay);",
     "w->param[j] = fmaf(-step_size, mm / denom, w->param[j]);"),
    ("update sign flipped", "w->param[j] = fmaf(-step_size, mm / denom, w->param[j] * decay);",
     "w->param[j] = fmaf(step_size, mm / denom, w->param[j] * decay);"),
    ("v recurrence on g instead of g^2", "vv = fmaf(b2, v0, omb2 * (g * g));", "vv = fmaf(b2, v0, omb2 * g);"),
    ("m recurrence without beta1", "float mm = fmaf(b1, m0, omb1 * g);", "float mm = m0 + omb1 * g;"),
    ("second-moment bias correction dropped", "out[2] = (float)(1.0 / sqrt(bc2));", "out[2] = 1.0f;"),
    ("factored row mean over the wrong extent", "omb2 * ((float)(rs * s2) / (float)cols)",
     "omb2 * ((float)(rs * s2) / (float)rows)"),
    ("Philox word index off by one", "return (float)(w[i & 3] >> 8) * (1.0f / 16777216.0f);",
     "return (float)(w[(i + 1) & 3] >> 8) * (1.0f / 16777216.0f);"),
    ("Philox key words swapped", "uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };",
     "uint32_t key[2] = { (uint32_t)(seed >> 32), (uint32_t)seed };"),
    ("EDEN ratio inverted", "float S = sxq > 0.0f ? sxx / sxq : 1.0f;", "float S = sxx > 0.0f ? sxq / sxx : 1.0f;"),
    ("Update-SR decision reversed", "return u * den < num;", "return u * den > num;"),
    ("Update-SR probability measured in v", "float num = (sv - rlo) * (rhi + eps_sr);",
     "float num = (sv * sv - rlo * rlo) * (rhi + eps_sr);"),
    ("RTN ties to the upper level", "for (int j = 0; j + 1 < lv->n; ++j) if (x > lv->mid[j]) ++k;",
     "for (int j = 0; j + 1 < lv->n; ++j) if (x >= lv->mid[j]) ++k;"),
    ("absmax without the absolute value", "for (int k = 0; k < n; ++k) { float a = fabsf(m1[k]); if (a > s) s = a; }",
     "for (int k = 0; k < n; ++k) { float a = m1[k]; if (a > s) s = a; }"),
    # non-finite moments: a clamp that sends NaN to the top of the v range,
    # and a block maximum that lets NaN through
    ("v clamp sends NaN to 1", "static float or_clamp_unsigned(float x) {\n    if (x > 1.0f) x = 1.0f;",
     "static float or_clamp_unsigned(float x) {\n    x = fminf(x, 1.0f);"),
    ("v maximum keeps NaN", "for (int k = 0; k < n; ++k) if (v1[k] > s) s = v1[k];",
     "for (int k = 0; k < n; ++k) if (!(v1[k] <= s)) s = v1[k];"),
]


def _build(tmp, name, src):
    c = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"{name}.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", *O.CFLAGS, "-o", so, c, "-lm"])
    return so


def _pins_pass(so) -> bool:
    env = dict(os.environ, Q4_ORACLE_LIB=so, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode == 0


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(O.SRC) as f:
        src = f.read()
    sources = []
    for k, (name, old, new) in enumerate(MUTANTS):
        assert src.count(old) >= 1, f"mutant '{name}': its target text is gone from the oracle"
        sources.append((f"m{k}", src.replace(old, new, 1)))
    libs = [_build(str(tmp_path), nm, s) for nm, s in sources]
    with ThreadPoolExecutor(max_workers=6) as ex:
        survived = [MUTANTS[k][0] for k, ok in enumerate(ex.map(_pins_pass, libs)) if ok]
    assert not survived, f"mutants that pass every pin: {survived}"


def test_unmutated_copy_passes():
    """The harness itself: an unmodified copy, built the same way, passes."""
    import tempfile
    with tempfile.TemporaryDirectory() as tmp, open(O.SRC) as f:
        assert _pins_pass(_build(tmp, "same", f.read()))
