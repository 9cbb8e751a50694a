"""Pins of the oracle where it reads a non-zero state.

From the zero state every decode is 0, so the first step cannot show whether
the oracle reads its codes and scales correctly.  These tests start from
crafted non-zero states (random codes, block scales of realistic sizes, a
few zero blocks) and check each of a few consecutive steps against a decode
and an AdamW update written here, apart from the oracle:

  * the packed layout of the pages: one 4-bit code per element, element 2j
    in the low nibble of byte j (odd length: the last high nibble unused),
    one FP32 scale per 128-element block ([A] "State representation", [N]
    storage paragraph); the decoded moment is level[code] * block scale;
  * AdamW with decoupled decay in binary64 from the decoded moments ([N]
    AdamW paragraph; the bias correction is the torch form);
  * the requantized state: new scales = block absmax of the binary64
    moments, nearest levels (RTN) or the bracketing pair (SR) of m1 / s.

The level tables come from the oracle (they are pinned by
``test_oracle_pins.py``); everything else here is numpy.  A swapped nibble
order, or a decode that forgets the block scale, fails these pins
(``test_oracle_mutants.py`` plants such mistakes in a copy of the oracle and
checks that they do).
"""
import numpy as np
import pytest

from oracle import oracle as O

BLOCK = 128


# ---------------------------------------------------------------------------
# Independent decode and update (numpy; shares nothing with the oracle's C)
# ---------------------------------------------------------------------------

def nibbles(codes: np.ndarray, n: int) -> np.ndarray:
    """Element 2j is the low nibble of byte j, element 2j+1 the high one."""
    out = np.empty(2 * codes.size, np.int64)
    out[0::2] = codes % 16
    out[1::2] = codes // 16
    return out[:n]


def decode(codes: np.ndarray, scales: np.ndarray, table: np.ndarray, n: int, bytes_per_code: int = 0) -> np.ndarray:
    """level[code] * scale of the element's block, as one FP32 product."""
    idx = codes[:n].astype(np.int64) if bytes_per_code == 1 else nibbles(codes, n)
    per_elem = np.repeat(scales.astype(np.float32), BLOCK)[:n]
    return table.astype(np.float32)[idx] * per_elem


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def moments64(hp: O.HParams, m0, v0, g):
    """The unquantized moments of one AdamW step, in binary64."""
    b1, b2 = float(np.float32(hp.beta1)), float(np.float32(hp.beta2))
    m1 = b1 * m0 + (1.0 - b1) * g
    v1 = b2 * v0 + (1.0 - b2) * g * g if v0 is not None else None
    return m1, v1


def weight64(hp: O.HParams, w, m1, v1):
    """The weight after decoupled decay and the bias-corrected Adam term."""
    return weight64_terms(hp, w, m1, v1)[0]


def weight64_terms(hp: O.HParams, w, m1, v1):
    """The new weight and the size of the two terms it is the difference of
    (FP32 arithmetic is accurate relative to the terms, not to a result that
    cancels)."""
    b1, b2 = float(np.float32(hp.beta1)), float(np.float32(hp.beta2))
    lr, wd, eps = float(np.float32(hp.lr)), float(np.float32(hp.weight_decay)), float(np.float32(hp.eps))
    t = hp.step
    bc1, bc2 = 1.0 - b1 ** t, 1.0 - b2 ** t
    decayed = w * (1.0 - lr * wd)
    adam = (lr / bc1) * m1 / (np.sqrt(v1 / bc2) + eps)
    return decayed - adam, np.abs(decayed) + np.abs(adam)


def block_absmax(x: np.ndarray) -> np.ndarray:
    n = x.size
    nb = (n + BLOCK - 1) // BLOCK
    pad = np.zeros(nb * BLOCK)
    pad[:n] = np.abs(x)
    return pad.reshape(nb, BLOCK).max(axis=1)


def rel_err(a, b, floor):
    return np.abs(np.asarray(a, np.float64) - b) / np.maximum(np.abs(b), floor)


def check_nearest(codes_idx, x, table, slack=2e-6):
    """Each code's level is (within slack) a nearest level to x."""
    L = table.astype(np.float64)
    d = np.abs(x[:, None] - L[None, :])
    assert np.all(d[np.arange(x.size), codes_idx] <= d.min(axis=1) + slack)


def check_bracket(codes_idx, x, table, slack=2e-6):
    """Each code's level lies in the bracket of x, widened by slack: between
    the largest level <= x - slack and the smallest level >= x + slack (SR
    picks the level just below or just above x)."""
    L = table.astype(np.float64)
    q = L[codes_idx]
    lo = np.where(L[None, :] <= x[:, None] - slack, L[None, :], -np.inf).max(axis=1)
    hi = np.where(L[None, :] >= x[:, None] + slack, L[None, :], np.inf).min(axis=1)
    assert np.all((q >= lo) & (q <= hi))


# ---------------------------------------------------------------------------
# Crafted states
# ---------------------------------------------------------------------------

def crafted_state(rng, st: O.TensorState, m_exp=(-4, -2), v_exp=(-8, -5)):
    """Random codes and block scales of realistic sizes; one block of each
    moment with scale 0 (where there are several blocks)."""
    n = st.numel
    nb = (n + BLOCK - 1) // BLOCK
    st.m_codes[:] = rng.integers(0, 256, st.m_codes.size, dtype=np.uint8)
    if n % 2:
        st.m_codes[-1] &= 0x0F
    st.m_scales[:] = (10.0 ** rng.uniform(*m_exp, nb)).astype(np.float32)
    if nb > 1:
        st.m_scales[1] = 0.0
    if st.v_codes is not None:
        st.v_codes[:] = rng.integers(0, 256, st.v_codes.size, dtype=np.uint8)
        if n % 2:
            st.v_codes[-1] &= 0x0F
        st.v_scales[:] = (10.0 ** rng.uniform(*v_exp, nb)).astype(np.float32)
        if nb > 2:
            st.v_scales[2] = 0.0


def grads_bits(rng, n, scale=1e-3):
    g = (rng.standard_t(3, n) * scale).astype(np.float32)
    # round to nearest even BF16
    u = g.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ---------------------------------------------------------------------------
# Dequantization
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("recipe", [O.ZIP_SR, O.ZE_EDEN, O.FACTORED])
@pytest.mark.parametrize("n", [1, 129, 1000, 2 * BLOCK * 5])
def test_dequant_equals_level_times_block_scale(recipe, n):
    rng = np.random.default_rng(n + 10 * recipe)
    cfg = O.Config.of(recipe)
    st = O.TensorState(cfg, (n,), 5)
    crafted_state(rng, st)
    m, v = st.dequant()
    nb = (n + BLOCK - 1) // BLOCK
    assert np.array_equal(m.view(np.uint32), decode(st.m_codes, st.m_scales, O.codebook(cfg.m_cb), n).view(np.uint32))
    assert np.array_equal(v.view(np.uint32), decode(st.v_codes, st.v_scales, O.codebook(cfg.v_cb), n).view(np.uint32))
    # a window that starts at a later block reads the window's own bytes
    if nb > 2:
        base = BLOCK
        mw, vw = O.dequant_window(cfg, numel=n, base=base, length=n - base, m_codes=st.m_codes[base // 2:],
                                  m_scales=st.m_scales[1:], v_codes=st.v_codes[base // 2:], v_scales=st.v_scales[1:])
        assert np.array_equal(mw.view(np.uint32), m[base:].view(np.uint32))
        assert np.array_equal(vw.view(np.uint32), v[base:].view(np.uint32))


def test_dequant_8bit_equals_level_times_block_scale():
    rng = np.random.default_rng(7)
    n = 777
    st = O.TensorState8((n,), 2)
    st.m_codes[:] = rng.integers(0, 256, n, dtype=np.uint8)
    st.v_codes[:] = rng.integers(0, 256, n, dtype=np.uint8)
    st.m_scales[:] = (10.0 ** rng.uniform(-4, -2, st.m_scales.size)).astype(np.float32)
    st.v_scales[:] = (10.0 ** rng.uniform(-8, -5, st.v_scales.size)).astype(np.float32)
    m, v = st.dequant()
    assert np.array_equal(m.view(np.uint32), decode(st.m_codes, st.m_scales, O.codebook8(O.CB8_SDYN8), n, 1).view(np.uint32))
    assert np.array_equal(v.view(np.uint32), decode(st.v_codes, st.v_scales, O.codebook8(O.CB8_DYN8), n, 1).view(np.uint32))


def test_dequant_factored_matrix_is_rank_one_estimate():
    rng = np.random.default_rng(8)
    rows, cols = 7, 300
    cfg = O.Config.of(O.FACTORED)
    st = O.TensorState(cfg, (rows, cols), 4)
    crafted_state(rng, st)
    st.R[:] = (10.0 ** rng.uniform(-8, -5, rows)).astype(np.float32)
    st.Cc[:] = (10.0 ** rng.uniform(-8, -5, cols)).astype(np.float32)
    st.inv_meanR = float(np.float32(1) / np.float32(st.R.astype(np.float64).mean()))
    m, v = st.dequant()
    n = rows * cols
    assert np.array_equal(m.view(np.uint32), decode(st.m_codes, st.m_scales, O.codebook(cfg.m_cb), n).view(np.uint32))
    ref = (np.outer(st.R, st.Cc).astype(np.float32) * np.float32(st.inv_meanR)).reshape(-1)
    assert np.array_equal(v.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------------------
# Steps from a non-zero state
# ---------------------------------------------------------------------------

HPS = [dict(), dict(lr=3e-3, beta1=0.8, beta2=0.95, weight_decay=0.0, seed=0x9E3779B97F4A7C15)]


@pytest.mark.parametrize("hpk", HPS, ids=["default", "other"])
@pytest.mark.parametrize("recipe", [O.ZIP_SR, O.ZE_EDEN, O.FACTORED])
@pytest.mark.parametrize("n", [1000, 4 * BLOCK + 37])
def test_steps_from_crafted_state(recipe, n, hpk):
    """Three steps from a crafted non-zero state; before each step the state
    is decoded here and the step recomputed in binary64."""
    rng = np.random.default_rng(n * 7 + recipe)
    cfg = O.Config.of(recipe)
    st = O.TensorState(cfg, (n,), 9)
    crafted_state(rng, st)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Lm, Lv = O.codebook(cfg.m_cb), O.codebook(cfg.v_cb)
    Lm_sorted, _, _ = O.sorted_levels(cfg.m_cb)
    Lv_sorted, _, _ = O.sorted_levels(cfg.v_cb)
    for t in (3, 4, 5):
        hp = O.HParams(step=t, **hpk)
        g = grads_bits(rng, n)
        m0 = decode(st.m_codes, st.m_scales, Lm, n).astype(np.float64)
        v0 = decode(st.v_codes, st.v_scales, Lv, n).astype(np.float64)
        w_before = w.astype(np.float64)
        m1, v1 = moments64(hp, m0, v0, bf16_to_f64(g))
        w_ref = weight64(hp, w_before, m1, v1)
        st.step(hp, w, g)
        rms = float(np.sqrt(np.mean(w_ref ** 2)))
        assert rel_err(w, w_ref, rms).max() <= 1e-6
        # new scales: block absmax of the binary64 moments
        sm = block_absmax(m1)
        assert rel_err(st.m_scales, sm, 1e-30).max() <= 1e-6
        xm = m1 / np.repeat(np.where(sm > 0, sm, 1.0), BLOCK)[:n]
        check_nearest(nibbles(st.m_codes, n), xm, Lm)
        sv = block_absmax(v1)
        xv = v1 / np.repeat(np.where(sv > 0, sv, 1.0), BLOCK)[:n]
        cv = nibbles(st.v_codes, n)
        if cfg.v_rule == O.UPDATE_SR:
            assert rel_err(st.v_scales, sv, 1e-30).max() <= 1e-6
            check_bracket(cv, xv, Lv)
        else:
            check_nearest(cv, xv, Lv)
            q = Lv.astype(np.float64)[cv]
            nb = sv.size
            pad = lambda a: np.concatenate([a, np.zeros(nb * BLOCK - n)]).reshape(nb, BLOCK)
            if cfg.eden:
                sxx, sxq = (pad(xv) ** 2).sum(1), (pad(xv) * pad(q)).sum(1)
                S = np.where(sxq > 0, sxx / np.where(sxq > 0, sxq, 1), 1.0)
                assert rel_err(st.v_scales, sv * S, 1e-30).max() <= 1e-5
            else:
                assert rel_err(st.v_scales, sv, 1e-30).max() <= 1e-6
        if n % 2:
            assert st.m_codes[-1] >> 4 == 0 and st.v_codes[-1] >> 4 == 0


def test_factored_matrix_steps_from_crafted_state():
    """A factored matrix from a crafted state: m is decoded as above, v is
    the rank-1 estimate R_r C_c / mean(R) of the row and column means of g^2
    after their exponential update ([A] "State representation")."""
    rng = np.random.default_rng(12)
    rows, cols = 9, 200
    n = rows * cols
    cfg = O.Config.of(O.FACTORED)
    st = O.TensorState(cfg, (rows, cols), 6)
    crafted_state(rng, st)
    st.R[:] = (10.0 ** rng.uniform(-8, -6, rows)).astype(np.float32)
    st.Cc[:] = (10.0 ** rng.uniform(-8, -6, cols)).astype(np.float32)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Lm = O.codebook(cfg.m_cb)
    for t in (2, 3):
        hp = O.HParams(step=t)
        g = grads_bits(rng, n)
        g64 = bf16_to_f64(g).reshape(rows, cols)
        b2 = float(np.float32(hp.beta2))
        R = b2 * st.R.astype(np.float64) + (1 - b2) * (g64 ** 2).mean(axis=1)
        Cc = b2 * st.Cc.astype(np.float64) + (1 - b2) * (g64 ** 2).mean(axis=0)
        v1 = (np.outer(R, Cc) / R.mean()).reshape(-1)
        m0 = decode(st.m_codes, st.m_scales, Lm, n).astype(np.float64)
        m1, _ = moments64(hp, m0, None, g64.reshape(-1))
        w_ref = weight64(hp, w.astype(np.float64), m1, v1)
        st.step(hp, w, g)
        assert rel_err(st.R, R, 1e-30).max() <= 1e-6 and rel_err(st.Cc, Cc, 1e-30).max() <= 1e-6
        rms = float(np.sqrt(np.mean(w_ref ** 2)))
        assert rel_err(w, w_ref, rms).max() <= 1e-6
        sm = block_absmax(m1)
        assert rel_err(st.m_scales, sm, 1e-30).max() <= 1e-6
        check_nearest(nibbles(st.m_codes, n), m1 / np.repeat(np.where(sm > 0, sm, 1), BLOCK)[:n], Lm)


def test_8bit_steps_from_crafted_state():
    rng = np.random.default_rng(13)
    n = 1000
    st = O.TensorState8((n,), 2)
    st.m_codes[:] = rng.integers(0, 256, n, dtype=np.uint8)
    st.v_codes[:] = rng.integers(0, 256, n, dtype=np.uint8)
    st.m_scales[:] = (10.0 ** rng.uniform(-4, -2, st.m_scales.size)).astype(np.float32)
    st.v_scales[:] = (10.0 ** rng.uniform(-8, -5, st.v_scales.size)).astype(np.float32)
    st.v_scales[1] = 0.0
    Lm, Lv = O.codebook8(O.CB8_SDYN8), O.codebook8(O.CB8_DYN8)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    for t in (4, 5):
        hp = O.HParams(step=t)
        g = grads_bits(rng, n)
        m0 = decode(st.m_codes, st.m_scales, Lm, n, 1).astype(np.float64)
        v0 = decode(st.v_codes, st.v_scales, Lv, n, 1).astype(np.float64)
        m1, v1 = moments64(hp, m0, v0, bf16_to_f64(g))
        w_ref = weight64(hp, w.astype(np.float64), m1, v1)
        st.step(hp, w, g)
        rms = float(np.sqrt(np.mean(w_ref ** 2)))
        assert rel_err(w, w_ref, rms).max() <= 1e-6
        sm, sv = block_absmax(m1), block_absmax(v1)
        assert rel_err(st.m_scales, sm, 1e-30).max() <= 1e-6
        assert rel_err(st.v_scales, sv, 1e-30).max() <= 1e-6
        check_nearest(st.m_codes.astype(np.int64), m1 / np.repeat(np.where(sm > 0, sm, 1), BLOCK)[:n], Lm)
        check_nearest(st.v_codes.astype(np.int64), v1 / np.repeat(np.where(sv > 0, sv, 1), BLOCK)[:n], Lv)
