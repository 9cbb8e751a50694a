"""Pins of the oracle on non-finite gradients (NaN, +-inf, and finite values
whose square overflows FP32).

The pages say nothing about non-finite values.  The oracle's reading is that
its IEEE operations, in the order written, decide:

  * a block maximum takes a value only when it compares greater, so a NaN is
    skipped and +inf kept;
  * an infinite scale has the inverse 1/inf = 0, so its block normalizes
    finite values to 0 and infinite ones to NaN (inf * 0);
  * normalized values are clamped to the range of the levels by comparison,
    which a NaN fails, and a NaN lies above no midpoint and no level: it
    takes sorted index 0 under every rule (round to nearest counts the
    midpoints below it; the stochastic rules start from the lower bracket 0
    and no comparison moves them up);
  * EDEN's ratio over a block that holds a NaN normalized value is 1 (its
    sums are NaN and the guard <x,Q(x)> > 0 fails);
  * the weight follows IEEE arithmetic: NaN where the Adam term is NaN
    (a NaN gradient, or inf / inf), the decayed weight where it is 0
    (a finite first moment over an infinite denominator).

The expectations below are worked out from those rules with numpy, apart
from the oracle's C.  The 8-bit quantizer clamps the same way.
"""
import numpy as np
import pytest
import torch

from bit_adamw_update_amd import inputs
from oracle import oracle as O

BLOCK = 128
N = 1000  # eight blocks, the last one ragged: every class of the generator once
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _grads(step: int, n: int = N):
    w = inputs.custom([(n,)], grad_kind="nonfinite", seed=3)
    g = w.grads(step)[0].reshape(-1)
    return g.view(torch.int16).numpy().view(np.uint16).copy(), g.float().numpy().astype(np.float32)


def _params(n: int = N):
    return inputs.custom([(n,)], grad_kind="nonfinite", seed=3).init_params()[0].reshape(-1).numpy().copy()


def _classes(n: int = N):
    return [(b, inputs.Workload.NONFINITE_CLASSES[b % len(inputs.Workload.NONFINITE_CLASSES)])
            for b in range((n + BLOCK - 1) // BLOCK)]


def _nibbles(codes, n):
    out = np.empty(2 * codes.size, np.int64)
    out[0::2] = codes & 15
    out[1::2] = codes >> 4
    return out[:n]


def _index0_code(cb: int) -> int:
    L, code, _ = O.sorted_levels(cb)
    return int(code[0])


def _zero_level_code(cb: int):
    L, code, _ = O.sorted_levels(cb)
    hit = np.nonzero(L == 0.0)[0]
    return int(code[hit[0]]) if hit.size else int(code[0])


def _first_moments(g32):
    """Step 1 from the zero state: m1 = (1 - b1) g and v1 = (1 - b2) g^2 in
    FP32 (the multiply-adds add exact zeros)."""
    omb1, omb2 = np.float32(1) - np.float32(HP["beta1"]), np.float32(1) - np.float32(HP["beta2"])
    with np.errstate(over="ignore", invalid="ignore"):
        return omb1 * g32, omb2 * (g32 * g32)


def _block_max(x):
    """Maximum that skips NaN (0 for a block of NaN only), as '>' does."""
    f = x[~np.isnan(x)]
    return np.float32(f.max()) if f.size else np.float32(0.0)


RECIPES = [("zip_sr", O.ZIP_SR), ("ze_eden", O.ZE_EDEN), ("factored_vector", O.FACTORED)]


@pytest.mark.parametrize("name,recipe", RECIPES)
def test_step_one_scales_codes_and_weights(name, recipe):
    bits, g32 = _grads(1)
    p = _params()
    w0 = p.copy()
    cfg = O.Config.of(recipe)
    st = O.TensorState(cfg, (N,), tensor_id=5)
    st.step(O.HParams(step=1, **HP), p, bits)
    m1, v1 = _first_moments(g32)
    mcodes, vcodes = _nibbles(st.m_codes, N), _nibbles(st.v_codes, N)
    m_idx0, v_idx0 = _index0_code(cfg.m_cb), _index0_code(cfg.v_cb)
    m_zero, v_zero = _zero_level_code(cfg.m_cb), _zero_level_code(cfg.v_cb)
    for b, cls in _classes():
        sl = slice(BLOCK * b, min(N, BLOCK * b + BLOCK))
        sm, sv = _block_max(np.abs(m1[sl])), _block_max(v1[sl])
        # scales: NaN skipped, +inf kept (EDEN folds a ratio of 1 into a
        # block with a NaN normalized value)
        assert st.m_scales[b].tobytes() == sm.tobytes(), (name, b)
        if cfg.eden and not np.all(np.isfinite(v1[sl])):
            assert st.v_scales[b].tobytes() == sv.tobytes(), (name, b)
        elif not cfg.eden:
            assert st.v_scales[b].tobytes() == sv.tobytes(), (name, b)
        with np.errstate(invalid="ignore", divide="ignore"):
            xm = m1[sl] * (np.float32(0) if np.isinf(sm) else np.float32(1) / sm)
            xv = v1[sl] * (np.float32(0) if np.isinf(sv) else np.float32(1) / sv)
        # a NaN normalized value takes sorted index 0
        assert np.all(mcodes[sl][np.isnan(xm)] == m_idx0), (name, b)
        assert np.all(vcodes[sl][np.isnan(xv)] == v_idx0), (name, b)
        if np.isinf(sm):
            # an infinite scale sends every finite value to 0
            assert np.all(mcodes[sl][~np.isnan(xm)] == m_zero), (name, b)
        if np.isinf(sv):
            assert np.all(vcodes[sl][~np.isnan(xv)] == (v_zero if cfg.v_cb == O.CB_DYN4 else v_idx0)), (name, b)
    # weights: NaN exactly where the Adam term is NaN; the overflowing
    # gradient's weight only decays (m1 / inf = 0)
    nan_g = np.isnan(g32) | np.isinf(g32)
    assert np.array_equal(np.isnan(p), nan_g), name
    over = np.isfinite(g32) & np.isinf(v1)
    decay = np.float32(1.0 - np.float64(np.float32(HP["lr"])) * np.float64(np.float32(HP["weight_decay"])))
    assert over.sum() == 1 and np.array_equal(p[over], w0[over] * decay), name
    assert np.all(np.isfinite(p[~nan_g])), name


@pytest.mark.parametrize("name,recipe", RECIPES)
def test_blocks_without_non_finite_values_are_untouched(name, recipe):
    """Blocks are independent: a block's codes, scales and weights are those
    of the same step with every other block's gradients replaced by zeros;
    and in a block with one NaN gradient the other elements get the codes
    they get with that gradient replaced by 0 (NaN is skipped by the
    maximum, as a 0 is), except under EDEN, whose ratio the NaN sets to 1."""
    bits, g32 = _grads(1)
    cfg = O.Config.of(recipe)

    def run(b):
        p = _params()
        st = O.TensorState(cfg, (N,), tensor_id=5)
        st.step(O.HParams(step=1, seed=11, **HP), p, b)
        return p, _nibbles(st.m_codes, N), _nibbles(st.v_codes, N), st.m_scales.copy(), st.v_scales.copy()

    ref = run(bits)
    for b, cls in _classes():
        if cls != [(37, float("nan"))]:
            continue
        zb = bits.copy()
        zb[BLOCK * b + 37] = 0
        alt = run(zb)
        sl = slice(BLOCK * b, BLOCK * b + BLOCK)
        keep = np.ones(BLOCK, bool)
        keep[37] = False
        assert np.array_equal(ref[1][sl][keep], alt[1][sl][keep])
        assert ref[3][b] == alt[3][b]
        if not cfg.eden:
            assert np.array_equal(ref[2][sl][keep], alt[2][sl][keep])
            assert ref[4][b] == alt[4][b]
    # finite blocks equal those of a run where only they hold gradients
    only = np.zeros_like(bits)
    fin = [b for b, cls in _classes() if cls == []]
    for b in fin:
        only[BLOCK * b:BLOCK * b + BLOCK] = bits[BLOCK * b:BLOCK * b + BLOCK]
    alt = run(only)
    for b in fin:
        sl = slice(BLOCK * b, min(N, BLOCK * b + BLOCK))
        for k in range(5):
            if k < 3:
                assert np.array_equal(ref[k][sl], alt[k][sl]), (name, b, k)
            else:
                assert ref[k][b] == alt[k][b], (name, b, k)


@pytest.mark.parametrize("name,recipe", RECIPES)
def test_blocks_with_infinite_gradients_over_steps(name, recipe):
    """A block with an infinite gradient (at the same place every step) has
    infinite m and v scales after step 1, its finite values normalize to 0
    and the infinite one to NaN.  Its codes decode to level * inf or
    0 * inf from then on, so every moment of the block is +-inf or NaN, or
    0 after a step whose moments were all NaN (the maximum skips each NaN
    and the scale is 0).  Over the steps its scales are only 0 or inf, its
    codes only the zero level or sorted index 0, and from step 2 every
    weight of the block is NaN.  Finite blocks stay finite."""
    cfg = O.Config.of(recipe)
    p = _params()
    st = O.TensorState(cfg, (N,), tensor_id=5)
    m_ok = {_index0_code(cfg.m_cb), _zero_level_code(cfg.m_cb)}
    v_ok = {_index0_code(cfg.v_cb), _zero_level_code(cfg.v_cb)}
    seen_zero = False
    for step in (1, 2, 3, 4):
        bits, g32 = _grads(step)
        st.step(O.HParams(step=step, **HP), p, bits)
        mcodes, vcodes = _nibbles(st.m_codes, N), _nibbles(st.v_codes, N)
        for b, cls in _classes():
            sl = slice(BLOCK * b, min(N, BLOCK * b + BLOCK))
            if cls and any(np.isinf(v) for _, v in cls):
                for s in (st.m_scales[b], st.v_scales[b]):
                    assert s == 0.0 or s == np.inf, (name, step, b, s)
                    seen_zero |= s == 0.0
                if step == 1:
                    assert np.isinf(st.m_scales[b]) and np.isinf(st.v_scales[b]), (name, b)
                assert set(mcodes[sl].tolist()) <= m_ok, (name, step, b)
                assert set(vcodes[sl].tolist()) <= v_ok, (name, step, b)
                if step > 1:
                    assert np.all(np.isnan(p[sl])), (name, step, b)
            elif cls == []:
                assert np.isfinite(st.m_scales[b]) and np.isfinite(st.v_scales[b]), (name, step, b)
                assert st.m_scales[b] > 0 and st.v_scales[b] > 0, (name, step, b)
                assert np.all(np.isfinite(p[sl])), (name, step, b)
    assert seen_zero   # the all-NaN step of a +inf block


def test_eden_ratio_is_one_with_a_nan_value():
    """ZE-EDEN: a block whose normalized values include NaN stores its plain
    maximum (ratio 1); a finite block stores the maximum times
    <x,x>/<x,Q(x)>, which is not 1 for these gradients."""
    bits, g32 = _grads(1)
    cfg = O.Config.of(O.ZE_EDEN)
    st = O.TensorState(cfg, (N,), tensor_id=5)
    st.step(O.HParams(step=1, **HP), _params(), bits)
    _, v1 = _first_moments(g32)
    for b, cls in _classes():
        sl = slice(BLOCK * b, min(N, BLOCK * b + BLOCK))
        sv = _block_max(v1[sl])
        if cls is None or any(np.isnan(v) for _, v in (cls or [])):
            assert st.v_scales[b] == sv
        elif cls == []:
            assert st.v_scales[b] != sv


def test_fp32_recipe_weights():
    bits, g32 = _grads(1)
    p = _params()
    st = O.TensorState(O.Config.of(O.FP32), (N,), tensor_id=5)
    st.step(O.HParams(step=1, **HP), p, bits)
    bad = ~np.isfinite(g32)
    assert np.array_equal(np.isnan(p), bad)
    assert np.array_equal(np.isnan(st.m32), np.isnan(g32))
    assert np.array_equal(np.isinf(st.m32), np.isinf(g32))
    assert np.array_equal(np.isinf(st.v32), np.isinf(g32) | (np.isfinite(g32) & (np.abs(g32) > 1e20)))


def test_8bit_quantizer():
    """The 8-bit quantizer follows the same reading: NaN normalized values
    take sorted index 0 of each map (v: the level 0; m: the level -1)."""
    bits, g32 = _grads(1)
    p = _params()
    st = O.TensorState8((N,), tensor_id=5)
    st.step(O.HParams(step=1, **HP), p, bits)
    Lm, cm, _ = O.sorted_levels8(O.CB8_SDYN8)
    Lv, cv, _ = O.sorted_levels8(O.CB8_DYN8)
    assert Lm[0] == -1.0 and Lv[0] == 0.0
    m1, v1 = _first_moments(g32)
    for b, cls in _classes():
        sl = slice(BLOCK * b, min(N, BLOCK * b + BLOCK))
        sm, sv = _block_max(np.abs(m1[sl])), _block_max(v1[sl])
        assert st.m_scales[b].tobytes() == sm.tobytes() and st.v_scales[b].tobytes() == sv.tobytes()
        with np.errstate(invalid="ignore", divide="ignore"):
            xm = m1[sl] * (np.float32(0) if np.isinf(sm) else np.float32(1) / sm)
            xv = v1[sl] * (np.float32(0) if np.isinf(sv) else np.float32(1) / sv)
        assert np.all(st.m_codes[sl][np.isnan(xm)] == cm[0])
        assert np.all(st.v_codes[sl][np.isnan(xv)] == cv[0])
    assert np.array_equal(np.isnan(p), ~np.isfinite(g32))


def test_accumulation_norm_and_clip():
    """BF16 accumulation keeps NaN quiet and adds infinities by IEEE rules;
    the binary64 norm is NaN or inf; the clip factor of a NaN norm is 1
    (c < 1 fails) and of an infinite norm 0."""
    nan, inf = 0x7FC0, 0x7F80
    acc = np.array([nan, inf, inf, 0x3F80, 0x7F7F], np.uint16)            # NaN, inf, inf, 1, max
    micro = np.array([0x3F80, 0x3F80, 0xFF80, 0x7FC0, 0x7F7F], np.uint16)  # 1, 1, -inf, NaN, max
    O.accumulate_bf16(acc, micro, first=False)
    f = (acc.astype(np.uint32) << 16).view(np.float32)
    assert np.isnan(f[0]) and f[1] == np.inf and np.isnan(f[2]) and np.isnan(f[3]) and f[4] == np.inf
    assert acc[0] & 0x0040 and acc[2] & 0x0040 and acc[3] & 0x0040   # quiet NaNs
    assert np.isnan(O.grad_sumsq(np.array([0x3F80, nan], np.uint16)))
    assert O.grad_sumsq(np.array([0x3F80, inf], np.uint16)) == np.inf
    assert O.clip_factor(float("nan"), 1.0) == 1.0
    assert O.clip_factor(float("inf"), 1.0) == 0.0


def test_factored_statistics():
    """A factored matrix whose gradients hold +inf: its row and column
    statistics are infinite at that row and column, mean(R) is infinite and
    the inverse the step uses is 0; a NaN makes its row and column NaN."""
    rows, cols = 8, 256
    w = inputs.custom([(rows, cols)], grad_kind="nonfinite", seed=3)
    g = w.grads(1)[0].reshape(-1)
    bits = g.view(torch.int16).numpy().view(np.uint16).copy()
    g32 = g.float().numpy().reshape(rows, cols)
    R = np.zeros(rows, np.float32)
    Cc = np.zeros(cols, np.float32)
    inv = O.factored_update(O.HParams(step=1, **HP), rows, cols, bits, R, Cc)
    with np.errstate(over="ignore", invalid="ignore"):
        sq = g32.astype(np.float64) ** 2
    row_nan = np.isnan(sq).any(axis=1)
    row_inf = ~row_nan & np.isinf(sq).any(axis=1)
    assert np.array_equal(np.isnan(R), row_nan) and np.array_equal(np.isinf(R), row_inf)
    col_nan = np.isnan(sq).any(axis=0)
    assert np.array_equal(np.isnan(Cc), col_nan)
    assert row_nan.any() and row_inf.any()
    # mean(R) over a NaN row is NaN: 1/mean is NaN, and the guard mean > 0
    # fails, so the inverse is 0
    assert inv == 0.0
