"""Property tests of the oracle (hypothesis): random shapes, hyper-parameters,
seeds and step counts against invariants that hold at any size.

  * a step from a random non-zero state equals the binary64 AdamW update of
    the decoded state, its new scales are the block absmax of the binary64
    moments, and its codes are nearest levels (RTN) or bracketing levels
    (SR) of the normalized moments;
  * stepping block-aligned windows equals stepping the whole tensor;
  * the same inputs give the same bits, on every recipe;
  * dequantization is level[code] * block scale, read in the packed layout;
  * the FP32 recipe follows binary64 AdamW for any hyper-parameters;
  * storage is one nibble per element plus one FP32 scale per block and
    moment (1.0625 B/param whenever 128 divides the size);
  * every uniform is a multiple of 2^-24 in [0, 1 - 2^-24].

The decode and the binary64 update are the ones of
``test_oracle_decode_pins.py``, written apart from the oracle.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import oracle as O
from tests.test_oracle_decode_pins import (BLOCK, bf16_to_f64, block_absmax, check_bracket, check_nearest,
                                           crafted_state, decode, grads_bits, moments64, nibbles, rel_err,
                                           weight64, weight64_terms)

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])

hparams = st.fixed_dictionaries({
    "lr": st.floats(1e-5, 3e-2),
    "beta1": st.sampled_from([0.0, 0.5, 0.8, 0.9, 0.95]),
    "beta2": st.sampled_from([0.9, 0.95, 0.99, 0.999, 0.9999]),
    "eps": st.sampled_from([1e-12, 1e-10, 1e-8, 1e-6]),
    "weight_decay": st.sampled_from([0.0, 0.01, 0.1, 0.3]),
    "seed": st.integers(0, 2 ** 64 - 1),
})
recipes = st.sampled_from([O.ZIP_SR, O.ZE_EDEN, O.FACTORED])
sizes = st.integers(1, 2500)


@SETTINGS
@given(recipe=recipes, n=sizes, hpk=hparams, t0=st.integers(1, 2 ** 40), gexp=st.integers(-6, -1),
       data_seed=st.integers(0, 2 ** 32 - 1))
def test_step_from_random_state_matches_binary64(recipe, n, hpk, t0, gexp, data_seed):
    rng = np.random.default_rng(data_seed)
    cfg = O.Config.of(recipe)
    state = O.TensorState(cfg, (n,), int(rng.integers(0, 2 ** 32)))
    crafted_state(rng, state, m_exp=(gexp - 2, gexp), v_exp=(2 * gexp - 3, 2 * gexp))
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    Lm, Lv = O.codebook(cfg.m_cb), O.codebook(cfg.v_cb)
    for t in (t0, t0 + 1):
        hp = O.HParams(step=t, **hpk)
        g = grads_bits(rng, n, 10.0 ** gexp)
        m0 = decode(state.m_codes, state.m_scales, Lm, n).astype(np.float64)
        v0 = decode(state.v_codes, state.v_scales, Lv, n).astype(np.float64)
        m1, v1 = moments64(hp, m0, v0, bf16_to_f64(g))
        w_ref, terms = weight64_terms(hp, w.astype(np.float64), m1, v1)
        state.step(hp, w, g)
        assert rel_err(w, w_ref, terms).max() <= 1e-6
        sm, sv = block_absmax(m1), block_absmax(v1)
        assert rel_err(state.m_scales, sm, 1e-30).max() <= 1e-6
        check_nearest(nibbles(state.m_codes, n), m1 / np.repeat(np.where(sm > 0, sm, 1), BLOCK)[:n], Lm)
        xv = v1 / np.repeat(np.where(sv > 0, sv, 1), BLOCK)[:n]
        if cfg.v_rule == O.UPDATE_SR:
            check_bracket(nibbles(state.v_codes, n), xv, Lv)
        else:
            check_nearest(nibbles(state.v_codes, n), xv, Lv)
        if n % 2:
            assert state.m_codes[-1] >> 4 == 0 and state.v_codes[-1] >> 4 == 0


@SETTINGS
@given(recipe=recipes, nblocks=st.integers(2, 20), tail=st.integers(0, 127), hpk=hparams,
       cut=st.integers(1, 19), data_seed=st.integers(0, 2 ** 32 - 1))
def test_windows_equal_whole_tensor(recipe, nblocks, tail, hpk, cut, data_seed):
    n = nblocks * BLOCK + tail
    cut = min(cut, nblocks - 1) * BLOCK
    rng = np.random.default_rng(data_seed)
    cfg = O.Config.of(recipe)
    whole, parts = O.TensorState(cfg, (n,), 11), O.TensorState(cfg, (n,), 11)
    crafted_state(rng, whole)
    for f in ("m_codes", "m_scales", "v_codes", "v_scales"):
        getattr(parts, f)[:] = getattr(whole, f)
    pw = (rng.standard_normal(n) * 0.02).astype(np.float32)
    pp = pw.copy()
    for t in (1, 2):
        hp = O.HParams(step=t, **hpk)
        g = grads_bits(rng, n)
        whole.step(hp, pw, g)
        for lo, hi in ((0, cut), (cut, n)):
            O.step_window(cfg, hp, tensor_id=11, flags=0, numel=n, base=lo, param=pp[lo:hi], grad=g[lo:hi].copy(),
                          m_codes=parts.m_codes[lo // 2:(hi + 1) // 2], m_scales=parts.m_scales[lo // BLOCK:],
                          v_codes=parts.v_codes[lo // 2:(hi + 1) // 2], v_scales=parts.v_scales[lo // BLOCK:])
    assert np.array_equal(pw.view(np.uint32), pp.view(np.uint32))
    for f in ("m_codes", "m_scales", "v_codes", "v_scales"):
        assert np.array_equal(getattr(whole, f).view(np.uint8), getattr(parts, f).view(np.uint8))


@SETTINGS
@given(recipe=st.sampled_from([O.ZIP_SR, O.ZE_EDEN, O.FACTORED, O.FP32]), n=sizes, hpk=hparams,
       data_seed=st.integers(0, 2 ** 32 - 1))
def test_same_inputs_same_bits(recipe, n, hpk, data_seed):
    outs = []
    for _ in range(2):
        rng = np.random.default_rng(data_seed)
        state = O.TensorState(O.Config.of(recipe), (n,), 3)
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        for t in (1, 2, 3):
            state.step(O.HParams(step=t, **hpk), w, grads_bits(rng, n))
        m, v = state.dequant()
        outs.append((w.view(np.uint32).copy(), m.view(np.uint32), v.view(np.uint32)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@SETTINGS
@given(recipe=recipes, n=sizes, data_seed=st.integers(0, 2 ** 32 - 1))
def test_dequant_reads_the_packed_layout(recipe, n, data_seed):
    rng = np.random.default_rng(data_seed)
    cfg = O.Config.of(recipe)
    state = O.TensorState(cfg, (n,), 1)
    crafted_state(rng, state)
    m, v = state.dequant()
    assert np.array_equal(m.view(np.uint32), decode(state.m_codes, state.m_scales, O.codebook(cfg.m_cb), n).view(np.uint32))
    assert np.array_equal(v.view(np.uint32), decode(state.v_codes, state.v_scales, O.codebook(cfg.v_cb), n).view(np.uint32))


@SETTINGS
@given(n=sizes, hpk=hparams, gexp=st.integers(-6, -1), data_seed=st.integers(0, 2 ** 32 - 1))
def test_fp32_recipe_follows_binary64_adamw(n, hpk, gexp, data_seed):
    rng = np.random.default_rng(data_seed)
    state = O.TensorState(O.Config.of(O.FP32), (n,), 0)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w64 = w.astype(np.float64)
    m64 = np.zeros(n)
    v64 = np.zeros(n)
    for t in range(1, 6):
        hp = O.HParams(step=t, **hpk)
        g = grads_bits(rng, n, 10.0 ** gexp)
        m64, v64 = moments64(hp, m64, v64, bf16_to_f64(g))
        w64 = weight64(hp, w64, m64, v64)
        state.step(hp, w, g)
    rms = float(np.sqrt(np.mean(w64 ** 2)))
    assert rel_err(w, w64, rms).max() <= 5e-6
    assert rel_err(state.m32, m64, float(np.sqrt(np.mean(m64 ** 2))) or 1e-30).max() <= 5e-6


@SETTINGS
@given(shape=st.lists(st.integers(1, 300), min_size=1, max_size=3))
def test_state_bytes_formula(shape):
    n = int(np.prod(shape))
    nb = (n + BLOCK - 1) // BLOCK
    for recipe in (O.ZIP_SR, O.ZE_EDEN):
        q, meta, tot = O.state_bytes(recipe, n, shape[0], len(shape) > 1)
        assert q == 2 * ((n + 1) // 2) and meta == 2 * 4 * nb and tot == q + meta
        if n % BLOCK == 0:
            assert tot == 1.0625 * n
    if len(shape) > 1:
        q, meta, tot = O.state_bytes(O.FACTORED, n, shape[0], True)
        assert q == (n + 1) // 2 and meta == 4 * nb + 4 * shape[0] + 4 * (n // shape[0])


@SETTINGS
@given(seed=st.integers(0, 2 ** 64 - 1), step=st.integers(1, 2 ** 64 - 1), tid=st.integers(0, 2 ** 32 - 1),
       stream=st.integers(0, 1), i=st.integers(0, 2 ** 40))
def test_uniform_is_on_the_2_24_grid(seed, step, tid, stream, i):
    u = O.uniform(seed, step, tid, stream, i)
    k = u * 2 ** 24
    assert 0.0 <= u <= 1 - 2 ** -24 and k == int(k)
    # the counter word of the step is its low 32 bits
    assert O.uniform(seed, step % 2 ** 32 + 2 ** 32, tid, stream, i) == u
