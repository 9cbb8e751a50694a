"""GPU parity on non-finite gradients: NaN, +-inf and finite values whose
square overflows FP32, at fixed places of each 128-block class (the input
generator's "nonfinite" kind), over several steps, so that infinite scales
and NaN moments also come back through the decode.  The oracle's reading
of non-finite moments decides (block maxima skip NaN and keep +inf; a NaN
normalized value takes sorted index 0; EDEN's ratio over such a block is 1;
the weight follows IEEE arithmetic); the kernels must agree with it code for
code and scale for scale, and match every NaN and infinite weight exactly."""
import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import inputs
from oracle import oracle as O
from tests import parity
from tests.test_accumulate_gpu import K, host_accumulate, setup
from tests.test_block8_gpu import run_windows

pytestmark = pytest.mark.gpu

SHAPES = [(1000,), (4100,), (48, 300), (7, 129), (1,), (2, 1031)]


def _flush(msg):
    print(msg, flush=True)


def _workload(seed=51, flags=None):
    return inputs.custom(SHAPES, grad_kind="nonfinite", seed=seed, flags=flags)


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_recipes(recipe):
    _flush(f"non-finite gradients {recipe}")
    rep = parity.run(_workload(), recipe, 4)
    rep.check()
    assert rep.codes_differ == 0
    assert rep.nonfinite_weights > 0


@pytest.mark.parametrize("variant", parity.VARIANTS, ids=lambda v: "-".join(map(str, v)))
def test_variants(variant):
    cfg = q4.q4adamw_default_config(q4.RECIPE_CUSTOM)
    cfg.m_codebook, cfg.v_codebook, cfg.m_rule, cfg.v_rule, cfg.eden = variant
    _flush(f"non-finite gradients variant {variant}")
    rep = parity.run(_workload(seed=52), "custom", 3, cfg=cfg)
    rep.check()
    assert rep.codes_differ == 0
    assert rep.nonfinite_weights > 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden"])
def test_lm_head_final_phase(recipe):
    """The LM head's first moment by state-space SR (the final phase, step
    4 of 4) with NaN and infinite moments."""
    _flush(f"non-finite gradients, LM-head phase {recipe}")
    w = _workload(seed=53, flags=[inputs.TF_LM_HEAD, 0, inputs.TF_LM_HEAD, 0, 0, 0])
    rep = parity.run(w, recipe, 4, lm_head_phase=True)
    rep.check()
    assert rep.codes_differ == 0


def test_block8():
    _flush("non-finite gradients, 8-bit")
    run_windows(_workload(seed=54), 4)


def _poisoned_microbatches(w, step, offsets, total, value):
    """K microbatches of Student-t draws; microbatch 2 holds `value` at two
    places of the first tensor and one of the matrix."""
    g = torch.Generator().manual_seed(7000 + step)
    out = []
    for k in range(K):
        flat = np.zeros(total, np.uint16)
        for i, t in enumerate(w.tensors):
            z = torch.randn(t.numel, generator=g) * 1e-3
            flat[offsets[i]: offsets[i] + t.numel] = z.to(torch.bfloat16).view(torch.uint16).numpy()
        if k == 2:
            bits = np.array([value], np.float32).view(np.uint32)[0] >> 16
            for pos in (offsets[0] + 3, offsets[0] + 700, offsets[1] + 1234):
                flat[pos] = bits
        out.append(flat)
    return out


@pytest.mark.parametrize("value", [float("inf"), float("nan")], ids=["inf", "nan"])
@pytest.mark.parametrize("recipe", ["zip_sr", "factored"])
def test_accumulated_and_clipped(recipe, value):
    """An infinite microbatch value makes the norm infinite and the clip
    factor 0 (finite gradients clip to 0, the infinite ones to NaN); a NaN
    makes the norm NaN and the clip factor 1.  The accumulated gradients
    match bit for bit, the clip factor bit for bit, and two clipped steps
    match the oracle."""
    w, st, params, grads, offsets, total = setup(recipe, seed=55)
    _flush(f"non-finite microbatch {value} {recipe}")
    ocfg = parity.oracle_config(recipe)
    ost = [O.TensorState(ocfg, t.shape, t.tensor_id, t.flags) for t in w.tensors]
    op = [p.cpu().numpy().copy() for p in params]
    for s in (1, 2):
        micro = _poisoned_microbatches(w, s, offsets, total, value)
        for k, flat in enumerate(micro):
            m = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
            st.accumulate(params, grads, m, first=(k == 0), last=(k == K - 1))
        st.step(params, grads, s, grad_stats=True, max_grad_norm=1.0, **w.hp)
        acc = host_accumulate(w, micro, offsets)
        for i in range(len(w.tensors)):
            assert np.array_equal(grads[i].view(torch.uint16).cpu().numpy(), acc[i]), f"tensor {i}"
        sq = sum(O.grad_sumsq(a) for a in acc)
        assert np.isinf(sq) if value == np.inf else np.isnan(sq)
        c = O.clip_factor(sq, 1.0)
        assert c == (0.0 if value == np.inf else 1.0)
        gpu_c = float(st.ws[8:12].view(torch.float32).cpu()[0])
        assert np.float32(gpu_c).view(np.uint32) == np.float32(c).view(np.uint32), (gpu_c, c)
        hp = O.HParams(step=s, grad_scale=c, **w.hp)
        for i, o in enumerate(ost):
            o.step(hp, op[i], acc[i])
    torch.cuda.synchronize()
    for i, (b, o) in enumerate(zip(st.bufs, ost)):
        err = parity._rel_err(params[i].cpu().numpy(), op[i])
        assert err.max() <= parity.W_TOL, f"tensor {i} weights"
        assert np.array_equal(b.m_codes.cpu().numpy(), o.m_codes), f"tensor {i} m codes"
        assert np.array_equal(b.m_scales.cpu().numpy().view(np.uint32), o.m_scales.view(np.uint32))
        if b.v_codes is not None:
            assert np.array_equal(b.v_codes.cpu().numpy(), o.v_codes), f"tensor {i} v codes"
            assert np.array_equal(b.v_scales.cpu().numpy().view(np.uint32), o.v_scales.view(np.uint32))
        elif b.numel > 0:
            for x, y in ((b.v_row, o.R), (b.v_col, o.Cc)):
                assert parity._rel_err(x.cpu().numpy(), y, floor=1e-30).max() <= parity.RC_TOL, f"tensor {i} R/C"
