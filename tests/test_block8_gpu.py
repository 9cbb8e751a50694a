"""GPU parity of the 8-bit blockwise AdamW recipe (SDyn8 m, Dyn8 v, one byte
per code) against the CPU oracle on the same seeded bytes: codes and scales
bit-exact, weights within 1e-6 relative to max(|w|, rms(w))."""
import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import inputs
from oracle import oracle as O
from tests import parity

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _check_weights(p, ref, what):
    """Within 1e-6 of max(|w|, rms(w)); NaN and infinities matched exactly."""
    if p.size == 0:
        return
    err = float(parity._rel_err(p, ref).max())
    assert err <= parity.W_TOL, f"{what}: weight error {err:.3e}"


def run_windows(w, steps, windows=None, grads_on="cpu", clip=0.0, hp=None, step_offset=0):
    """Step the GPU state over the whole workload and the oracle over
    block windows [(i, b0, b1)] (all of every tensor when None); compare.
    hp overrides the workload's hyper-parameters; the step counts are
    step_offset + 1 .. step_offset + steps."""
    hpk = dict(w.hp, **(hp or {}))
    dev = torch.device("cuda")
    consts = w._tensor_consts(grads_on)
    params = [p.reshape(-1) for p in w.init_params(grads_on)]
    gp = [p.to(dev).contiguous() for p in params]
    st = q4.Q4State("block8", w.tensors, dev)
    if windows is None:
        windows = [(i, 0, (t.numel + 127) // 128) for i, t in enumerate(w.tensors)]
    ost, op = [], []
    for i, b0, b1 in windows:
        t = w.tensors[i]
        lo, hi = b0 * 128, min(b1 * 128, t.numel)
        ost.append(O.TensorState8((hi - lo,), t.tensor_id, t.flags))
        op.append(params[i][lo:hi].cpu().numpy().copy())
    for s in range(1, steps + 1):
        g = w.grads(s, grads_on, consts)
        gg = [x.to(dev).reshape(-1).contiguous() for x in g]
        scale = 1.0
        if clip > 0:
            st.grad_stats(gp, gg)
            scale = O.clip_factor(sum(O.grad_sumsq(x.view(torch.uint16).cpu().numpy().reshape(-1)) for x in g),
                                  clip)
        st.step(gp, gg, step_offset + s, max_grad_norm=clip, **hpk)
        ohp = O.HParams(step=step_offset + s, grad_scale=scale, **hpk)
        for k, (i, b0, b1) in enumerate(windows):
            t = w.tensors[i]
            lo, hi = b0 * 128, min(b1 * 128, t.numel)
            # the window is its own tensor for the oracle: the tensor id and
            # the block-aligned offset are all the 8-bit step depends on
            gw = g[i].reshape(-1)[lo:hi].view(torch.uint16).cpu().numpy().copy()
            ost[k].step(ohp, op[k], gw)
    torch.cuda.synchronize()
    for k, (i, b0, b1) in enumerate(windows):
        b = st.bufs[i]
        t = w.tensors[i]
        lo, hi = b0 * 128, min(b1 * 128, t.numel)
        o = ost[k]
        assert np.array_equal(b.m_codes[lo:hi].cpu().numpy(), o.m_codes), f"tensor {i} m codes"
        assert np.array_equal(b.v_codes[lo:hi].cpu().numpy(), o.v_codes), f"tensor {i} v codes"
        assert np.array_equal(b.m_scales[b0:b1].cpu().numpy().view(np.uint32), o.m_scales.view(np.uint32))
        assert np.array_equal(b.v_scales[b0:b1].cpu().numpy().view(np.uint32), o.v_scales.view(np.uint32))
        _check_weights(gp[i][lo:hi].cpu().numpy(), op[k], f"tensor {i}")
    return st


def test_tiny_workload_10_steps():
    _flush("block8 tiny")
    run_windows(inputs.tiny(), 10)


@pytest.mark.parametrize("name,hpk,offset", [
    ("b0.9_0.95", dict(beta1=0.9, beta2=0.95), 0),
    ("b0_0.99_wd0", dict(beta1=0.0, beta2=0.99, weight_decay=0.0), 0),
    ("lr1e-4_eps1e-6", dict(lr=1e-4, eps=1e-6), 0),
    ("lr3e-3_step2^32", dict(lr=3e-3), 2 ** 32 - 3),
], ids=lambda x: x if isinstance(x, str) else "")
def test_hyperparameter_grid(name, hpk, offset):
    """Other betas, no decay, other learning rates and eps, and step counts
    past 2^32 (the bias correction in binary64), every element."""
    _flush(f"block8 hparams {name}")
    shapes = [(1,), (129,), (1000,), (4097,), (7, 129), (64, 520)]
    run_windows(inputs.custom(shapes, grad_kind="masked", seed=71), 5, hp=hpk, step_offset=offset)


def test_ragged_shapes():
    shapes = [(1,), (127,), (129,), (1000,), (4097,), (3, 5), (7, 129), (300, 3), (2, 1031)]
    _flush("block8 ragged")
    run_windows(inputs.custom(shapes, grad_kind="masked", seed=41), 5)


def test_zero_size_tensors_between_others():
    shapes = [(0,), (300,), (0,), (64, 520), (0, 5), (4097,), (0,)]
    _flush("block8 zero-size tensors")
    run_windows(inputs.custom(shapes, grad_kind="masked", seed=43), 4)


def test_mid_size_set_takes_short_runs():
    """About 10.2 M elements: the resident groups take runs of 2 slabs from
    the queue here, not 4 (fewer than 4 x 2,048 resident groups' worth of
    slabs)."""
    shapes = [(1024, 4096), (2048, 2048), (1_000_003,), (777, 1031), (4097,)]
    _flush("block8 mid-size set")
    run_windows(inputs.custom(shapes, grad_kind="masked", seed=45), 3)


def test_two_thousand_small_tensors():
    rng = np.random.default_rng(30)
    shapes = [(int(rng.integers(1, 1501)),) for _ in range(2000)]
    _flush("block8 2000 small tensors")
    run_windows(inputs.custom(shapes, grad_kind="masked", seed=44), 3)


def test_clipped_steps():
    _flush("block8 clipped")
    run_windows(inputs.custom([(3000,), (64, 200)], grad_kind="masked", seed=42), 4, clip=2e-3)


def test_dequant_matches_oracle():
    w = inputs.custom([(3000,), (48, 200)], grad_kind="masked", seed=43)
    st = run_windows(w, 3)
    # the oracle of the whole tensors again, for its dequantization
    consts = w._tensor_consts("cpu")
    params = [p.reshape(-1).numpy().copy() for p in w.init_params("cpu")]
    ost = [O.TensorState8(t.shape, t.tensor_id) for t in w.tensors]
    for s in range(1, 4):
        g = w.grads(s, "cpu", consts)
        for i, o in enumerate(ost):
            o.step(O.HParams(step=s, **w.hp), params[i], g[i].view(torch.uint16).numpy().reshape(-1).copy())
    for i, o in enumerate(ost):
        m, v = st.dequant(i)
        torch.cuda.synchronize()
        om, ov = o.dequant()
        assert np.array_equal(m.cpu().numpy().view(np.uint32), om.view(np.uint32))
        assert np.array_equal(v.cpu().numpy().view(np.uint32), ov.view(np.uint32))


def test_edge_magnitudes():
    """Tiny, BF16-subnormal (block scales below 2^-126), signed-zero, mixed
    and vanishing gradient blocks."""
    _flush("block8 edge magnitudes")
    run_windows(inputs.custom([(7 * 128 * 3 + 77,), (21, 140)], grad_kind="edge", seed=52), 6)


def test_gpt_162m_sampled_20_steps():
    """The GPT-style 162M set (123.6M parameters as written), 20 steps,
    first/last blocks of every tensor and random interior windows."""
    w = inputs.gpt_162m()
    wins = parity.sample_windows(w, n_random=32, seed=5)
    _flush("block8 gpt-162m")
    run_windows(w, 20, windows=wins, grads_on="cuda")


def test_gpt_2_7b_sampled():
    """The GPT-style 2.7B set in the launch configuration the benchmark times,
    10 steps, first/last blocks of every tensor and random interior windows."""
    w = inputs.gpt_2_7b()
    wins = parity.sample_windows(w, n_random=48, seed=6)
    _flush("block8 gpt-2.7b")
    run_windows(w, 10, windows=wins, grads_on="cuda")


def test_tensor_beyond_2_32_elements():
    """One tensor of 2^32 + 1000 elements: 64-bit element and code offsets,
    a ragged last block."""
    n = (1 << 32) + 1000
    w = inputs.custom([(n,)], grad_kind="masked", seed=28)
    nb = (n + 127) // 128
    lo32, lo31 = (1 << 32) // 128, (1 << 31) // 128
    wins = [(0, 0, 2), (0, lo31 - 2, lo31 + 2), (0, lo32 - 3, lo32 + 3), (0, nb - 3, nb)]
    _flush("block8 2^32 + 1000 elements")
    run_windows(w, 2, windows=wins, grads_on="cuda")
