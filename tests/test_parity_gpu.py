"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle on
the same seeded inputs.  Codes bit-exact (at most 1e-6 of them may differ,
only at SR ties), scales bit-exact, weights within 1e-6 relative, factored
R/C within 1e-6 relative."""
import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "fp32", "factored"])
def test_tiny_workload_10_steps(recipe):
    """The tiny check: one 65,536-element vector and one 256x512 matrix,
    Student-t grads at 1e-3 with a fixed 20% at 1e-9, 10 steps."""
    w = inputs.tiny()
    _flush(f"tiny {recipe}")
    rep = parity.run(w, recipe, 10)
    rep.check()
    assert rep.codes_differ == 0 and rep.weights_excluded == 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored"])
def test_ragged_shapes(recipe):
    """Empty-tail and ragged cases: single elements, partial blocks, partial
    lanes, odd lengths, a single block, factored matrices with odd column
    counts and columns shorter than a lane."""
    shapes = [(1,), (127,), (129,), (1000,), (4097,), (128,), (3, 5), (7, 129), (300, 3), (2, 1031), (64, 520)]
    w = inputs.custom(shapes, grad_kind="masked", seed=21)
    _flush(f"ragged {recipe}")
    rep = parity.run(w, recipe, 5)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_zero_size_tensors_between_others(recipe):
    """Tensors with no elements first, between others, in a row and last (a
    vector and a matrix with no rows): the chunk prefixes hold zero-width
    entries that the kernels' tensor search and run walk step over."""
    shapes = [(0,), (300,), (0,), (0,), (64, 520), (0, 5), (4097,), (0,)]
    w = inputs.custom(shapes, grad_kind="masked", seed=24)
    _flush(f"zero-size tensors {recipe}")
    rep = parity.run(w, recipe, 4)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_two_thousand_small_tensors(recipe):
    """2,000 tensors of 1 to 1,500 elements (vectors and small matrices):
    most step-prefix chunks only align the next tensor, a run of slabs spans
    dozens of tensors, and the tensor search walks a long prefix; every
    element over 3 steps."""
    rng = np.random.default_rng(30)
    shapes = []
    for k in range(2000):
        n = int(rng.integers(1, 1501))
        if k % 3 == 2 and n >= 4:
            r = int(rng.integers(1, 9))
            shapes.append((r, max(1, n // r)))
        else:
            shapes.append((n,))
    w = inputs.custom(shapes, grad_kind="masked", seed=31)
    _flush(f"2000 small tensors {recipe}")
    rep = parity.run(w, recipe, 3)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_mid_size_set_takes_short_runs(recipe):
    """A set of about 10.2 M elements (about 5,000 slabs of 4 chunks): with
    one work-group per run and at least as many runs as resident groups
    (1,536 for the ZIP-SR kernel, 2,048 for the others on MI355X), the
    launch takes runs of 2 slabs here: shortened for the ZIP-SR kernel, whose
    large sets take runs of 8, and the full length of the others.  Every
    element, 3 steps, tensors and matrices of uneven sizes."""
    shapes = [(1024, 4096), (2048, 2048), (1_000_003,), (777, 1031), (4097,)]
    w = inputs.custom(shapes, grad_kind="masked", seed=33)
    _flush(f"mid-size set {recipe}")
    rep = parity.run(w, recipe, 3)
    rep.check()
    assert rep.codes_differ == 0


def test_zip_sr_set_takes_runs_of_4():
    """About 19.1 M elements (about 9,300 slabs): the ZIP-SR kernel, whose
    groups take runs of up to 8 slabs, takes runs of 4 here (fewer than 8
    rounds of 1,536 resident groups, and more than 4 x 1,536 slabs).  Every
    element, 2 steps."""
    shapes = [(4096, 4096), (1_500_001,), (1031, 777), (3,)]
    w = inputs.custom(shapes, grad_kind="masked", seed=34)
    _flush("zip_sr runs of 4")
    rep = parity.run(w, "zip_sr", 2)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden"])
def test_zero_gradient_blocks(recipe):
    """A tensor whose gradient is exactly zero: scales stay 0, codes stay at
    the code of zero, weights only decay."""
    w = inputs.custom([(512,), (1000,)], grad_kind="masked", seed=22)
    orig = w.grads
    w.grads = lambda step, device="cpu", consts=None: [g * (0 if i == 0 else 1) for i, g in
                                                       enumerate(orig(step, device, consts))]
    rep = parity.run(w, recipe, 3)
    rep.check()


def test_lm_head_switch_final_phase():
    """ZIP-SR with the LM-head first moment switching to NF4-SR in the final
    10% of 10 steps (step 10 only)."""
    w = inputs.custom([(4096,), (64, 128), (32, 64)], grad_kind="masked", seed=23,
                      flags=[0, 0, q4.TF_LM_HEAD])
    rep = parity.run(w, "zip_sr", 10, lm_head_phase=True)
    rep.check()
    assert rep.codes_differ == 0


# Points of the hyper-parameter and seed space besides the workloads' own
# (lr 1e-3, betas (0.9, 0.999), eps 1e-8, wd 0.1, seed 0, eps_sr = eps):
# Philox keys with a non-zero high word, a separate eps_sr, other betas
# (beta1 = 0 included), no decay, other learning rates.
HP_GRID = [
    ("seed1", dict(seed=1)),
    ("seed9E3779B9", dict(seed=0x9E3779B9)),
    ("seed2^32+7", dict(seed=2 ** 32 + 7)),
    ("seed2^64-1", dict(seed=2 ** 64 - 1)),
    ("eps_sr1e-6", dict(eps_sr=1e-6, seed=5)),
    ("b0.9_0.95", dict(beta1=0.9, beta2=0.95, seed=3)),
    ("b0_0.99", dict(beta1=0.0, beta2=0.99, seed=4)),
    ("wd0", dict(weight_decay=0.0, seed=6)),
    ("lr1e-4", dict(lr=1e-4, seed=7)),
    ("lr3e-3", dict(lr=3e-3, seed=8)),
]
GRID_SHAPES = [(1,), (129,), (1000,), (4097,), (7, 129), (64, 520), (2, 1031)]


@pytest.mark.parametrize("hpk", [h for _, h in HP_GRID], ids=[n for n, _ in HP_GRID])
@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_hyperparameter_and_seed_grid(recipe, hpk):
    """Ragged tensors, one flagged as the LM head with its final-phase SR on
    the last step, 5 steps, every element, at each point of the grid."""
    w = inputs.custom(GRID_SHAPES, grad_kind="masked", seed=41,
                      flags=[0, 0, inputs.TF_LM_HEAD, 0, 0, 0, 0])
    _flush(f"grid {recipe} {hpk}")
    rep = parity.run(w, recipe, 5, hp=hpk, lm_head_phase=True)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("offset", [2 ** 32 - 3, 10 ** 6, 2 ** 40 + 5], ids=["2^32-3", "1e6", "2^40+5"])
@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored"])
def test_step_counts_past_the_counter_word(recipe, offset):
    """Steps offset+1 .. offset+5: the Philox counter takes the step's low
    32 bits (crossing 2^32 at the first offset), the bias correction the
    full count; the LM-head SR phase on the last step."""
    w = inputs.custom(GRID_SHAPES, grad_kind="masked", seed=42, flags=[0, 0, inputs.TF_LM_HEAD, 0, 0, 0, 0])
    _flush(f"steps from {offset} {recipe}")
    rep = parity.run(w, recipe, 5, hp=dict(seed=2 ** 64 - 1), lm_head_phase=True, step_offset=offset)
    rep.check()
    assert rep.codes_differ == 0


VARIANTS = parity.VARIANTS


@pytest.mark.parametrize("variant", VARIANTS)
def test_rule_and_codebook_variants(variant):
    """The component grid of the paper's Tables 1, 3 and 8 on the same kernel."""
    cfg = _variant_cfg(variant)
    w = inputs.custom([(3000,), (40, 300)], grad_kind="masked", seed=24)
    rep = parity.run(w, "custom", 6, cfg=cfg)
    rep.check()
    assert rep.codes_differ == 0


def _variant_cfg(variant):
    cfg = q4.q4adamw_default_config(q4.RECIPE_CUSTOM)
    cfg.m_codebook, cfg.v_codebook, cfg.m_rule, cfg.v_rule, cfg.eden = variant
    return cfg


@pytest.mark.parametrize("variant", VARIANTS)
def test_rule_and_codebook_variants_other_hyperparameters(variant):
    """The grid at another point of the hyper-parameter space: the all-ones
    seed, eps_sr = 1e-6, beta1 = 0, beta2 = 0.99, no decay, lr 3e-3, steps
    crossing 2^32."""
    cfg = _variant_cfg(variant)
    w = inputs.custom([(3000,), (40, 300)], grad_kind="masked", seed=43, flags=[inputs.TF_LM_HEAD, 0])
    hpk = dict(seed=2 ** 64 - 1, eps_sr=1e-6, beta1=0.0, beta2=0.99, weight_decay=0.0, lr=3e-3)
    _flush(f"variant {variant} other hparams")
    rep = parity.run(w, "custom", 6, cfg=cfg, hp=hpk, lm_head_phase=True, step_offset=2 ** 32 - 3)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("variant", VARIANTS)
def test_rule_and_codebook_variants_edge_magnitudes(variant):
    """The grid on the edge-magnitude blocks (subnormal scales, v below
    2^-96, signed zeros, underflowing squares), every element, 6 steps."""
    w = inputs.custom([(7 * 128 * 3 + 77,), (21, 140)], grad_kind="edge", seed=54)
    _flush(f"edge magnitudes variant {variant}")
    rep = parity.run(w, "custom", 6, cfg=_variant_cfg(variant))
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("variant", VARIANTS)
def test_rule_and_codebook_variants_gpt_162m_sampled(variant):
    """The grid on the GPT-style 162M set in the benchmark's launch
    configuration, 5 steps, on windows."""
    w = inputs.gpt_162m()
    wins = parity.sample_windows(w, n_random=16, seed=11)
    _flush(f"gpt-162m variant {variant}")
    rep = parity.run(w, "custom", 5, cfg=_variant_cfg(variant), windows=wins, grads_on="cuda",
                     check_every_step=False)
    rep.check()


def test_determinism_and_resume():
    """Two runs are bitwise equal; 3 steps, a state copy into fresh buffers,
    then 3 more steps equals 6 straight steps (the uniforms are keyed on the
    step, so resuming is exact)."""
    w = inputs.custom([(5000,), (64, 96)], grad_kind="masked", seed=25)
    dev = torch.device("cuda")
    consts = w._tensor_consts("cpu")
    grads = [[g.to(dev).reshape(-1).contiguous() for g in w.grads(s, "cpu", consts)] for s in range(1, 7)]

    def fresh():
        return [p.to(dev).reshape(-1).contiguous() for p in w.init_params("cpu")], q4.Q4State("zip_sr", w.tensors, dev)

    pa, sa = fresh()
    for s in range(1, 7):
        sa.step(pa, grads[s - 1], s, **w.hp)
    pb, sb = fresh()
    for s in range(1, 7):
        sb.step(pb, grads[s - 1], s, **w.hp)
    pc, sc = fresh()
    for s in range(1, 4):
        sc.step(pc, grads[s - 1], s, **w.hp)
    torch.cuda.synchronize()
    saved = [{f: getattr(b, f).clone() for f in ("m_codes", "m_scales", "v_codes", "v_scales")} for b in sc.bufs]
    hdr = q4.q4adamw_make_header(sc.cfg)
    _, sd = fresh()
    q4.q4adamw_check_header(sd.cfg, hdr)
    for b, s in zip(sd.bufs, saved):
        for f, x in s.items():
            getattr(b, f).copy_(x)
    for s in range(4, 7):
        sd.step(pc, grads[s - 1], s, **w.hp)
    torch.cuda.synchronize()
    for x, y, z in zip(pa, pb, pc):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(x.view(torch.int32), z.view(torch.int32))
    for a, b, d in zip(sa.bufs, sb.bufs, sd.bufs):
        for f in ("m_codes", "m_scales", "v_codes", "v_scales"):
            assert torch.equal(getattr(a, f), getattr(b, f))
            assert torch.equal(getattr(a, f), getattr(d, f))


@pytest.mark.parametrize("recipe,variant", [("zip_sr", None), ("ze_eden", None), ("factored", None)]
                         + [("custom", v) for v in parity.VARIANTS])
def test_dequant_matches_oracle(recipe, variant):
    w = inputs.custom([(3000,), (48, 200)], grad_kind="masked", seed=26)
    dev = torch.device("cuda")
    from oracle import oracle as O
    cfg = _variant_cfg(variant) if variant is not None else None
    params = w.init_params("cpu")
    consts = w._tensor_consts("cpu")
    gp = [p.to(dev).reshape(-1).contiguous() for p in params]
    st = q4.Q4State(recipe, w.tensors, dev, cfg=cfg)
    ost = [O.TensorState(parity.oracle_config(recipe, cfg), t.shape, t.tensor_id) for t in w.tensors]
    op = [p.numpy().reshape(-1).copy() for p in params]
    for s in range(1, 4):
        g = w.grads(s, "cpu", consts)
        st.step(gp, [x.to(dev).reshape(-1).contiguous() for x in g], s, **w.hp)
        for i, o in enumerate(ost):
            o.step(O.HParams(step=s, **w.hp), op[i], g[i].view(torch.uint16).numpy().reshape(-1).copy())
    for i, o in enumerate(ost):
        m, v = st.dequant(i)
        torch.cuda.synchronize()
        om, ov = o.dequant()
        assert np.array_equal(m.cpu().numpy().view(np.uint32), om.view(np.uint32))
        if recipe == "factored" and len(w.tensors[i].shape) > 1:
            assert np.allclose(v.cpu().numpy(), ov, rtol=1e-6, atol=0)
        else:
            assert np.array_equal(v.cpu().numpy().view(np.uint32), ov.view(np.uint32))


def test_gpt_162m_sampled_20_steps():
    """GPT-style 162M parameter set (tied embedding as written: 123.6M), both
    recipes, 20 steps, compared on windows: the first and last blocks of every
    tensor and random interior windows."""
    w = inputs.gpt_162m()
    wins = parity.sample_windows(w, n_random=32)
    for recipe in ("zip_sr", "ze_eden"):
        _flush(f"gpt-162m {recipe}")
        rep = parity.run(w, recipe, 20, windows=wins, grads_on="cuda", check_every_step=False)
        rep.check()


def test_llama_1_1b_sampled_lm_head_phase():
    """Llama-style 1.1B set, ZIP-SR, 10 steps, the LM-head first moment on
    NF4-SR in the final 10% (step 10); windows of every tensor."""
    w = inputs.llama_1_1b()
    wins = parity.sample_windows(w, n_random=48, seed=1)
    _flush("llama-1.1b zip_sr")
    rep = parity.run(w, "zip_sr", 10, windows=wins, grads_on="cuda", lm_head_phase=True, check_every_step=False)
    rep.check()


@pytest.mark.parametrize("recipe", ["ze_eden", "zip_sr"])
def test_gpt_2_7b_sampled(recipe):
    """GPT-style 2.7B set (all state resident in HBM), 10 steps, windows."""
    w = inputs.gpt_2_7b()
    wins = parity.sample_windows(w, n_random=48, seed=2)
    _flush(f"gpt-2.7b {recipe}")
    rep = parity.run(w, recipe, 10, windows=wins, grads_on="cuda", check_every_step=False)
    rep.check()


def test_qwen3_factored_full_rc():
    """Factored mode on the Qwen3-0.6B-shaped set (4 BF16 microbatches per
    step): the oracle recomputes every matrix's R and C from the full
    gradient each step; weights and m codes compared on windows."""
    w = inputs.qwen3_0_6b_factored()
    wins = parity.sample_windows(w, n_random=32, seed=3)
    _flush("qwen3-0.6b factored")
    rep = parity.run(w, "factored", 10, windows=wins, grads_on="cuda", check_every_step=False)
    rep.check()


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_edge_magnitudes(recipe):
    """Blocks whose v falls below 2^-96 (the square root's wave-level IEEE
    fallback), BF16-subnormal blocks (block scales below 2^-126: the
    reciprocal's division fallback, finite between 2^-128 and 2^-126 and
    overflowing below), signed zeros (the negative half of the
    flat bucket table), mixed zeros and large values, and squares that
    underflow; every element, 6 steps."""
    w = inputs.custom([(7 * 128 * 3 + 77,), (21, 140)], grad_kind="edge", seed=51)
    _flush(f"edge magnitudes {recipe}")
    rep = parity.run(w, recipe, 6)
    rep.check()
    assert rep.codes_differ == 0


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored"])
def test_edge_magnitudes_lm_head_phase(recipe):
    """The edge-magnitude blocks on a tensor flagged as the LM head, with the
    final-phase switch: its m takes state-space SR (Philox stream 0) on the
    last of 10 steps.  ZIP-SR finds the level through its flat table, the
    other recipes through the compact ones."""
    w = inputs.custom([(7 * 128 * 3 + 77,), (21, 140)], grad_kind="edge", seed=53, flags=[inputs.TF_LM_HEAD, 0])
    _flush(f"edge magnitudes {recipe} + LM-head phase")
    rep = parity.run(w, recipe, 10, lm_head_phase=True)
    rep.check()
    assert rep.codes_differ == 0


def test_factored_matrix_beyond_2_32_elements():
    """A factored matrix of 65,537 x 65,539 elements (4.3e9, past 2^32) and
    a vector: the fused step's 64-bit row division for chunks that start
    past 2^32, K2's row/column statistics over every element (R and C
    compared in full each step), codes and weights on windows around 2^31,
    2^32 and both ends."""
    rows, cols = 65537, 65539
    n = rows * cols
    w = inputs.custom([(rows, cols), (1000,)], grad_kind="masked", seed=28)
    nb = (n + 127) // 128
    lo32 = (1 << 32) // 128
    lo31 = (1 << 31) // 128
    wins = [(0, 0, 2), (0, lo31 - 2, lo31 + 2), (0, lo32 - 3, lo32 + 3), (0, nb - 3, nb), (1, 0, 8)]
    _flush("factored 65537 x 65539")
    rep = parity.run(w, "factored", 2, windows=wins, grads_on="cuda")
    rep.check()
    assert rep.codes_differ == 0


def test_tensor_beyond_2_32_elements():
    """One tensor of 2^32 + 1000 elements (17 GB of FP32 masters): 64-bit
    element indices, Philox counters past 2^32 / 4, a ragged last block."""
    n = (1 << 32) + 1000
    w = inputs.custom([(n,)], grad_kind="masked", seed=27)
    nb = (n + 127) // 128
    lo32 = (1 << 32) // 128
    lo31 = (1 << 31) // 128
    wins = [(0, 0, 2), (0, lo31 - 2, lo31 + 2), (0, lo32 - 3, lo32 + 3), (0, nb - 3, nb)]
    _flush("2^32 + 1000 elements zip_sr")
    rep = parity.run(w, "zip_sr", 2, windows=wins, grads_on="cuda")
    rep.check()
    assert rep.codes_differ == 0
