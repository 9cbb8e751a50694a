"""GPU parity of the step before ([A] "State representation": BF16
microbatch accumulation into the gradient buffers, the gradient norm and
clipping on them) against the CPU oracle on the same seeded bytes.

Accumulated gradients must match bit for bit; the global norm is a binary64
sum in another order on each side, so it matches to 1e-12 and the FP32 clip
factor derived from it matches bit for bit (a flip would need the factor to
sit within ~1e-16 of an FP32 rounding boundary).  Clipped steps then keep
the step's own bar: codes and scales bit-exact, weights within 1e-6, factored
R and C within 1e-6."""
import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import inputs
from oracle import oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

SHAPES = [(1000,), (64, 520), (7, 129), (4096,), (300, 3), (512, 256)]
# with tensors of no elements first, between others and last
SHAPES_WITH_EMPTY = [(0,), (1000,), (0,), (64, 520), (0, 5), (7, 129), (0,)]
K = 4  # microbatches per step


def _flush(msg):
    print(msg, flush=True)


def microbatches(w, step, offsets, total, seed=0):
    """K flat BF16 microbatch buffers (host uint16) of the workload's tensors:
    Student-t draws scaled per tensor, a fresh draw per microbatch."""
    g = torch.Generator().manual_seed(1000 * seed + step)
    out = []
    for k in range(K):
        flat = np.zeros(total, np.uint16)
        for i, t in enumerate(w.tensors):
            z = torch.randn(t.numel, generator=g) / torch.sqrt(
                (torch.randn(t.numel, generator=g) ** 2 + torch.randn(t.numel, generator=g) ** 2
                 + torch.randn(t.numel, generator=g) ** 2) / 3)
            b = (z * (1e-3 * (1 + i % 3))).to(torch.bfloat16).view(torch.uint16).numpy()
            flat[offsets[i]: offsets[i] + t.numel] = b
        out.append(flat)
    return out


def host_accumulate(w, micro, offsets):
    acc = [np.zeros(t.numel, np.uint16) for t in w.tensors]
    for k, flat in enumerate(micro):
        for i, t in enumerate(w.tensors):
            O.accumulate_bf16(acc[i], flat[offsets[i]: offsets[i] + t.numel].copy(), first=(k == 0))
    return acc


def setup(recipe, seed=31, shapes=SHAPES, cfg=None):
    w = inputs.custom(shapes, grad_kind="masked", seed=seed)
    dev = torch.device("cuda")
    st = q4.Q4State(recipe, w.tensors, dev, cfg=cfg)
    params = [p.to(dev).reshape(-1).contiguous() for p in w.init_params("cpu")]
    grads = [torch.full((t.numel,), 7.0, dtype=torch.bfloat16, device=dev) for t in w.tensors]  # stale values
    offsets, total = st.flat_offsets()
    return w, st, params, grads, offsets, total


@pytest.mark.parametrize("recipe", ["zip_sr", "factored"])
def test_accumulation_and_norm_match_oracle(recipe):
    w, st, params, grads, offsets, total = setup(recipe)
    _flush(f"accumulate {recipe}")
    micro = microbatches(w, 1, offsets, total)
    for k, flat in enumerate(micro):
        m = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
        st.accumulate(params, grads, m, first=(k == 0), last=(k == K - 1))
    norm = st.grad_norm()
    acc = host_accumulate(w, micro, offsets)
    for i in range(len(w.tensors)):
        assert np.array_equal(grads[i].view(torch.uint16).cpu().numpy(), acc[i]), f"tensor {i}"
    ref = np.sqrt(sum(O.grad_sumsq(a) for a in acc))
    assert abs(norm - ref) <= 1e-12 * ref
    # the statistics pass on the accumulated gradients gives the same norm
    st.grad_stats(params, grads)
    assert abs(st.grad_norm() - ref) <= 1e-12 * ref


@pytest.mark.parametrize("recipe", ["zip_sr", "factored"])
def test_mid_size_accumulation_and_norm(recipe):
    """About 10.2 M elements: the accumulation pass takes one work-group per
    run of 2 slabs (about 2,500 partial sums, totalled in two stages); the
    factored recipe's matrices go through the tile pass instead, the vector
    through the chunk pass."""
    shapes = [(1024, 4096), (2048, 2048), (1_000_003,), (777, 1031), (4097,)]
    w, st, params, grads, offsets, total = setup(recipe, seed=35, shapes=shapes)
    _flush(f"accumulate mid-size {recipe}")
    micro = microbatches(w, 2, offsets, total)
    for k, flat in enumerate(micro):
        m = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
        st.accumulate(params, grads, m, first=(k == 0), last=(k == len(micro) - 1))
    norm = st.grad_norm()
    acc = host_accumulate(w, micro, offsets)
    for i in range(len(w.tensors)):
        assert np.array_equal(grads[i].view(torch.uint16).cpu().numpy(), acc[i]), f"tensor {i}"
    ref = np.sqrt(sum(O.grad_sumsq(a) for a in acc))
    assert abs(norm - ref) <= 1e-12 * ref


def _variant_cfg(variant):
    cfg = q4.q4adamw_default_config(q4.RECIPE_CUSTOM)
    cfg.m_codebook, cfg.v_codebook, cfg.m_rule, cfg.v_rule, cfg.eden = variant
    return cfg


CLIP_CASES = [("zip_sr", SHAPES, None), ("ze_eden", SHAPES, None), ("factored", SHAPES, None), ("fp32", SHAPES, None),
              ("zip_sr", SHAPES_WITH_EMPTY, None), ("factored", SHAPES_WITH_EMPTY, None)]
# the clipped kernel of every codebook/rule variant
CLIP_CASES += [("custom", SHAPES, v) for v in parity.VARIANTS]


@pytest.mark.parametrize("recipe,shapes,variant", CLIP_CASES)
def test_clipped_steps_match_oracle(recipe, shapes, variant):
    """Five steps, each: four microbatches accumulated on the GPU, then a step
    with the statistics of the last pass and clipping to a norm below the
    gradients' (so every step clips)."""
    cfg = _variant_cfg(variant) if variant is not None else None
    w, st, params, grads, offsets, total = setup(recipe, seed=32, shapes=shapes, cfg=cfg)
    _flush(f"clipped steps {recipe} {variant} {len(shapes)} tensors")
    ocfg = parity.oracle_config(recipe, cfg)
    ost = [O.TensorState(ocfg, t.shape, t.tensor_id, t.flags) for t in w.tensors]
    op = [p.cpu().numpy().copy() for p in params]
    max_norm = 2e-3
    for s in range(1, 6):
        micro = microbatches(w, s, offsets, total, seed=2)
        for k, flat in enumerate(micro):
            m = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
            st.accumulate(params, grads, m, first=(k == 0), last=(k == K - 1))
        st.step(params, grads, s, grad_stats=True, max_grad_norm=max_norm, **w.hp)
        acc = host_accumulate(w, micro, offsets)
        c = O.clip_factor(sum(O.grad_sumsq(a) for a in acc), max_norm)
        assert c < 1.0
        gpu_c = float(st.ws[8:12].view(torch.float32).cpu()[0])
        assert np.float32(gpu_c).view(np.uint32) == np.float32(c).view(np.uint32), (gpu_c, c)
        hp = O.HParams(step=s, grad_scale=c, **w.hp)
        for i, o in enumerate(ost):
            o.step(hp, op[i], acc[i])
    torch.cuda.synchronize()
    for i, (b, o) in enumerate(zip(st.bufs, ost)):
        ref = op[i]
        p = params[i].cpu().numpy()
        if ref.size:
            scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
            assert (np.abs(p - ref) / scale).max() <= parity.W_TOL, f"tensor {i} weights"
        if recipe == "fp32":
            continue
        assert np.array_equal(b.m_codes.cpu().numpy(), o.m_codes), f"tensor {i} m codes"
        assert np.array_equal(b.m_scales.cpu().numpy().view(np.uint32), o.m_scales.view(np.uint32))
        if b.v_codes is not None:
            assert np.array_equal(b.v_codes.cpu().numpy(), o.v_codes), f"tensor {i} v codes"
            assert np.array_equal(b.v_scales.cpu().numpy().view(np.uint32), o.v_scales.view(np.uint32))
        elif b.numel > 0:  # a matrix with no elements keeps no statistics
            for x, y in ((b.v_row, o.R), (b.v_col, o.Cc)):
                x = x.cpu().numpy()
                assert np.allclose(x, y, rtol=parity.RC_TOL, atol=0), f"tensor {i} R/C"


@pytest.mark.parametrize("recipe", ["ze_eden", "factored"])
def test_statistics_inside_the_step_equal_the_accumulated_ones(recipe):
    """A clipped step that gathers its own statistics equals one that takes
    them from the accumulation pass, and a factored step that reuses the
    accumulation's row/column partials equals one that gathers them (no
    clipping): bit for bit on the GPU."""
    results = []
    for mode in ("inside", "accumulated"):
        w, st, params, grads, offsets, total = setup(recipe, seed=33)
        for s in range(1, 4):
            micro = microbatches(w, s, offsets, total, seed=3)
            for k, flat in enumerate(micro):
                m = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
                st.accumulate(params, grads, m, first=(k == 0), last=(mode == "accumulated" and k == K - 1))
            st.step(params, grads, s, grad_stats=(mode == "accumulated"), max_grad_norm=2e-3 if s < 3 else 0.0,
                    **w.hp)
        torch.cuda.synchronize()
        results.append((params, st))
    (pa, sa), (pb, sb) = results
    for x, y in zip(pa, pb):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    for a, b in zip(sa.bufs, sb.bufs):
        for f in ("m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col"):
            if getattr(a, f) is not None:
                assert torch.equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("recipe", ["zip_sr", "factored"])
def test_single_microbatch_is_first_and_last(recipe):
    """One microbatch per step (first and last in one call): the gradients
    equal the microbatch, the norm the oracle's, and the clipped steps that
    reuse these statistics equal steps that gather their own, bit for bit.
    For the factored matrices this is the tile kernel's copying mode."""
    results = []
    for mode in ("accumulated", "inside"):
        w, st, params, grads, offsets, total = setup(recipe, seed=34)
        for s in range(1, 4):
            flat = microbatches(w, s, offsets, total, seed=4)[0]
            m = torch.from_numpy(flat.view(np.int16)).view(torch.bfloat16).cuda()
            st.accumulate(params, grads, m, first=True, last=(mode == "accumulated"))
            if mode == "accumulated":
                for i, t in enumerate(w.tensors):
                    assert np.array_equal(grads[i].view(torch.uint16).cpu().numpy(),
                                          flat[offsets[i]: offsets[i] + t.numel]), f"step {s} tensor {i}"
                ref = np.sqrt(sum(O.grad_sumsq(flat[offsets[i]: offsets[i] + t.numel].copy())
                                  for i, t in enumerate(w.tensors)))
                assert abs(st.grad_norm() - ref) <= 1e-12 * ref
            st.step(params, grads, s, grad_stats=(mode == "accumulated"), max_grad_norm=2e-3, **w.hp)
        torch.cuda.synchronize()
        results.append((params, st))
    (pa, sa), (pb, sb) = results
    for x, y in zip(pa, pb):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    for a, b in zip(sa.bufs, sb.bufs):
        for f in ("m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col"):
            if getattr(a, f) is not None:
                assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_gpt_2_7b_accumulation_and_clipped_step_sampled():
    """The GPT-style 2.7B set in the launch configuration the benchmark times
    for the step before: one accumulation pass with the statistics, then a
    clipped ZIP-SR step that reuses them.  Accumulated gradients on sampled
    windows bit for bit; the norm against a float64 sum of every accumulated
    gradient (an independent reduction, 1e-12); the clip factor bit for bit;
    the step's codes, scales and weights on the windows."""
    w = inputs.gpt_2_7b()
    dev = torch.device("cuda")
    st = q4.Q4State("zip_sr", w.tensors, dev)
    params = [p.reshape(-1) for p in w.init_params(dev)]
    consts = w._tensor_consts(dev)
    grads = [g.reshape(-1).contiguous() for g in w.grads(1, dev, consts)]
    offsets, total = st.flat_offsets()
    micro = torch.zeros(total, dtype=torch.bfloat16, device=dev)
    for i, g in enumerate(w.grads(2, dev, consts)):
        micro[offsets[i]: offsets[i] + g.numel()].copy_(g.reshape(-1))
    del consts
    wins = parity.sample_windows(w, n_random=32, seed=8)
    ocfg = parity.oracle_config("zip_sr")
    host = []
    for i, b0, b1 in wins:
        t = w.tensors[i]
        lo, hi = 128 * b0, min(128 * b1, t.numel)
        n = hi - lo
        zm, zv = O.zero_code(ocfg.m_cb), O.zero_code(ocfg.v_cb)
        win = dict(i=i, b0=b0, b1=b1, lo=lo, hi=hi, param=params[i][lo:hi].cpu().numpy().copy(),
                   g0=grads[i][lo:hi].view(torch.uint16).cpu().numpy().copy(),
                   mic=micro[offsets[i] + lo: offsets[i] + hi].view(torch.uint16).cpu().numpy().copy(),
                   m_codes=np.full((n + 1) // 2, zm | (zm << 4), np.uint8), m_scales=np.zeros(b1 - b0, np.float32),
                   v_codes=np.full((n + 1) // 2, zv | (zv << 4), np.uint8), v_scales=np.zeros(b1 - b0, np.float32))
        if n % 2:
            win["m_codes"][-1], win["v_codes"][-1] = zm, zv
        host.append(win)
    _flush("gpt-2.7b accumulate + clipped zip_sr step")
    st.accumulate(params, grads, micro, first=False, last=True)
    norm = st.grad_norm()
    ref_sq = sum(float((g.double() ** 2).sum()) for g in grads)
    assert abs(norm - np.sqrt(ref_sq)) <= 1e-12 * np.sqrt(ref_sq)
    for h in host:
        acc = h["g0"].copy()
        O.accumulate_bf16(acc, h["mic"], first=False)
        got = grads[h["i"]][h["lo"]:h["hi"]].view(torch.uint16).cpu().numpy()
        assert np.array_equal(got, acc), f"tensor {h['i']} accumulated gradients"
        h["acc"] = acc
    max_norm = 0.5 * norm
    st.step(params, grads, 1, grad_stats=True, max_grad_norm=max_norm, **w.hp)
    c = O.clip_factor(ref_sq, max_norm)
    gpu_c = float(st.ws[8:12].view(torch.float32).cpu()[0])
    assert np.float32(gpu_c).view(np.uint32) == np.float32(c).view(np.uint32), (gpu_c, c)
    hp = O.HParams(step=1, grad_scale=c, **w.hp)
    torch.cuda.synchronize()
    for h in host:
        t = w.tensors[h["i"]]
        O.step_window(ocfg, hp, tensor_id=t.tensor_id, flags=t.flags, numel=t.numel, base=h["lo"], param=h["param"],
                      grad=h["acc"], m_codes=h["m_codes"], m_scales=h["m_scales"], v_codes=h["v_codes"],
                      v_scales=h["v_scales"])
        b = st.bufs[h["i"]]
        cl, ch = h["lo"] // 2, (h["hi"] + 1) // 2
        for mine, ref in ((b.m_codes, h["m_codes"]), (b.v_codes, h["v_codes"])):
            assert np.array_equal(parity.unpack(mine[cl:ch].cpu().numpy())[:h["hi"] - h["lo"]],
                                  parity.unpack(ref)[:h["hi"] - h["lo"]]), f"tensor {h['i']} codes"
        for mine, ref in ((b.m_scales, h["m_scales"]), (b.v_scales, h["v_scales"])):
            assert np.array_equal(mine[h["b0"]:h["b1"]].cpu().numpy().view(np.uint32), ref.view(np.uint32))
        p = params[h["i"]][h["lo"]:h["hi"]].cpu().numpy()
        ref = h["param"]
        scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
        assert (np.abs(p - ref) / scale).max() <= parity.W_TOL, f"tensor {h['i']} weights"


def test_qwen3_factored_step_from_accumulated_statistics():
    """The Qwen3-0.6B-shaped factored set in the benchmark's launch
    configuration: one accumulation pass leaves the row/column partials, and
    the step that reuses them (no second gradient read) gives every matrix's
    R and C within 1e-6 of the oracle's full recomputation from the
    accumulated gradients; m codes, scales and weights on sampled windows."""
    w = inputs.qwen3_0_6b_factored()
    dev = torch.device("cuda")
    st = q4.Q4State("factored", w.tensors, dev)
    params = [p.reshape(-1) for p in w.init_params(dev)]
    consts = w._tensor_consts(dev)
    grads = [g.reshape(-1).contiguous() for g in w.grads(1, dev, consts)]
    offsets, total = st.flat_offsets()
    micro = torch.zeros(total, dtype=torch.bfloat16, device=dev)
    for i, g in enumerate(w.grads(2, dev, consts)):
        micro[offsets[i]: offsets[i] + g.numel()].copy_(g.reshape(-1))
    del consts
    wins = parity.sample_windows(w, n_random=24, seed=9)
    ocfg = parity.oracle_config("factored")
    p0 = {i: params[i].cpu().numpy().copy() for i in {i for i, _, _ in wins}}
    _flush("qwen3-0.6b factored step from accumulated statistics")
    st.accumulate(params, grads, micro, first=False, last=True)
    st.step(params, grads, 1, grad_stats=True, **w.hp)
    torch.cuda.synchronize()
    hp = O.HParams(step=1, **w.hp)
    fact = {}
    max_rc = 0.0
    for i, t in enumerate(w.tensors):
        if len(t.shape) < 2:
            continue
        g = grads[i].view(torch.uint16).cpu().numpy()
        rows, cols = t.shape[0], t.numel // t.shape[0]
        R, Cc = np.zeros(rows, np.float32), np.zeros(cols, np.float32)
        inv = O.factored_update(hp, rows, cols, g, R, Cc)
        fact[i] = (R, Cc, inv)
        b = st.bufs[i]
        for mine, ref in ((b.v_row, R), (b.v_col, Cc)):
            x = mine.cpu().numpy().astype(np.float64)
            r = ref.astype(np.float64)
            max_rc = max(max_rc, float((np.abs(x - r) / np.maximum(np.abs(r), 1e-30)).max()))
    assert max_rc <= parity.RC_TOL, max_rc
    for i, b0, b1 in wins:
        t = w.tensors[i]
        lo, hi = 128 * b0, min(128 * b1, t.numel)
        n = hi - lo
        zm = O.zero_code(ocfg.m_cb)
        mc = np.full((n + 1) // 2, zm | (zm << 4), np.uint8)
        if n % 2:
            mc[-1] = zm
        ms = np.zeros(b1 - b0, np.float32)
        kw = dict(tensor_id=t.tensor_id, flags=t.flags, numel=t.numel, base=lo, param=p0[i][lo:hi].copy(),
                  grad=grads[i][lo:hi].view(torch.uint16).cpu().numpy().copy(), m_codes=mc, m_scales=ms)
        if i in fact:
            R, Cc, inv = fact[i]
            kw.update(cols=t.numel // t.shape[0], R=R, Cc=Cc, inv_meanR=inv)
        else:
            zv = O.zero_code(ocfg.v_cb)
            vc = np.full((n + 1) // 2, zv | (zv << 4), np.uint8)
            if n % 2:
                vc[-1] = zv
            kw.update(v_codes=vc, v_scales=np.zeros(b1 - b0, np.float32))
        O.step_window(ocfg, hp, **kw)
        b = st.bufs[i]
        cl, ch = lo // 2, (hi + 1) // 2
        assert np.array_equal(parity.unpack(b.m_codes[cl:ch].cpu().numpy())[:n], parity.unpack(mc)[:n]), f"tensor {i}"
        assert np.array_equal(b.m_scales[b0:b1].cpu().numpy().view(np.uint32), ms.view(np.uint32))
        if i not in fact:
            assert np.array_equal(parity.unpack(b.v_codes[cl:ch].cpu().numpy())[:n], parity.unpack(kw["v_codes"])[:n])
        p = params[i][lo:hi].cpu().numpy()
        ref = kw["param"]
        scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
        assert (np.abs(p - ref) / scale).max() <= parity.W_TOL, f"tensor {i} weights"
