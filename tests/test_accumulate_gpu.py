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


def setup(recipe, seed=31):
    w = inputs.custom(SHAPES, grad_kind="masked", seed=seed)
    dev = torch.device("cuda")
    st = q4.Q4State(recipe, w.tensors, dev)
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


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "fp32"])
def test_clipped_steps_match_oracle(recipe):
    """Five steps, each: four microbatches accumulated on the GPU, then a step
    with the statistics of the last pass and clipping to a norm below the
    gradients' (so every step clips)."""
    w, st, params, grads, offsets, total = setup(recipe, seed=32)
    _flush(f"clipped steps {recipe}")
    ocfg = parity.oracle_config(recipe)
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
        scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
        assert (np.abs(p - ref) / scale).max() <= parity.W_TOL, f"tensor {i} weights"
        if recipe == "fp32":
            continue
        assert np.array_equal(b.m_codes.cpu().numpy(), o.m_codes), f"tensor {i} m codes"
        assert np.array_equal(b.m_scales.cpu().numpy().view(np.uint32), o.m_scales.view(np.uint32))
        if b.v_codes is not None:
            assert np.array_equal(b.v_codes.cpu().numpy(), o.v_codes), f"tensor {i} v codes"
            assert np.array_equal(b.v_scales.cpu().numpy().view(np.uint32), o.v_scales.view(np.uint32))
        else:
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
