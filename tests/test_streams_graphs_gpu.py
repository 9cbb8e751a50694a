"""The step as a caller's training loop would run it: on a stream other than
the default one, and captured once in a HIP graph and replayed.  The step
enqueues kernels only (after the first call the tensor table stays in the
workspace), so both must give the same bits as eager steps on the default
stream."""
import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import inputs

pytestmark = pytest.mark.gpu

SHAPES = [(1000,), (64, 520), (4097,), (7, 129)]


def _flush(msg):
    print(msg, flush=True)


def _make(w, recipe, dev):
    params = [p.to(dev).reshape(-1).contiguous() for p in w.init_params("cpu")]
    return params, q4.Q4State(recipe, w.tensors, dev)


def _same(pa, sa, pb, sb, what):
    for i, (x, y) in enumerate(zip(pa, pb)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"{what}: tensor {i} weights"
    for i, (a, b) in enumerate(zip(sa.bufs, sb.bufs)):
        for f in ("m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col", "m32", "v32"):
            x, y = getattr(a, f), getattr(b, f)
            if x is not None:
                assert np.array_equal(x.cpu().numpy().view(np.uint8), y.cpu().numpy().view(np.uint8)), \
                    f"{what}: tensor {i} {f}"


@pytest.mark.parametrize("recipe", ["zip_sr", "ze_eden", "factored", "block8"])
def test_step_on_a_side_stream(recipe):
    w = inputs.custom(SHAPES, grad_kind="masked", seed=25)
    dev = torch.device("cuda")
    consts = w._tensor_consts("cpu")
    pa, sa = _make(w, recipe, dev)
    pb, sb = _make(w, recipe, dev)
    side = torch.cuda.Stream()  # default priority
    _flush(f"side stream {recipe}")
    for s in (1, 2, 3):
        grads = [g.to(dev).reshape(-1).contiguous() for g in w.grads(s, "cpu", consts)]
        sa.step(pa, grads, s, **w.hp)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sb.step(pb, grads, s, **w.hp)
        torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _same(pa, sa, pb, sb, f"{recipe} side stream")


@pytest.mark.parametrize("recipe", ["zip_sr", "factored"])
def test_step_in_a_hip_graph_replays_like_eager(recipe):
    """Two eager steps fill the launch caches and the workspace's tensor
    table; step 3 is then captured and replayed three times, each replay
    followed by the same eager step on a twin state, a synchronization and
    a comparison of every buffer."""
    w = inputs.custom(SHAPES, grad_kind="masked", seed=26)
    dev = torch.device("cuda")
    consts = w._tensor_consts("cpu")
    grads = [g.to(dev).reshape(-1).contiguous() for g in w.grads(1, "cpu", consts)]
    pa, sa = _make(w, recipe, dev)
    pb, sb = _make(w, recipe, dev)
    for s in (1, 2):
        sa.step(pa, grads, s, **w.hp)
        sb.step(pb, grads, s, **w.hp)
    torch.cuda.synchronize()
    _flush(f"graph capture {recipe}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sb.step(pb, grads, 3, **w.hp)
    torch.cuda.synchronize()
    _same(pa, sa, pb, sb, f"{recipe} after capture (nothing ran)")
    for r in range(3):
        graph.replay()
        sa.step(pa, grads, 3, **w.hp)
        torch.cuda.synchronize()
        _same(pa, sa, pb, sb, f"{recipe} replay {r}")


def test_pointer_checks_refuse_host_memory_before_any_work():
    """With Q4_HP_CHECK_POINTERS a step whose master weights live in host
    memory is refused (Q4_ERR_DEVICE) before anything is enqueued: a twin
    state that never saw the refused call stays bit-identical."""
    w = inputs.custom([(1000,), (64, 130)], grad_kind="masked", seed=29)
    dev = torch.device("cuda")
    consts = w._tensor_consts("cpu")
    pa, sa = _make(w, "zip_sr", dev)
    pb, sb = _make(w, "zip_sr", dev)
    g1 = [g.to(dev).reshape(-1).contiguous() for g in w.grads(1, "cpu", consts)]
    sa.step(pa, g1, 1, flags=q4.HP_CHECK_POINTERS, **w.hp)
    sb.step(pb, g1, 1, **w.hp)
    torch.cuda.synchronize()
    # pinned host memory: refused by the check as host memory, and harmless
    # host RAM (not an unmapped page) should the check ever let it through
    host = [pb[0].cpu().pin_memory(), pb[1]]
    with pytest.raises(q4.Q4Error) as e:
        sb.step(host, g1, 2, flags=q4.HP_CHECK_POINTERS, **w.hp)
    assert e.value.status == 6
    g2 = [g.to(dev).reshape(-1).contiguous() for g in w.grads(2, "cpu", consts)]
    sa.step(pa, g2, 2, **w.hp)
    sb.step(pb, g2, 2, **w.hp)
    torch.cuda.synchronize()
    _same(pa, sa, pb, sb, "after a refused call")


@pytest.mark.parametrize("recipe", ["zip_sr", "factored"])
def test_capture_refuses_a_table_upload(recipe):
    """A step whose tensor table is not yet in the workspace needs a host
    upload, which a graph cannot replay safely: under capture it is refused
    (Q4_ERR_INVALID_ARG) before anything is recorded.  The capture is ended
    and never replayed; the state is untouched, and the same step then runs
    eagerly and equals a twin's."""
    w = inputs.custom(SHAPES, grad_kind="masked", seed=27)
    dev = torch.device("cuda")
    consts = w._tensor_consts("cpu")
    grads = [g.to(dev).reshape(-1).contiguous() for g in w.grads(1, "cpu", consts)]
    pa, sa = _make(w, recipe, dev)
    pb, sb = _make(w, recipe, dev)      # never stepped: its workspace holds no table
    torch.cuda.synchronize()
    _flush(f"capture refusal {recipe}")
    graph = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(graph):
        try:
            sb.step(pb, grads, 1, **w.hp)
        except q4.Q4Error as e:
            refused = e
    torch.cuda.synchronize()
    assert refused is not None and refused.status == 1, refused
    _same(pa, sa, pb, sb, f"{recipe} after the refused capture")
    sa.step(pa, grads, 1, **w.hp)
    sb.step(pb, grads, 1, **w.hp)
    torch.cuda.synchronize()
    _same(pa, sa, pb, sb, f"{recipe} eager after the refusal")
