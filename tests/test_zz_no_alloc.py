"""q4adamw_step_noalloc, the step for callers that cannot allocate: its
workspace is the library's static device scratch.  Through the C ABI it must
give exactly the bits q4adamw_step gives with a workspace of its own, on
calls in a row whose tensor lists differ (the second smaller: the scratch
keeps the first call's contents), with clipping (the statistics and the clip
factor live in the scratch) and on the factored recipe (its row/column
partial sums live there too).  A list whose workspace exceeds the scratch is
refused before any device work."""
import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import api, inputs

SCRATCH = 32 << 20
BIG = [(5000,), (64, 520), (4097,), (7, 129), (1,), (300, 3)]
SMALL = [(129,), (5, 40)]


def _same(pa, sa, pb, sb, what):
    for i, (x, y) in enumerate(zip(pa, pb)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"{what}: tensor {i} weights"
    for i, (a, b) in enumerate(zip(sa.bufs, sb.bufs)):
        for f in ("m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col", "m32", "v32"):
            x, y = getattr(a, f), getattr(b, f)
            if x is not None:
                assert np.array_equal(x.cpu().numpy().view(np.uint8), y.cpu().numpy().view(np.uint8)), \
                    f"{what}: tensor {i} {f}"


@pytest.mark.gpu
@pytest.mark.parametrize("recipe,clip", [("zip_sr", 0.0), ("zip_sr", 0.05), ("ze_eden", 0.0), ("factored", 0.0),
                                         ("factored", 0.05), ("block8", 0.0), ("fp32", 0.0)])
def test_noalloc_equals_step_on_two_calls_the_second_smaller(recipe, clip):
    dev = torch.device("cuda")
    print(f"noalloc {recipe} clip {clip}", flush=True)
    for k, shapes in enumerate((BIG, SMALL)):
        w = inputs.custom(shapes, grad_kind="masked", seed=90 + k)
        consts = w._tensor_consts("cpu")
        pa = [p.to(dev).reshape(-1).contiguous() for p in w.init_params("cpu")]
        pb = [p.clone() for p in pa]
        sa = q4.Q4State(recipe, w.tensors, dev)
        sb = q4.Q4State(recipe, w.tensors, dev)
        for s in (1, 2):
            g = [x.to(dev).reshape(-1).contiguous() for x in w.grads(s, "cpu", consts)]
            sa.step(pa, g, s, max_grad_norm=clip, **w.hp)
            sb.step_noalloc(pb, g, s, max_grad_norm=clip, **w.hp)
            torch.cuda.synchronize()
            _same(pa, sa, pb, sb, f"{recipe} list {k} step {s}")


def _desc(shapes):
    out = []
    for i, shp in enumerate(shapes):
        t = api.Q4Tensor()
        t.tensor_id = i
        t.ndim = len(shp)
        n = 1
        for d, x in enumerate(shp):
            t.shape[d] = x
            n *= x
        t.numel = n
        # plausible 16-byte-aligned addresses: refused before any is used
        for j, f in enumerate(("param", "grad", "m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col")):
            setattr(t, f, 0x10000000 * (j + 1) + 0x100000 * i)
        out.append(t)
    return out


def test_a_list_beyond_the_scratch_is_refused_before_any_device_work():
    """The factored GPT-2.7B list needs 118 MiB of row/column partials: the
    call returns Q4_ERR_WORKSPACE, naming both sizes (no device is touched,
    so this runs without a GPU)."""
    w = inputs.gpt_2_7b()
    cfg = api.q4adamw_default_config(api.RECIPE_FACTORED)
    desc = _desc([t.shape for t in w.tensors])
    need = api.q4adamw_workspace_bytes(cfg, desc)
    assert need > SCRATCH
    hp = api.Q4HParams(1e-3, 0.9, 0.999, 1e-8, 0.1, 0.0, 1, 0, 0, 0, 0.0, 0)
    with pytest.raises(api.Q4Error) as e:
        api.q4adamw_step_noalloc(cfg, hp, desc, 0)
    assert e.value.status == 7 and str(need) in str(e.value) and str(SCRATCH) in str(e.value)
    # the packed recipes' lists are small (128 bytes of table per tensor)
    for rec in (api.RECIPE_ZIP_SR, api.RECIPE_ZE_EDEN, api.RECIPE_BLOCK8):
        assert api.q4adamw_workspace_bytes(api.q4adamw_default_config(rec), desc) < SCRATCH
