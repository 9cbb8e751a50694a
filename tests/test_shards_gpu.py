"""Data-parallel shards on one GPU.  A data-parallel rank owns a share of
each tensor (ZeRO style): a run of whole 128-blocks starting on a
512-element boundary, passed through the C
ABI as a tensor of its own with every pointer advanced to its first block
and elem_offset set, so that the stochastic-rounding draws use the index in
the whole tensor.  Stepping the shards (all in one call, or one call per
shard as separate ranks would) must give bit for bit the weights, codes and
scales of the whole-tensor step, which the parity tests hold against the
oracle.  What is left out on one GPU are the collectives around the step."""
import ctypes

import numpy as np
import pytest
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import api, inputs

pytestmark = pytest.mark.gpu

SHAPES = [(5000,), (64, 300), (1,), (129,), (4097,)]
# shard boundaries (elements) per tensor, multiples of 512; the last shard
# ends the tensor
CUTS = [[0, 512 * 3, 512 * 7, 5000], [0, 512 * 19, 19200], [0, 1], [0, 129],
        [0, 512 * 2, 512 * 3, 512 * 7, 4097]]
HP = dict(lr=3e-3, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.1, eps_sr=1e-6, seed=2 ** 64 - 1)


def _custom(m_cb, v_cb, m_rule, v_rule, eden):
    cfg = q4.q4adamw_default_config(q4.RECIPE_CUSTOM)
    cfg.m_codebook, cfg.v_codebook, cfg.m_rule, cfg.v_rule, cfg.eden = m_cb, v_cb, m_rule, v_rule, eden
    return cfg


CASES = {
    "zip_sr": ("zip_sr", None),
    "ze_eden": ("ze_eden", None),
    "block8": ("block8", None),
    "fp32": ("fp32", None),
    # m by state-space SR on every tensor: the m stream's draws too
    "m_state_sr": ("custom", _custom(q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_SR, q4.RULE_UPDATE_SR, 0)),
}


def _shard(t: api.Q4Tensor, lo: int, hi: int, byte_codes: bool) -> api.Q4Tensor:
    """Blocks [lo/128, ...) of tensor t as a tensor of its own."""
    s = api.Q4Tensor()
    ctypes.memmove(ctypes.addressof(s), ctypes.addressof(t), ctypes.sizeof(t))
    s.ndim = 1
    for d in range(len(s.shape)):
        s.shape[d] = 0
    s.shape[0] = hi - lo
    s.numel = hi - lo
    s.elem_offset = lo

    def adv(name, nbytes):
        p = getattr(t, name)
        setattr(s, name, p + nbytes if p else None)

    adv("param", 4 * lo)
    adv("grad", 2 * lo)
    adv("m_codes", lo if byte_codes else lo // 2)
    adv("v_codes", lo if byte_codes else lo // 2)
    adv("m_scales", 4 * (lo // 128))
    adv("v_scales", 4 * (lo // 128))
    adv("m_fp32", 4 * lo)
    adv("v_fp32", 4 * lo)
    return s


def _state(st):
    out = []
    for b in st.bufs:
        for f in ("m_codes", "m_scales", "v_codes", "v_scales", "m32", "v32"):
            x = getattr(b, f)
            if x is not None:
                out.append((f, x.cpu().numpy().view(np.uint8).copy()))
    return out


@pytest.mark.parametrize("separate_calls", [False, True], ids=["one_call", "call_per_shard"])
@pytest.mark.parametrize("case", list(CASES))
def test_shards_equal_the_whole_tensor(case, separate_calls):
    recipe, cfg = CASES[case]
    print(f"shards {case} separate_calls={separate_calls}", flush=True)
    w = inputs.custom(SHAPES, grad_kind="masked", seed=61, flags=[inputs.TF_LM_HEAD, 0, 0, 0, 0])
    dev = torch.device("cuda")
    consts = w._tensor_consts("cpu")
    p0 = [p.reshape(-1).contiguous() for p in w.init_params("cpu")]
    whole = q4.Q4State(recipe, w.tensors, dev, cfg=cfg)
    parts = q4.Q4State(recipe, w.tensors, dev, cfg=cfg)
    pw = [p.to(dev) for p in p0]
    ps = [p.to(dev) for p in p0]
    byte_codes = parts.cfg.recipe == api.RECIPE_BLOCK8
    steps = 4
    shards = None
    ws = None
    for k in range(1, steps + 1):
        g = [x.to(dev).reshape(-1).contiguous() for x in w.grads(k, "cpu", consts)]
        phase = inputs.lm_head_sr_on(k, steps)
        whole.step(pw, g, k, lm_head_sr=phase, **HP)
        desc = parts.describe(ps, g)
        shards = [_shard(desc[i], lo, hi, byte_codes)
                  for i, cuts in enumerate(CUTS) for lo, hi in zip(cuts[:-1], cuts[1:])]
        if ws is None:
            nbytes = max(api.q4adamw_workspace_bytes(parts.cfg, [s]) for s in shards)
            nbytes = max(nbytes, api.q4adamw_workspace_bytes(parts.cfg, shards))
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        h = parts.hparams(k, lm_head_sr=phase, **HP)
        if separate_calls:
            for s in shards:
                api.q4adamw_step(parts.cfg, h, [s], ws)
        else:
            api.q4adamw_step(parts.cfg, h, shards, ws)
    torch.cuda.synchronize()
    assert len(shards) == sum(len(c) - 1 for c in CUTS)
    for i in range(len(SHAPES)):
        assert torch.equal(pw[i].view(torch.int32), ps[i].view(torch.int32)), f"tensor {i} weights"
    for (f, a), (_, b) in zip(_state(whole), _state(parts)):
        assert np.array_equal(a, b), f


def test_a_shard_without_its_offset_draws_other_uniforms():
    """The control: ZIP-SR shards passed with elem_offset = 0 round v with
    the uniforms of the tensor's first elements and so differ from the
    whole-tensor step; with their offsets they match it (above)."""
    print("shards without offsets", flush=True)
    w = inputs.custom([(8192,)], grad_kind="masked", seed=62)
    dev = torch.device("cuda")
    p0 = w.init_params("cpu")[0].reshape(-1).contiguous()
    g = w.grads(1, "cpu")[0].reshape(-1).contiguous().to(dev)
    whole = q4.Q4State("zip_sr", w.tensors, dev)
    parts = q4.Q4State("zip_sr", w.tensors, dev)
    pw, ps = p0.to(dev), p0.to(dev)
    whole.step([pw], [g], 1, **HP)
    desc = parts.describe([ps], [g])
    shards = [_shard(desc[0], lo, hi, False) for lo, hi in ((0, 4096), (4096, 8192))]
    shards[1].elem_offset = 0
    ws = torch.empty(api.q4adamw_workspace_bytes(parts.cfg, shards), dtype=torch.uint8, device=dev)
    api.q4adamw_step(parts.cfg, parts.hparams(1, **HP), shards, ws)
    torch.cuda.synchronize()
    a, b = whole.bufs[0].v_codes.cpu().numpy(), parts.bufs[0].v_codes.cpu().numpy()
    assert np.array_equal(a[:2048], b[:2048])
    assert not np.array_equal(a[2048:], b[2048:])
