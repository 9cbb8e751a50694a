"""Optimizer-state buffers allocated with torch and handed to the C ABI.

``Q4State`` owns, per parameter tensor, the buffers the library's header
describes (packed codes, block scales, factored row/column vectors or FP32
moments) plus the step workspace, and forwards to ``q4adamw_init_state``,
``q4adamw_step`` and ``q4adamw_dequant_state``.  It computes nothing itself.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import api

RECIPE_BY_NAME = {"zip_sr": api.RECIPE_ZIP_SR, "ze_eden": api.RECIPE_ZE_EDEN, "factored": api.RECIPE_FACTORED,
                  "fp32": api.RECIPE_FP32, "custom": api.RECIPE_CUSTOM, "block8": api.RECIPE_BLOCK8}


class _Buffers:
    __slots__ = ("shape", "numel", "tensor_id", "flags", "kind", "m_codes", "m_scales", "v_codes", "v_scales",
                 "v_row", "v_col", "m32", "v32")


class Q4State:
    def __init__(self, recipe, specs, device="cuda", cfg: api.Q4Config | None = None, stream=None):
        """specs: iterable of objects with .shape, .tensor_id, .flags (see inputs.TensorSpec)."""
        self.recipe = RECIPE_BY_NAME[recipe] if isinstance(recipe, str) else int(recipe)
        self.cfg = cfg if cfg is not None else api.q4adamw_default_config(self.recipe)
        self.device = torch.device(device)
        self.bufs = []
        for s in specs:
            b = _Buffers()
            b.shape = tuple(int(x) for x in s.shape)
            n = 1
            for x in b.shape:
                n *= x
            b.numel = n
            b.tensor_id = int(s.tensor_id)
            b.flags = int(getattr(s, "flags", 0))
            nb = (n + 127) // 128
            nc = (n + 1) // 2
            b.m_codes = b.m_scales = b.v_codes = b.v_scales = b.v_row = b.v_col = b.m32 = b.v32 = None
            if self.cfg.recipe == api.RECIPE_FP32:
                b.kind = "fp32"
                b.m32 = torch.empty(n, dtype=torch.float32, device=self.device)
                b.v32 = torch.empty(n, dtype=torch.float32, device=self.device)
            elif self.cfg.recipe == api.RECIPE_BLOCK8:
                b.kind = "byte8"   # one byte per code
                b.m_codes = torch.empty(n, dtype=torch.uint8, device=self.device)
                b.m_scales = torch.empty(nb, dtype=torch.float32, device=self.device)
                b.v_codes = torch.empty(n, dtype=torch.uint8, device=self.device)
                b.v_scales = torch.empty(nb, dtype=torch.float32, device=self.device)
            else:
                b.m_codes = torch.empty(nc, dtype=torch.uint8, device=self.device)
                b.m_scales = torch.empty(nb, dtype=torch.float32, device=self.device)
                if self.cfg.recipe == api.RECIPE_FACTORED and len(b.shape) >= 2:
                    b.kind = "factored"
                    b.v_row = torch.empty(b.shape[0], dtype=torch.float32, device=self.device)
                    cols = 1
                    for d in b.shape[1:]:
                        cols *= int(d)
                    b.v_col = torch.empty(cols, dtype=torch.float32, device=self.device)
                else:
                    b.kind = "packed"
                    b.v_codes = torch.empty(nc, dtype=torch.uint8, device=self.device)
                    b.v_scales = torch.empty(nb, dtype=torch.float32, device=self.device)
            self.bufs.append(b)
        desc = self.describe(None, None)
        self.ws_bytes = api.q4adamw_workspace_bytes(self.cfg, desc)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self._last_key = None
        self._flat = None
        api.q4adamw_init_state(self.cfg, desc, stream)

    def describe(self, params, grads) -> list:
        """The C tensor list for these parameter and gradient tensors."""
        out = []
        for i, b in enumerate(self.bufs):
            t = api.Q4Tensor()
            t.tensor_id = b.tensor_id
            t.flags = b.flags
            t.ndim = len(b.shape)
            for d, x in enumerate(b.shape):
                t.shape[d] = x
            t.numel = b.numel
            t.param = params[i].data_ptr() if params is not None else None
            t.grad = grads[i].data_ptr() if grads is not None else None
            for f in ("m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col"):
                x = getattr(b, f)
                setattr(t, f, x.data_ptr() if x is not None else None)
            t.m_fp32 = b.m32.data_ptr() if b.m32 is not None else None
            t.v_fp32 = b.v32.data_ptr() if b.v32 is not None else None
            out.append(t)
        return out

    def hparams(self, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, eps_sr=0.0, seed=0,
                lm_head_sr=0, flags=0, max_grad_norm=0.0) -> api.Q4HParams:
        return api.Q4HParams(lr, beta1, beta2, eps, weight_decay, eps_sr, step, seed, lm_head_sr, flags,
                             max_grad_norm, 0)

    def _table(self, params, grads) -> bool:
        """The C tensor list for these buffers; True when the workspace
        already holds it (the previous call passed the same pointers)."""
        for p, g, b in zip(params, grads, self.bufs):
            if p.dtype != torch.float32 or g.dtype != torch.bfloat16 or p.numel() != b.numel or g.numel() != b.numel:
                raise ValueError("params must be float32 and grads bfloat16, matching the state's shapes")
            if not (p.is_contiguous() and g.is_contiguous()):
                raise ValueError("params and grads must be contiguous")
        key = (tuple(p.data_ptr() for p in params), tuple(g.data_ptr() for g in grads), self.ws.data_ptr())
        same = key == self._last_key
        if not same:
            self._desc = (api.Q4Tensor * len(self.bufs))(*self.describe(params, grads))
        self._last_key = key
        return same

    def step(self, params, grads, step: int, stream=None, grad_stats: bool = False, **hp) -> None:
        """One q4adamw_step.  grad_stats: the workspace holds the statistics
        of these gradients from accumulate(..., last=True) or grad_stats()."""
        flags = hp.pop("flags", 0)
        if self._table(params, grads):
            flags |= api.HP_REUSE_TABLE
        if grad_stats:
            flags |= api.HP_GRAD_STATS
        h = self.hparams(step, flags=flags, **hp)
        self._call(api.q4adamw_step, self.cfg, h, self._desc, self.ws, self.ws_bytes, stream)

    def step_noalloc(self, params, grads, step: int, stream=None, **hp) -> None:
        """One q4adamw_step_noalloc: the workspace is the library's static
        scratch, which every such call on the device shares, so the table is
        always uploaded (no Q4_HP_REUSE_TABLE)."""
        flags = hp.pop("flags", 0) & ~api.HP_REUSE_TABLE
        self._table(params, grads)
        self._last_key = None   # the state's own workspace does not hold this call's table
        h = self.hparams(step, flags=flags, **hp)
        api.q4adamw_step_noalloc(self.cfg, h, self._desc, stream)

    def _call(self, fn, *args) -> None:
        """A call that may upload the tensor table: if it is refused, the
        workspace may not hold the table, so the next call uploads it."""
        try:
            fn(*args)
        except Exception:
            self._last_key = None
            raise

    def flat_offsets(self) -> tuple[list, int]:
        """Element offsets of each tensor in a flat microbatch gradient buffer, and its length."""
        if self._flat is None:   # fixed by the shapes
            self._flat = api.q4adamw_flat_offsets(self.describe(None, None))
        offs, total = self._flat
        return list(offs), total

    def accumulate(self, params, grads, micro, first: bool, last: bool, stream=None) -> None:
        """grads <- micro (first) or bf16(grads + micro), from the flat BF16
        microbatch buffer `micro`; with last, also the statistics."""
        if micro.dtype != torch.bfloat16 or not micro.is_contiguous():
            raise ValueError("micro must be a contiguous bfloat16 buffer")
        _, total = self.flat_offsets()
        if micro.numel() < total:
            raise ValueError(f"micro holds {micro.numel()} elements, the flat layout needs {total}")
        flags = (api.ACC_FIRST if first else 0) | (api.ACC_LAST if last else 0)
        if self._table(params, grads):
            flags |= api.ACC_REUSE_TABLE
        self._call(api.q4adamw_accumulate, self.cfg, self._desc, micro, flags, self.ws, self.ws_bytes, stream)

    def grad_stats(self, params, grads, stream=None) -> None:
        self._table(params, grads)
        self._call(api.q4adamw_grad_stats, self.cfg, self._desc, self.ws, self.ws_bytes, stream)

    def grad_norm(self, stream=None) -> float:
        return api.q4adamw_grad_norm(self.ws, self.ws_bytes, stream)

    def dequant(self, i: int, stream=None):
        b = self.bufs[i]
        m = torch.empty(b.numel, dtype=torch.float32, device=self.device)
        v = torch.empty(b.numel, dtype=torch.float32, device=self.device)
        t = self.describe(None, None)[i]
        # a workspace of its own, so the step's tensor table stays intact
        need = 256 + 8 * ((b.shape[0] + 255) // 256) + 256
        dq = torch.empty(need, dtype=torch.uint8, device=self.device)
        api.q4adamw_dequant_state(self.cfg, t, m, v, dq, need, stream)
        return m, v

    def state_bytes(self) -> dict:
        return api.q4adamw_state_bytes(self.cfg, self.describe(None, None))
