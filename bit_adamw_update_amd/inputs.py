"""Seeded synthetic workloads: tensor lists, master weights and BF16 gradients.

This module serves both the GPU path and the CPU oracle and therefore holds
none of the optimizer's arithmetic: it only draws numbers.  Shapes follow the
architectures of the paper's Table 6 ("Rounding in Preconditioner Space",
appendix) and the factored-mode page ("4-bit AdamW", AReno docs); value
distributions follow the workload recipes stated in the design notes:

* masters ~ N(0, 0.02) in FP32 for every tensor;
* gradients are Student-t (df = 3) draws, built as z / sqrt(chi2_3 / 3) from
  four standard normals, times a per-tensor scale, rounded to BF16 (RNE);
* "tiny" and "llama-1.1b": scale 1e-3, with a fixed 20% of coordinates per
  tensor at 1e-9 so that they sit in the cell next to zero;
* "gpt-162m", "gpt-2.7b": a per-tensor scale 10^U(-5,-2), drawn once;
* "qwen3-0.6b-factored": four such microbatches per step, accumulated in BF16.

A fresh gradient is drawn for every step from a generator keyed on
(seed, step).  The same bytes are handed to both implementations.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

TF_LM_HEAD = 1


@dataclass
class TensorSpec:
    name: str
    shape: tuple
    tensor_id: int
    flags: int = 0

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= int(s)
        return n


@dataclass
class Workload:
    name: str
    tensors: list
    grad_kind: str            # "masked" | "logscale" | "microbatch4" | "edge" | "nonfinite"
    steps: int
    recipes: tuple
    seed: int = 0
    lm_head_switch: bool = False   # the final-10% phase flag on the LM head
    hp: dict = field(default_factory=lambda: dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                                  weight_decay=0.1))

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)

    # --- drawing -------------------------------------------------------
    def _gen(self, device, salt: int) -> torch.Generator:
        g = torch.Generator(device=device)
        g.manual_seed((self.seed * 1_000_003 + salt) & 0x7FFF_FFFF_FFFF_FFFF)
        return g

    def init_params(self, device="cpu") -> list:
        g = self._gen(device, 1)
        return [torch.randn(t.shape, generator=g, device=device, dtype=torch.float32).mul_(0.02)
                for t in self.tensors]

    def _tensor_consts(self, device):
        """Per-tensor constants drawn once: masks or log-uniform scales."""
        g = self._gen(device, 2)
        out = []
        for t in self.tensors:
            if self.grad_kind == "masked":
                out.append(torch.rand(t.shape, generator=g, device=device) < 0.2)
            else:
                e = torch.rand((), generator=g, device=device, dtype=torch.float64).item() * 3.0 - 5.0
                out.append(10.0 ** e)
        return out

    @staticmethod
    def _student_t3(shape, g, device) -> torch.Tensor:
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        c = torch.zeros(shape, device=device, dtype=torch.float32)
        for _ in range(3):
            w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            c.addcmul_(w, w)
        return z.div_(c.div_(3.0).sqrt_())

    # magnitude classes of the "edge" kind, one per 128-block in turn
    EDGE_SCALES = (1e-3, 1e-16, 1e-39, 0.0, 1e-3, 1e-25, 1e-20, 8e-39)

    def _edge(self, shape, g, device) -> torch.Tensor:
        """Blocks of normal, tiny (squares below 2^-96), BF16-subnormal
        (first-moment scales below 2^-128, whose reciprocal overflows, and
        between 2^-128 and 2^-126, whose reciprocal is finite), signed-zero,
        mixed (exact zeros and values 10^6 times larger), and vanishing
        (squares underflow to zero or to subnormals) gradients."""
        x = self._student_t3(shape, g, device).reshape(-1)
        cls = (torch.arange(x.numel(), device=device) // 128) % len(self.EDGE_SCALES)
        y = x * torch.tensor(self.EDGE_SCALES, device=device, dtype=torch.float32)[cls]
        y = torch.where(cls == 3, torch.where(x < 0, torch.tensor(-0.0, device=device),
                                              torch.tensor(0.0, device=device)), y)
        idx = torch.arange(x.numel(), device=device)
        mixed = cls == 4
        y = torch.where(mixed & (idx % 9 == 0), torch.zeros_like(y), y)
        y = torch.where(mixed & (idx % 61 == 0), x * 1e3, y)
        return y.to(torch.bfloat16).reshape(shape)

    # non-finite classes of the "nonfinite" kind, one per 128-block in turn:
    # (offset in the block, value) pairs written over Student-t gradients;
    # None in place of a list sets the whole block
    NONFINITE_CLASSES = (
        [],                                                   # finite
        [(37, float("nan"))],                                 # one NaN
        [(5, float("inf"))],                                  # one +inf
        [(100, float("-inf"))],                               # one -inf
        [(64, 1e30)],                                         # finite, its square overflows FP32
        None,                                                 # every element NaN
        [(0, float("nan")), (127, float("-inf"))],            # NaN and -inf
        [],                                                   # finite
    )

    def _nonfinite(self, shape, g, device) -> torch.Tensor:
        """Student-t gradients (scale 1e-3) with NaN, +-inf and overflowing
        values at fixed places of each block class, the same every step."""
        x = (self._student_t3(shape, g, device) * 1e-3).reshape(-1)
        n = x.numel()
        for b in range((n + 127) // 128):
            cls = self.NONFINITE_CLASSES[b % len(self.NONFINITE_CLASSES)]
            if cls is None:
                x[128 * b:min(n, 128 * b + 128)] = float("nan")
                continue
            for off, val in cls:
                if 128 * b + off < n:
                    x[128 * b + off] = val
        return x.to(torch.bfloat16).reshape(shape)

    def grads(self, step: int, device="cpu", consts=None) -> list:
        """BF16 gradients of `step` (1-based), one tensor per parameter."""
        if consts is None:
            consts = self._tensor_consts(device)
        out = []
        g = self._gen(device, 1000 + step)
        for t, c in zip(self.tensors, consts):
            if self.grad_kind == "masked":
                x = self._student_t3(t.shape, g, device)
                scale = torch.where(c, torch.tensor(1e-9, device=device), torch.tensor(1e-3, device=device))
                out.append(x.mul_(scale).to(torch.bfloat16))
            elif self.grad_kind == "edge":
                out.append(self._edge(t.shape, g, device))
            elif self.grad_kind == "nonfinite":
                out.append(self._nonfinite(t.shape, g, device))
            elif self.grad_kind == "logscale":
                out.append(self._student_t3(t.shape, g, device).mul_(c).to(torch.bfloat16))
            else:  # four microbatches, accumulated in BF16 in order
                acc = self._student_t3(t.shape, g, device).mul_(c).to(torch.bfloat16)
                for _ in range(3):
                    mb = self._student_t3(t.shape, g, device).mul_(c).to(torch.bfloat16)
                    acc = (acc.float() + mb.float()).to(torch.bfloat16)
                out.append(acc)
        return out


def _gpt(name, vocab, d, layers, ffn, recipes, steps, grad_kind="logscale"):
    ts = [TensorSpec("wte", (vocab, d), 0, TF_LM_HEAD)]  # tied embedding / LM head
    tid = 1
    for layer in range(layers):
        for nm, shp in (("qkv", (d, 3 * d)), ("proj", (d, d)), ("fc", (d, ffn)), ("fc2", (ffn, d)),
                        ("ln1_w", (d,)), ("ln1_b", (d,)), ("ln2_w", (d,)), ("ln2_b", (d,))):
            ts.append(TensorSpec(f"h{layer}.{nm}", shp, tid))
            tid += 1
    return Workload(name, ts, grad_kind, steps, recipes)


def tiny() -> Workload:
    return Workload("tiny", [TensorSpec("vec", (65536,), 0), TensorSpec("mat", (256, 512), 1)],
                    "masked", 10, ("zip_sr", "ze_eden", "fp32"))


def gpt_162m() -> Workload:
    return _gpt("gpt-162m", 50304, 768, 12, 3072, ("zip_sr", "ze_eden"), 20)


def gpt_2_7b() -> Workload:
    return _gpt("gpt-2.7b", 50304, 2560, 32, 10240, ("ze_eden", "zip_sr"), 10)


def llama_1_1b() -> Workload:
    d, kv, ffn, vocab = 2048, 256, 5632, 32000
    ts = [TensorSpec("embed", (vocab, d), 0)]
    tid = 1
    for layer in range(22):
        for nm, shp in (("q", (d, d)), ("k", (d, kv)), ("v", (d, kv)), ("o", (d, d)), ("gate", (d, ffn)),
                        ("up", (d, ffn)), ("down", (ffn, d)), ("attn_norm", (d,)), ("mlp_norm", (d,))):
            ts.append(TensorSpec(f"l{layer}.{nm}", shp, tid))
            tid += 1
    ts.append(TensorSpec("final_norm", (d,), tid))
    ts.append(TensorSpec("lm_head", (vocab, d), tid + 1, TF_LM_HEAD))
    return Workload("llama-1.1b", ts, "masked", 10, ("zip_sr",), lm_head_switch=True)


def qwen3_0_6b_factored() -> Workload:
    d, vocab = 1024, 151936
    ts = [TensorSpec("embed", (vocab, d), 0, TF_LM_HEAD)]
    tid = 1
    for layer in range(28):
        for nm, shp in (("q", (d, 2048)), ("k", (d, d)), ("v", (d, d)), ("o", (2048, d)), ("gate", (d, 3072)),
                        ("up", (d, 3072)), ("down", (3072, d)), ("in_norm", (d,)), ("post_norm", (d,)),
                        ("q_norm", (128,)), ("k_norm", (128,))):
            ts.append(TensorSpec(f"l{layer}.{nm}", shp, tid))
            tid += 1
    ts.append(TensorSpec("final_norm", (d,), tid))
    return Workload("qwen3-0.6b-factored", ts, "microbatch4", 10, ("factored",))


WORKLOADS = {
    "tiny": tiny,
    "gpt-162m": gpt_162m,
    "llama-1.1b": llama_1_1b,
    "gpt-2.7b": gpt_2_7b,
    "qwen3-0.6b-factored": qwen3_0_6b_factored,
}


def lm_head_sr_on(step: int, total_steps: int) -> int:
    """Phase flag of the final 10% of training: on iff step > floor(0.9 T)."""
    return int(step > (9 * total_steps) // 10)


def custom(shapes, grad_kind="masked", seed=0, steps=10, flags=None) -> Workload:
    """Ad-hoc workload for edge cases (ragged sizes, single blocks, ...)."""
    flags = flags or [0] * len(shapes)
    ts = [TensorSpec(f"t{i}", tuple(s), i, f) for i, (s, f) in enumerate(zip(shapes, flags))]
    return Workload("custom", ts, grad_kind, steps, (), seed=seed)
