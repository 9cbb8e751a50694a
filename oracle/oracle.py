"""ctypes front end of the CPU oracle (``q4_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports this
module, and this module never imports the GPU library.

Every function takes and returns numpy arrays; the arithmetic all happens in
the C file, which cites the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libq4oracle.so")

# codebooks / rules / recipes (same numbering as the C file)
CB_NF4, CB_SDYN4, CB_DYN4, CB_DYN4_NZ, CB_LIN4_NZ = range(5)
STATE_RTN, STATE_SR, UPDATE_RTN, UPDATE_SR = range(4)
ZIP_SR, ZE_EDEN, FACTORED, FP32, CUSTOM = range(5)
TF_LM_HEAD = 1
BLOCK = 128

# Recipes of the paper's Table 2 plus the factored mode and FP32 AdamW:
# (m codebook, v codebook, m rule, v rule, eden)
RECIPES = {
    ZIP_SR: (CB_NF4, CB_DYN4, STATE_RTN, UPDATE_SR, 0),
    ZE_EDEN: (CB_NF4, CB_DYN4_NZ, STATE_RTN, STATE_RTN, 1),
    FACTORED: (CB_NF4, CB_DYN4_NZ, STATE_RTN, STATE_RTN, 0),
    FP32: (CB_NF4, CB_DYN4, STATE_RTN, STATE_RTN, 0),
}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Hp(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("eps_sr", C.c_float), ("step", C.c_uint64),
                ("seed", C.c_uint64), ("lm_head_sr", C.c_uint32), ("grad_scale", C.c_float)]


class _Cfg(C.Structure):
    _fields_ = [("recipe", C.c_int32), ("m_cb", C.c_int32), ("v_cb", C.c_int32), ("m_rule", C.c_int32),
                ("v_rule", C.c_int32), ("eden", C.c_int32)]


class _Win(C.Structure):
    _fields_ = [("tensor_id", C.c_uint32), ("flags", C.c_uint32), ("numel", C.c_int64), ("cols", C.c_int64),
                ("base", C.c_int64), ("len", C.c_int64),
                ("param", C.c_void_p), ("grad", C.c_void_p),
                ("m_codes", C.c_void_p), ("m_scales", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_scales", C.c_void_p),
                ("R", C.c_void_p), ("C", C.c_void_p), ("inv_meanR", C.c_float),
                ("m32", C.c_void_p), ("v32", C.c_void_p), ("m1_out", C.c_void_p), ("v1_out", C.c_void_p)]


_lib = None


def lib():
    """The oracle library: the build above, or the file named by the
    Q4_ORACLE_LIB environment variable (the tests point it at a build made
    with sanitizers, or at a copy with a mistake planted in it, to show that
    the pins catch it)."""
    global _lib
    if _lib is None:
        L = C.CDLL(os.environ.get("Q4_ORACLE_LIB") or build())
        fp, vp, i32, u32, u64, i64 = (C.POINTER(C.c_float), C.c_void_p, C.c_int, C.c_uint32, C.c_uint64,
                                      C.c_int64)
        L.or_codebook.argtypes = [i32, fp]
        L.or_sorted_levels.argtypes = [i32, fp, C.POINTER(C.c_int), fp]
        L.or_sorted_levels.restype = i32
        L.or_philox4x32_10.argtypes = [C.POINTER(C.c_uint32), C.POINTER(C.c_uint32), C.POINTER(C.c_uint32)]
        L.or_uniform.argtypes = [u64, u64, u32, u32, u64]
        L.or_uniform.restype = C.c_float
        L.or_host_scalars.argtypes = [C.POINTER(_Hp), fp]
        L.or_cell_round.argtypes = [i32] + [C.c_float] * 7
        L.or_cell_round.restype = i32
        L.or_cell_prob_up.argtypes = [i32] + [C.c_double] * 4
        L.or_cell_prob_up.restype = C.c_double
        L.or_requant_m_block.argtypes = [i32, i32, fp, i32, u64, u64, u32, u64, vp, i64]
        L.or_requant_m_block.restype = C.c_float
        L.or_requant_v_block.argtypes = [i32, i32, i32, fp, i32, C.c_float, u64, u64, u32, u64, vp, i64]
        L.or_requant_v_block.restype = C.c_float
        L.or_factored_update.argtypes = [C.POINTER(_Hp), i64, i64, vp, fp, fp, fp]
        L.or_step_window.argtypes = [C.POINTER(_Cfg), C.POINTER(_Hp), C.POINTER(_Win)]
        L.or_step_window.restype = i32
        L.or_dequant_window.argtypes = [C.POINTER(_Cfg), C.POINTER(_Win), fp, fp]
        L.or_zero_code.argtypes = [i32]
        L.or_zero_code.restype = i32
        L.or_state_bytes.argtypes = [i32, i64, i64, i32, C.POINTER(C.c_uint64)]
        L.or_codebook8.argtypes = [i32, fp]
        L.or_sorted_levels8.argtypes = [i32, fp, C.POINTER(C.c_int), fp]
        L.or_sorted_levels8.restype = i32
        L.or_step8_window.argtypes = [C.POINTER(_Hp), C.POINTER(_Win)]
        L.or_step8_window.restype = i32
        L.or_dequant8_window.argtypes = [C.POINTER(_Win), fp, fp]
        L.or_accumulate_bf16.argtypes = [vp, vp, i64, i32]
        L.or_grad_sumsq.argtypes = [vp, i64]
        L.or_grad_sumsq.restype = C.c_double
        L.or_clip_factor.argtypes = [C.c_double, C.c_float]
        L.or_clip_factor.restype = C.c_float
        _lib = L
    return _lib


@dataclass
class HParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1
    eps_sr: float | None = None
    step: int = 1
    seed: int = 0
    lm_head_sr: int = 0
    grad_scale: float = 1.0

    def c(self) -> _Hp:
        return _Hp(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay,
                   self.eps if self.eps_sr is None else self.eps_sr, self.step, self.seed, self.lm_head_sr,
                   self.grad_scale)


@dataclass
class Config:
    recipe: int = ZIP_SR
    m_cb: int = CB_NF4
    v_cb: int = CB_DYN4
    m_rule: int = STATE_RTN
    v_rule: int = UPDATE_SR
    eden: int = 0

    @staticmethod
    def of(recipe: int) -> "Config":
        m_cb, v_cb, m_rule, v_rule, eden = RECIPES[recipe]
        return Config(recipe, m_cb, v_cb, m_rule, v_rule, eden)

    def c(self) -> _Cfg:
        return _Cfg(self.recipe, self.m_cb, self.v_cb, self.m_rule, self.v_rule, self.eden)


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _fp(a: np.ndarray):
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(C.c_float))


def codebook(cb: int) -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().or_codebook(cb, _fp(out))
    return out


def sorted_levels(cb: int):
    L = np.zeros(16, np.float32)
    code = (C.c_int * 16)()
    mid = np.zeros(15, np.float32)
    n = lib().or_sorted_levels(cb, _fp(L), code, _fp(mid))
    return L[:n].copy(), np.array(code[:n], np.int32), mid[:n - 1].copy()


def zero_code(cb: int) -> int:
    return lib().or_zero_code(cb)


def philox(ctr, key) -> np.ndarray:
    c = (C.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (C.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (C.c_uint32 * 4)()
    lib().or_philox4x32_10(c, k, o)
    return np.array(o[:], np.uint32)


def uniform(seed: int, step: int, tensor_id: int, stream: int, i: int) -> float:
    return lib().or_uniform(seed, step, tensor_id, stream, i)


def host_scalars(hp: HParams) -> np.ndarray:
    out = np.zeros(5, np.float32)
    h = hp.c()
    lib().or_host_scalars(C.byref(h), _fp(out))
    return out


def cell_round(rule, x, L_lo, L_hi, s, sv, eps_sr, u) -> int:
    return lib().or_cell_round(rule, x, L_lo, L_hi, s, sv, eps_sr, u)


def cell_prob_up(rule, a_lo, a_hi, v, eps) -> float:
    return lib().or_cell_prob_up(rule, a_lo, a_hi, v, eps)


def requant_m_block(cb, rule, m1, seed=0, step=1, tensor_id=0, elem0=0):
    m1 = np.ascontiguousarray(m1, np.float32)
    n = m1.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    s = lib().or_requant_m_block(cb, rule, _fp(m1), n, seed, step, tensor_id, elem0, _p(codes), 0)
    return codes, np.float32(s)


def requant_v_block(cb, rule, eden, v1, eps_sr=1e-8, seed=0, step=1, tensor_id=0, elem0=0):
    v1 = np.ascontiguousarray(v1, np.float32)
    n = v1.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    s = lib().or_requant_v_block(cb, rule, eden, _fp(v1), n, eps_sr, seed, step, tensor_id, elem0, _p(codes), 0)
    return codes, np.float32(s)


def unpack(codes: np.ndarray, n: int) -> np.ndarray:
    """Nibbles in element order (even element in the low nibble)."""
    out = np.empty(2 * codes.size, np.uint8)
    out[0::2] = codes & 0x0F
    out[1::2] = codes >> 4
    return out[:n]


def factored_update(hp: HParams, rows: int, cols: int, grad: np.ndarray, R: np.ndarray, Cc: np.ndarray) -> float:
    assert grad.dtype == np.uint16 and grad.size == rows * cols
    inv = np.zeros(1, np.float32)
    h = hp.c()
    lib().or_factored_update(C.byref(h), rows, cols, _p(grad), _fp(R), _fp(Cc), _fp(inv))
    return float(inv[0])


def step_window(cfg: Config, hp: HParams, *, tensor_id: int, flags: int, numel: int, base: int,
                param, grad, m_codes=None, m_scales=None, v_codes=None, v_scales=None,
                cols: int = 0, R=None, Cc=None, inv_meanR: float = 0.0, m32=None, v32=None,
                m1_out=None, v1_out=None) -> None:
    """Step elements [base, base + len(param)) of a tensor in place.  With
    m1_out / v1_out (float32, the window's length) the unquantized moments
    of the step are written there too."""
    length = param.size
    assert grad.size == length and grad.dtype == np.uint16 and param.dtype == np.float32
    for o in (m1_out, v1_out):
        assert o is None or (o.dtype == np.float32 and o.size == length)
    w = _Win(tensor_id, flags, numel, cols, base, length, _p(param), _p(grad), _p(m_codes), _p(m_scales),
             _p(v_codes), _p(v_scales), _p(R), _p(Cc), inv_meanR, _p(m32), _p(v32), _p(m1_out), _p(v1_out))
    c, h = cfg.c(), hp.c()
    rc = lib().or_step_window(C.byref(c), C.byref(h), C.byref(w))
    if rc != 0:
        raise ValueError("oracle: window base must be a multiple of 128")


def dequant_window(cfg: Config, *, numel: int, base: int, length: int, m_codes, m_scales, v_codes=None,
                   v_scales=None, cols: int = 0, R=None, Cc=None, inv_meanR: float = 0.0):
    w = _Win(0, 0, numel, cols, base, length, None, None, _p(m_codes), _p(m_scales), _p(v_codes), _p(v_scales),
             _p(R), _p(Cc), inv_meanR, None, None)
    m = np.zeros(length, np.float32)
    v = np.zeros(length, np.float32)
    c = cfg.c()
    lib().or_dequant_window(C.byref(c), C.byref(w), _fp(m), _fp(v))
    return m, v


def accumulate_bf16(acc: np.ndarray, micro: np.ndarray, first: bool) -> None:
    """acc <- micro (first) or bf16(f32(acc) + f32(micro)), in place (uint16 BF16 bits)."""
    assert acc.dtype == np.uint16 and micro.dtype == np.uint16 and acc.size == micro.size
    lib().or_accumulate_bf16(_p(acc), _p(micro), acc.size, int(bool(first)))


def grad_sumsq(g: np.ndarray) -> float:
    """Binary64 sum of the FP32 squares of a BF16 gradient, in index order."""
    assert g.dtype == np.uint16
    return float(lib().or_grad_sumsq(_p(g), g.size))


def clip_factor(sq: float, max_norm: float) -> float:
    """min(1, max_norm / (sqrt(sq) + 1e-6)) rounded to FP32; 1.0 when max_norm <= 0."""
    return float(lib().or_clip_factor(float(sq), float(max_norm)))


def state_bytes(recipe: int, numel: int, rows: int, is_matrix: bool) -> tuple[int, int, int]:
    out = (C.c_uint64 * 3)()
    lib().or_state_bytes(recipe, numel, rows, int(is_matrix), out)
    return int(out[0]), int(out[1]), int(out[2])


# ----------------------------------------------------------------------------
# Whole-tensor state held on the host, for multi-step runs in the tests.
# ----------------------------------------------------------------------------

class TensorState:
    """Host copy of one tensor's optimizer state, initialised as 'moments
    start at 0' (codes of zero, scales +0, R = C = 0, FP32 moments 0)."""

    def __init__(self, cfg: Config, shape, tensor_id: int, flags: int = 0):
        self.cfg = cfg
        self.shape = tuple(int(s) for s in shape)
        self.numel = int(np.prod(self.shape))
        self.tensor_id = tensor_id
        self.flags = flags
        n, nb = self.numel, (self.numel + BLOCK - 1) // BLOCK
        self.factored = cfg.recipe == FACTORED and len(self.shape) >= 2
        # the matrix viewed as [shape[0], -1]: its columns are the trailing dimensions
        self.cols = int(np.prod(self.shape[1:])) if self.factored else 0
        self.m32 = self.v32 = self.m_codes = self.m_scales = self.v_codes = self.v_scales = None
        self.R = self.Cc = None
        self.inv_meanR = 0.0
        if cfg.recipe == FP32:
            self.m32 = np.zeros(n, np.float32)
            self.v32 = np.zeros(n, np.float32)
            return
        zm = zero_code(cfg.m_cb)
        self.m_codes = np.full((n + 1) // 2, zm | (zm << 4), np.uint8)
        if n % 2:
            self.m_codes[-1] = zm
        self.m_scales = np.zeros(nb, np.float32)
        if self.factored:
            self.R = np.zeros(self.shape[0], np.float32)
            self.Cc = np.zeros(self.cols, np.float32)
        else:
            zv = zero_code(cfg.v_cb)
            self.v_codes = np.full((n + 1) // 2, zv | (zv << 4), np.uint8)
            if n % 2:
                self.v_codes[-1] = zv
            self.v_scales = np.zeros(nb, np.float32)

    def step(self, hp: HParams, param: np.ndarray, grad: np.ndarray) -> None:
        if self.numel == 0:  # no elements: no moments, no statistics to update
            return
        if self.factored:
            self.inv_meanR = factored_update(hp, self.shape[0], self.cols, grad, self.R, self.Cc)
        step_window(self.cfg, hp, tensor_id=self.tensor_id, flags=self.flags, numel=self.numel, base=0,
                    param=param, grad=grad, m_codes=self.m_codes, m_scales=self.m_scales, v_codes=self.v_codes,
                    v_scales=self.v_scales, cols=self.cols, R=self.R, Cc=self.Cc, inv_meanR=self.inv_meanR,
                    m32=self.m32, v32=self.v32)

    def dequant(self):
        if self.cfg.recipe == FP32:
            return self.m32.copy(), self.v32.copy()
        return dequant_window(self.cfg, numel=self.numel, base=0, length=self.numel, m_codes=self.m_codes,
                              m_scales=self.m_scales, v_codes=self.v_codes, v_scales=self.v_scales,
                              cols=self.cols, R=self.R, Cc=self.Cc, inv_meanR=self.inv_meanR)


# ---------------------------------------------------------------------------
# 8-bit blockwise AdamW
# ---------------------------------------------------------------------------

CB8_SDYN8, CB8_DYN8 = 0, 1


def codebook8(cb8: int) -> np.ndarray:
    """Code-indexed 256-entry table: SDyn8 (m) or Dyn8 (v)."""
    out = np.zeros(256, np.float32)
    lib().or_codebook8(cb8, _fp(out))
    return out


def sorted_levels8(cb8: int):
    L = np.zeros(256, np.float32)
    code = (C.c_int * 256)()
    mid = np.zeros(255, np.float32)
    n = lib().or_sorted_levels8(cb8, _fp(L), code, _fp(mid))
    return L[:n].copy(), np.array(code[:n]), mid[: n - 1].copy()


class TensorState8:
    """Host copy of one tensor's 8-bit state (one byte per code), zero state:
    codes 0 (both maps decode code 0 to 0), scales +0."""

    def __init__(self, shape, tensor_id: int, flags: int = 0):
        self.shape = tuple(int(s) for s in shape)
        self.numel = int(np.prod(self.shape))
        self.tensor_id = tensor_id
        self.flags = flags
        nb = (self.numel + BLOCK - 1) // BLOCK
        self.m_codes = np.zeros(self.numel, np.uint8)
        self.v_codes = np.zeros(self.numel, np.uint8)
        self.m_scales = np.zeros(nb, np.float32)
        self.v_scales = np.zeros(nb, np.float32)

    def step(self, hp: HParams, param: np.ndarray, grad: np.ndarray, base: int = 0, length: int | None = None):
        """Step elements [base, base + length) (base a multiple of 128; the
        arrays passed are the whole tensor's)."""
        length = self.numel - base if length is None else length
        b0 = base // BLOCK
        nb = (length + BLOCK - 1) // BLOCK
        p = param[base: base + length]
        g = np.ascontiguousarray(grad[base: base + length])
        mc = self.m_codes[base: base + length]
        vc = self.v_codes[base: base + length]
        ms = self.m_scales[b0: b0 + nb]
        vs = self.v_scales[b0: b0 + nb]
        assert p.flags.c_contiguous and mc.flags.c_contiguous
        w = _Win(self.tensor_id, self.flags, self.numel, 0, base, length, _p(p), _p(g), _p(mc), _p(ms), _p(vc),
                 _p(vs), None, None, 0.0, None, None)
        h = hp.c()
        if lib().or_step8_window(C.byref(h), C.byref(w)) != 0:
            raise ValueError("oracle: window base must be a multiple of 128")

    def dequant(self):
        w = _Win(0, 0, self.numel, 0, 0, self.numel, None, None, _p(self.m_codes), _p(self.m_scales),
                 _p(self.v_codes), _p(self.v_scales), None, None, 0.0, None, None)
        m = np.zeros(self.numel, np.float32)
        v = np.zeros(self.numel, np.float32)
        lib().or_dequant8_window(C.byref(w), _fp(m), _fp(v))
        return m, v
