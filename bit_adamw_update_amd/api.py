"""ctypes declarations of the C ABI (``include/q4adamw.h``), same names.

Argument marshalling only: structures mirror the header field by field, and
each function forwards to the library and turns a non-OK status into a
``Q4Error`` carrying the library's message.
"""
from __future__ import annotations

import ctypes as C
import os

from .build import LIB_PATH

RECIPE_ZIP_SR, RECIPE_ZE_EDEN, RECIPE_FACTORED, RECIPE_FP32, RECIPE_CUSTOM, RECIPE_BLOCK8 = range(6)
CB_NF4, CB_SDYN4, CB_DYN4, CB_DYN4_NZ, CB_LIN4_NZ, CB_SDYN8, CB_DYN8 = range(7)
RULE_STATE_RTN, RULE_STATE_SR, RULE_UPDATE_RTN, RULE_UPDATE_SR = range(4)
HP_REUSE_TABLE, HP_CHECK_POINTERS, HP_GRAD_STATS = 1, 2, 4
ACC_FIRST, ACC_LAST, ACC_REUSE_TABLE = 1, 2, 4
TF_LM_HEAD = 1
ABI_VERSION = 3
MAX_NDIM = 8

STATUS = {0: "Q4_OK", 1: "Q4_ERR_INVALID_ARG", 2: "Q4_ERR_SHAPE", 3: "Q4_ERR_ALIGNMENT", 4: "Q4_ERR_CONFLICT",
          5: "Q4_ERR_STATE_FORMAT", 6: "Q4_ERR_DEVICE", 7: "Q4_ERR_WORKSPACE", 8: "Q4_ERR_HIP"}


class Q4Config(C.Structure):
    _fields_ = [("abi_version", C.c_uint32), ("recipe", C.c_int32), ("block", C.c_int32),
                ("m_codebook", C.c_int32), ("v_codebook", C.c_int32), ("m_rule", C.c_int32),
                ("v_rule", C.c_int32), ("eden", C.c_int32)]


class Q4HParams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("eps_sr", C.c_float), ("step", C.c_uint64), ("seed", C.c_uint64),
                ("lm_head_sr", C.c_uint32), ("flags", C.c_uint32), ("max_grad_norm", C.c_float),
                ("reserved", C.c_uint32)]


class Q4Tensor(C.Structure):
    _fields_ = [("tensor_id", C.c_uint32), ("flags", C.c_uint32), ("ndim", C.c_int32), ("reserved", C.c_int32),
                ("shape", C.c_int64 * MAX_NDIM), ("numel", C.c_int64),
                ("param", C.c_void_p), ("grad", C.c_void_p), ("m_codes", C.c_void_p), ("m_scales", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_scales", C.c_void_p), ("v_row", C.c_void_p), ("v_col", C.c_void_p),
                ("m_fp32", C.c_void_p), ("v_fp32", C.c_void_p), ("elem_offset", C.c_int64)]


class Q4StateBytes(C.Structure):
    _fields_ = [("adam4_quantized_state_bytes", C.c_uint64), ("adam4_scale_metadata_bytes", C.c_uint64),
                ("adam4_total_bytes", C.c_uint64)]


class Q4StateHeader(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("abi_version", C.c_uint32), ("layout_version", C.c_uint32),
                ("recipe", C.c_int32), ("m_codebook", C.c_int32), ("v_codebook", C.c_int32),
                ("m_rule", C.c_int32), ("v_rule", C.c_int32), ("eden", C.c_int32), ("block", C.c_int32)]


class Q4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

_SIGNATURES = {
    "q4adamw_abi_version": ([], C.c_uint32),
    "q4adamw_status_string": ([C.c_int], C.c_char_p),
    "q4adamw_last_error": ([], C.c_char_p),
    "q4adamw_default_config": ([C.c_int32, C.POINTER(Q4Config)], C.c_int),
    "q4adamw_validate": ([C.POINTER(Q4Config), C.POINTER(Q4HParams), C.POINTER(Q4Tensor), C.c_int32], C.c_int),
    "q4adamw_workspace_bytes": ([C.POINTER(Q4Config), C.POINTER(Q4Tensor), C.c_int32, C.POINTER(C.c_size_t)],
                                C.c_int),
    "q4adamw_state_bytes": ([C.POINTER(Q4Config), C.POINTER(Q4Tensor), C.c_int32, C.POINTER(Q4StateBytes)],
                            C.c_int),
    "q4adamw_make_header": ([C.POINTER(Q4Config), C.POINTER(Q4StateHeader)], C.c_int),
    "q4adamw_check_header": ([C.POINTER(Q4Config), C.POINTER(Q4StateHeader)], C.c_int),
    "q4adamw_host_scalars": ([C.POINTER(Q4HParams), C.POINTER(C.c_float)], C.c_int),
    "q4adamw_codebook": ([C.c_int32, C.POINTER(C.c_float)], C.c_int),
    "q4adamw_init_state": ([C.POINTER(Q4Config), C.POINTER(Q4Tensor), C.c_int32, C.c_void_p], C.c_int),
    "q4adamw_step": ([C.POINTER(Q4Config), C.POINTER(Q4HParams), C.POINTER(Q4Tensor), C.c_int32, C.c_void_p,
                      C.c_size_t, C.c_void_p], C.c_int),
    "q4adamw_step_noalloc": ([C.POINTER(Q4Config), C.POINTER(Q4HParams), C.POINTER(Q4Tensor), C.c_int32,
                              C.c_void_p], C.c_int),
    "q4adamw_dequant_state": ([C.POINTER(Q4Config), C.POINTER(Q4Tensor), C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_size_t, C.c_void_p], C.c_int),
    "q4adamw_flat_offsets": ([C.POINTER(Q4Tensor), C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_int64)], C.c_int),
    "q4adamw_accumulate": ([C.POINTER(Q4Config), C.POINTER(Q4Tensor), C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                           C.c_size_t, C.c_void_p], C.c_int),
    "q4adamw_grad_stats": ([C.POINTER(Q4Config), C.POINTER(Q4Tensor), C.c_int32, C.c_void_p, C.c_size_t,
                           C.c_void_p], C.c_int),
    "q4adamw_grad_norm": ([C.c_void_p, C.c_size_t, C.POINTER(C.c_double), C.c_void_p], C.c_int),
}


def load_library(path: str = LIB_PATH):
    """Load libq4adamw.so; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libq4adamw.so not built ({path}); run bit_adamw_update_amd.build.build()")
    lib = C.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().q4adamw_last_error().decode(errors="replace")
        raise Q4Error(status, msg)


def _tensors(ts):
    if isinstance(ts, Q4Tensor):
        return C.pointer(ts), 1
    if isinstance(ts, C.Array):
        return ts, len(ts)
    arr = (Q4Tensor * len(ts))(*ts)
    return arr, len(ts)


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def q4adamw_abi_version() -> int:
    return load_library().q4adamw_abi_version()


def q4adamw_status_string(status: int) -> str:
    return load_library().q4adamw_status_string(status).decode()


def q4adamw_last_error() -> str:
    return load_library().q4adamw_last_error().decode(errors="replace")


def q4adamw_default_config(recipe: int) -> Q4Config:
    cfg = Q4Config()
    _check(load_library().q4adamw_default_config(recipe, C.byref(cfg)))
    return cfg


def q4adamw_validate(cfg: Q4Config, hp: Q4HParams | None, tensors) -> None:
    arr, n = _tensors(tensors)
    _check(load_library().q4adamw_validate(C.byref(cfg), C.byref(hp) if hp is not None else None, arr, n))


def q4adamw_workspace_bytes(cfg: Q4Config, tensors) -> int:
    arr, n = _tensors(tensors)
    out = C.c_size_t()
    _check(load_library().q4adamw_workspace_bytes(C.byref(cfg), arr, n, C.byref(out)))
    return out.value


def q4adamw_state_bytes(cfg: Q4Config, tensors) -> dict:
    arr, n = _tensors(tensors)
    out = Q4StateBytes()
    _check(load_library().q4adamw_state_bytes(C.byref(cfg), arr, n, C.byref(out)))
    return {"adam4_quantized_state_bytes": out.adam4_quantized_state_bytes,
            "adam4_scale_metadata_bytes": out.adam4_scale_metadata_bytes,
            "adam4_total_bytes": out.adam4_total_bytes}


def q4adamw_make_header(cfg: Q4Config) -> Q4StateHeader:
    h = Q4StateHeader()
    _check(load_library().q4adamw_make_header(C.byref(cfg), C.byref(h)))
    return h


def q4adamw_check_header(cfg: Q4Config, hdr: Q4StateHeader) -> None:
    _check(load_library().q4adamw_check_header(C.byref(cfg), C.byref(hdr)))


def q4adamw_host_scalars(hp: Q4HParams):
    out = (C.c_float * 5)()
    _check(load_library().q4adamw_host_scalars(C.byref(hp), out))
    return list(out)


def q4adamw_codebook(cb: int):
    out = (C.c_float * (256 if cb in (CB_SDYN8, CB_DYN8) else 16))()
    _check(load_library().q4adamw_codebook(cb, out))
    return list(out)


def q4adamw_init_state(cfg: Q4Config, tensors, stream=None) -> None:
    arr, n = _tensors(tensors)
    _check(load_library().q4adamw_init_state(C.byref(cfg), arr, n, _stream(stream)))


def q4adamw_step(cfg: Q4Config, hp: Q4HParams, tensors, ws, ws_bytes: int | None = None, stream=None) -> None:
    arr, n = _tensors(tensors)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load_library().q4adamw_step(C.byref(cfg), C.byref(hp), arr, n, _ptr(ws), ws_bytes, _stream(stream)))


def q4adamw_step_noalloc(cfg: Q4Config, hp: Q4HParams, tensors, stream=None) -> None:
    arr, n = _tensors(tensors)
    _check(load_library().q4adamw_step_noalloc(C.byref(cfg), C.byref(hp), arr, n, _stream(stream)))


def q4adamw_dequant_state(cfg: Q4Config, tensor: Q4Tensor, m_out, v_out, ws=None, ws_bytes: int | None = None,
                          stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().q4adamw_dequant_state(C.byref(cfg), C.byref(tensor), _ptr(m_out), _ptr(v_out), _ptr(ws),
                                                ws_bytes, _stream(stream)))


def q4adamw_flat_offsets(tensors) -> tuple[list, int]:
    arr, n = _tensors(tensors)
    offs = (C.c_int64 * n)()
    total = C.c_int64()
    _check(load_library().q4adamw_flat_offsets(arr, n, offs, C.byref(total)))
    return list(offs), total.value


def q4adamw_accumulate(cfg: Q4Config, tensors, micro, flags: int, ws, ws_bytes: int | None = None,
                       stream=None) -> None:
    arr, n = _tensors(tensors)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load_library().q4adamw_accumulate(C.byref(cfg), arr, n, _ptr(micro), flags, _ptr(ws), ws_bytes,
                                             _stream(stream)))


def q4adamw_grad_stats(cfg: Q4Config, tensors, ws, ws_bytes: int | None = None, stream=None) -> None:
    arr, n = _tensors(tensors)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load_library().q4adamw_grad_stats(C.byref(cfg), arr, n, _ptr(ws), ws_bytes, _stream(stream)))


def q4adamw_grad_norm(ws, ws_bytes: int | None = None, stream=None) -> float:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    out = C.c_double()
    _check(load_library().q4adamw_grad_norm(_ptr(ws), ws_bytes, C.byref(out), _stream(stream)))
    return out.value
