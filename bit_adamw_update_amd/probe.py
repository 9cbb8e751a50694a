"""ctypes binding of libq4probe.so (include/q4probe.h): the bandwidth probes
that give the step's practical ceiling.  Argument marshalling only."""
from __future__ import annotations

import ctypes as C

import torch

from . import build

_lib = None


def load_library():
    global _lib
    if _lib is None:
        import os
        if not os.path.exists(build.PROBE_PATH):
            raise RuntimeError(f"libq4probe.so not built ({build.PROBE_PATH}); run bit_adamw_update_amd.build.build()")
        L = C.CDLL(build.PROBE_PATH)
        vp, i64 = C.c_void_p, C.c_int64
        L.q4probe_byte_mix_bytes.argtypes = [i64]
        L.q4probe_byte_mix_bytes.restype = i64
        L.q4probe_byte_mix.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp]
        L.q4probe_byte_mix.restype = C.c_int
        L.q4probe_copy.argtypes = [vp, vp, C.c_size_t, vp]
        L.q4probe_copy.restype = C.c_int
        L.q4probe_byte_mix_queue.argtypes = L.q4probe_byte_mix.argtypes
        L.q4probe_byte_mix_queue.restype = C.c_int
        L.q4probe_byte_mix8_bytes.argtypes = [i64]
        L.q4probe_byte_mix8_bytes.restype = i64
        L.q4probe_byte_mix8.argtypes = L.q4probe_byte_mix.argtypes
        L.q4probe_byte_mix8.restype = C.c_int
        L.q4probe_byte_mix8_queue.argtypes = L.q4probe_byte_mix.argtypes
        L.q4probe_byte_mix8_queue.restype = C.c_int
        L.q4probe_update_in_place.argtypes = [vp, C.c_size_t, vp]
        L.q4probe_update_in_place.restype = C.c_int
        L.q4probe_read_sink_words.argtypes = []
        L.q4probe_read_sink_words.restype = i64
        L.q4probe_read.argtypes = [vp, C.c_size_t, vp, vp]
        L.q4probe_read.restype = C.c_int
        _lib = L
    return _lib


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def byte_mix_bytes(n: int, bits: int = 4) -> int:
    L = load_library()
    return int(L.q4probe_byte_mix_bytes(n) if bits == 4 else L.q4probe_byte_mix8_bytes(n))


class ByteMix:
    """Buffers of a step's byte mix for n elements (n a multiple of 512),
    filled with non-zero data: the 4-bit steps' (bits=4) or the 8-bit
    step's (bits=8)."""

    def __init__(self, n: int, device="cuda", bits: int = 4):
        assert n > 0 and n % 512 == 0 and bits in (4, 8)
        self.n = n
        self.bits = bits
        g = torch.Generator(device=device).manual_seed(7)
        self.param = torch.randn(n, generator=g, device=device) * 0.02
        self.grad = (torch.randn(n, generator=g, device=device) * 1e-3).to(torch.bfloat16)
        ncode = n * bits // 8
        self.m_codes = torch.randint(0, 256, (ncode,), generator=g, device=device, dtype=torch.uint8)
        self.v_codes = torch.randint(0, 256, (ncode,), generator=g, device=device, dtype=torch.uint8)
        self.m_scales = torch.rand(n // 128, generator=g, device=device) + 0.5
        self.v_scales = torch.rand(n // 128, generator=g, device=device) + 0.5

    def _args(self, stream):
        return (self.param.data_ptr(), self.grad.data_ptr(), self.m_codes.data_ptr(), self.v_codes.data_ptr(),
                self.m_scales.data_ptr(), self.v_scales.data_ptr(), self.n, _stream(stream))

    def bytes(self) -> int:
        return byte_mix_bytes(self.n, self.bits)

    def run(self, stream=None) -> None:
        """The step's own lane layout and work-group walk."""
        name = "q4probe_byte_mix" if self.bits == 4 else "q4probe_byte_mix8"
        _ok(getattr(load_library(), name)(*self._args(stream)), name)

    def run_queue(self, stream=None) -> None:
        """The same bytes taken from a queue of runs."""
        name = "q4probe_byte_mix_queue" if self.bits == 4 else "q4probe_byte_mix8_queue"
        _ok(getattr(load_library(), name)(*self._args(stream)), name)


def copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nbytes
    _ok(load_library().q4probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream)), "q4probe_copy")


def update_in_place(x: torch.Tensor, stream=None) -> None:
    assert x.dtype == torch.float32
    _ok(load_library().q4probe_update_in_place(x.data_ptr(), x.numel() * 4, _stream(stream)),
        "q4probe_update_in_place")


def read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    assert sink.dtype == torch.int32 and sink.numel() >= load_library().q4probe_read_sink_words()
    _ok(load_library().q4probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                    _stream(stream)), "q4probe_read")
