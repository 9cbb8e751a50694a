"""Exhaustive checks of the step kernels' exact primitives (q4_exact.h):

  * sqrt_rn_normal, the hardware square root plus a one-sided Tuckerman
    correction, is the correctly rounded square root at x = 0 and for every
    x in [2^-96, +inf];
  * inv_scale, the hardware reciprocal plus one Newton step, returns the
    correctly rounded 1/s for every s >= 2^-126 (through +inf) and +0 below
    that, for zero and for NaN;
  * clamp_unit, the clamp of a normalized second moment as the kernels form
    it (folded into the multiply), returns x on (0, 1], 1 above, and a zero
    for x <= 0 and for every NaN;
  * the nibble-addressed ds_bpermute decode fetches lane row + code for
    every nibble, and ds_bpermute ignores address bits 0-1 and 8-31;
  * the kernels' Philox4x32-10 (the element-independent products formed
    apart, as the kernels form them) gives the published known-answer
    vectors and the oracle's words on random counters and keys;
  * every round-to-nearest lookup of the step kernels (q4_quant.h: compact
    bucket tables of the five 4-bit maps, the Dyn4 floor table, the flat
    slots of the ZIP-SR kernels, the 8-bit bucket counts) equals the plain
    count of midpoints below x (levels at or below x for the floor) for
    every FP32 x in the lookup's domain, [-1, 1] or [0, 1].

The library checks each result against the definition of correct rounding
(the input must lie strictly between the squares, or reciprocals, of the
result's two midpoints, compared exactly in binary64).  The bare hardware
operations must fail the same check, which shows that it can fail.
"""
import ctypes
import os

import pytest

from bit_adamw_update_amd import build

SQRT, INV_SCALE, SQRT_FAITHFUL, SQRT_SMALL, CLAMP_UNIT = 0, 1, 2, 3, 4
FAST, BARE = 0, 1
F32_INF = 0x7F800000
ONE, NEG_ZERO, NEG_ONE = 0x3F800000, 0x80000000, 0xBF800000
# (name, signed domain) in the library's check order
QUANT_CHECKS = [("rtn_nf4", True), ("rtn_sdyn4", True), ("rtn_dyn4", False), ("rtn_dyn4_nz", False),
                ("rtn_lin4_nz", False), ("floor_dyn4", False), ("flat_nf4", True), ("flat_sdyn4", True),
                ("flat_floor_dyn4", False), ("rtn8_sdyn8", True), ("rtn8_dyn8", False)]


def _lib():
    if not os.path.exists(build.SELFTEST_PATH):
        pytest.fail(f"{build.SELFTEST_PATH} is not built")
    lib = ctypes.CDLL(build.SELFTEST_PATH)
    lib.q4st_sweep.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                               ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_uint32)]
    lib.q4st_sweep.restype = ctypes.c_int
    lib.q4st_nibble_decode.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_ulonglong)]
    lib.q4st_nibble_decode.restype = ctypes.c_int
    lib.q4st_quant_sweep.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.POINTER(ctypes.c_ulonglong), ctypes.POINTER(ctypes.c_uint32)]
    lib.q4st_quant_sweep.restype = ctypes.c_int
    lib.q4st_philox.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32]
    lib.q4st_philox.restype = ctypes.c_int
    return lib


def _sweep(lib, what, form, lo, hi):
    n, first = ctypes.c_ulonglong(0), ctypes.c_uint32(0)
    rc = lib.q4st_sweep(what, form, lo, hi, ctypes.byref(n), ctypes.byref(first))
    assert rc == 0, f"q4st_sweep returned {rc}"
    print(f"sweep what={what} form={form} [{lo:#010x}, {hi:#010x}): {n.value} mismatches, "
          f"first {first.value:#010x}", flush=True)
    return n.value, first.value


def test_selftest_library_exports_and_validates():
    lib = _lib()
    out = os.popen(f"nm -D --defined-only {build.SELFTEST_PATH}").read()
    for sym in ("q4st_sweep", "q4st_nibble_decode", "q4st_quant_sweep", "q4st_philox"):
        assert f" T {sym}" in out
    n, first = ctypes.c_ulonglong(0), ctypes.c_uint32(0)
    # rejected before any device call
    assert lib.q4st_sweep(5, 0, 0, 1, ctypes.byref(n), ctypes.byref(first)) == -1
    assert lib.q4st_sweep(0, 2, 0, 1, ctypes.byref(n), ctypes.byref(first)) == -1
    assert lib.q4st_sweep(0, 0, 5, 4, ctypes.byref(n), ctypes.byref(first)) == -1
    assert lib.q4st_sweep(0, 0, 0, (1 << 32) + 1, ctypes.byref(n), ctypes.byref(first)) == -1
    assert lib.q4st_nibble_decode(1, 6, 0, ctypes.byref(n)) == -1
    assert lib.q4st_nibble_decode(1, 0, 0, ctypes.byref(n)) == -1
    assert lib.q4st_philox(None, None, 1) == -1
    assert lib.q4st_quant_sweep(len(QUANT_CHECKS) + 1, 0, 1, ctypes.byref(n), ctypes.byref(first)) == -1
    # outside [+0, 1], and the negative half for an unsigned map
    assert lib.q4st_quant_sweep(0, 0, ONE + 2, ctypes.byref(n), ctypes.byref(first)) == -1
    assert lib.q4st_quant_sweep(2, NEG_ZERO, NEG_ONE + 1, ctypes.byref(n), ctypes.byref(first)) == -1
    assert lib.q4st_quant_sweep(0, ONE, NEG_ZERO, ctypes.byref(n), ctypes.byref(first)) == -1


@pytest.mark.gpu
def test_sqrt_rn_normal_exhaustive():
    lib = _lib()
    assert _sweep(lib, SQRT, FAST, 0, 1) == (0, 0xFFFFFFFF)                  # x = +0
    assert _sweep(lib, SQRT, FAST, 0x0F800000, F32_INF + 1) == (0, 0xFFFFFFFF)  # [2^-96, +inf]
    # the hardware square root alone is not correctly rounded
    assert _sweep(lib, SQRT, BARE, 0x3F800000, 0x40800000)[0] > 0             # [1, 4)
    # below 2^-96 the residuals underflow and the correction fails, which is
    # why a wave with such an input takes the IEEE square root instead
    assert _sweep(lib, SQRT, FAST, 1, 0x0F800000)[0] > 0


@pytest.mark.gpu
def test_hardware_sqrt_bounds():
    """Where a rule does not decide codes from sqrt(v1), the weight update's
    denominator sqrt(v1) rsbc2 + eps takes the bare hardware square root.
    It is faithful (one of the two floats around sqrt(x)) for +0, every
    normal float and +inf; for every subnormal input it is not, but it stays
    in [0, 2^-63], so the denominator moves by at most 2^-63 rsbc2 there."""
    lib = _lib()
    assert _sweep(lib, SQRT_FAITHFUL, BARE, 0, 1) == (0, 0xFFFFFFFF)
    assert _sweep(lib, SQRT_FAITHFUL, BARE, 0x00800000, F32_INF + 1) == (0, 0xFFFFFFFF)
    assert _sweep(lib, SQRT_FAITHFUL, BARE, 1, 0x00800000)[0] > 0
    assert _sweep(lib, SQRT_SMALL, BARE, 1, 0x00800000) == (0, 0xFFFFFFFF)


@pytest.mark.gpu
def test_clamp_unit_exhaustive():
    """The second moment's clamp over every bit pattern: NaN (and anything
    <= 0) to a zero, so a NaN takes sorted index 0 in every unsigned map."""
    lib = _lib()
    assert _sweep(lib, CLAMP_UNIT, FAST, 0, 1 << 32) == (0, 0xFFFFFFFF)


@pytest.mark.gpu
def test_inv_scale_exhaustive():
    lib = _lib()
    # every s >= +0: zero, subnormal, normal, +inf and NaN bit patterns
    assert _sweep(lib, INV_SCALE, FAST, 0, 0x80000000) == (0, 0xFFFFFFFF)
    # the hardware reciprocal alone is not correctly rounded
    assert _sweep(lib, INV_SCALE, BARE, 0x3F800000, 0x40000000)[0] > 0        # [1, 2)


@pytest.mark.gpu
@pytest.mark.parametrize("form", [FAST, BARE])
def test_nibble_decode(form):
    lib = _lib()
    for seed in (1, 2, 3):
        n = ctypes.c_ulonglong(0)
        assert lib.q4st_nibble_decode(seed, 1 << 16, form, ctypes.byref(n)) == 0
        assert n.value == 0, f"seed {seed}: {n.value} elements fetched the wrong lane"


@pytest.mark.gpu
@pytest.mark.parametrize("check", range(len(QUANT_CHECKS)), ids=[c[0] for c in QUANT_CHECKS])
def test_round_to_nearest_lookups_exhaustive(check):
    lib = _lib()
    name, signed = QUANT_CHECKS[check]
    ranges = [(0, ONE + 1)] + ([(NEG_ZERO, NEG_ONE + 1)] if signed else [])
    for lo, hi in ranges:
        n, first = ctypes.c_ulonglong(0), ctypes.c_uint32(0)
        rc = lib.q4st_quant_sweep(check, lo, hi, ctypes.byref(n), ctypes.byref(first))
        assert rc == 0, f"q4st_quant_sweep returned {rc}"
        print(f"{name} [{lo:#010x}, {hi:#010x}): {n.value} mismatches, first {first.value:#010x}", flush=True)
        assert (n.value, first.value) == (0, 0xFFFFFFFF), name


@pytest.mark.gpu
def test_round_to_nearest_sweep_sees_single_inputs():
    # control: an NF4 lookup that rounds a midpoint up differs from the count
    # at exactly the 15 midpoints, all inside [-1, 1]
    lib = _lib()
    total = 0
    for lo, hi in ((0, ONE + 1), (NEG_ZERO, NEG_ONE + 1)):
        n, first = ctypes.c_ulonglong(0), ctypes.c_uint32(0)
        assert lib.q4st_quant_sweep(len(QUANT_CHECKS), lo, hi, ctypes.byref(n), ctypes.byref(first)) == 0
        total += n.value
    assert total == 15


@pytest.mark.gpu
def test_philox_known_answers_and_oracle():
    import numpy as np
    import torch

    from oracle import oracle as O
    golden = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    kat = [[int(x, 16) for x in l.split()] for l in open(golden) if l.strip() and not l.startswith("#")]
    rng = np.random.default_rng(7)
    rand = rng.integers(0, 2 ** 32, size=(1 << 16, 6), dtype=np.uint64).astype(np.uint32)
    rows = np.concatenate([np.array([r[:6] for r in kat], np.uint32), rand])
    dev_in = torch.from_numpy(rows.view(np.int32).copy()).cuda()
    dev_out = torch.empty((rows.shape[0], 4), dtype=torch.int32, device="cuda")
    assert lib_call(_lib().q4st_philox, dev_in.data_ptr(), dev_out.data_ptr(), rows.shape[0]) == 0
    got = dev_out.cpu().numpy().view(np.uint32)
    for k, r in enumerate(kat):
        assert got[k].tolist() == r[6:10], f"known-answer vector {k}"
    for k in range(len(kat), rows.shape[0]):
        assert np.array_equal(got[k], O.philox(rows[k, :4], rows[k, 4:6])), f"row {k}: {rows[k]}"


def lib_call(fn, *args):
    import torch
    rc = fn(*args)
    torch.cuda.synchronize()
    return rc
