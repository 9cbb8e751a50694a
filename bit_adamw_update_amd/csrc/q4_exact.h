// q4_exact.h -- device primitives of the 4-bit AdamW step kernels that
// replace an IEEE operation or a plain lane exchange by a shorter sequence
// and must return exactly the same bits.  The kernels (q4_kernels.hip) and
// their self-test library (q4_selftest.hip) both include this header; the
// self-test sweeps every input in each stated range against a check built
// from the definition of correct rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// IEEE (correctly rounded) square root of x from the hardware one, which is
// faithful: the root lies on the side of s that the sign of the exact
// residual x - s s shows (one FMA), and only the neighbour t of s on that
// side can be nearer; the sign of the exact residual x - s t decides it
// (Tuckerman's rounding test).  A zero (or NaN, x = inf) residual leans up,
// where the test then keeps s.  Valid while the residuals cannot underflow:
// x >= 2^-96 (through +inf) and x = 0.
__device__ __forceinline__ float sqrt_rn_normal(float x) {
    const float s = __builtin_amdgcn_sqrtf(x);
    const bool up = !(__builtin_fmaf(-s, s, x) < 0.0f);
    const float t = __uint_as_float(__float_as_uint(s) + (up ? 1u : 0xFFFFFFFFu));
    const bool beyond = __builtin_fmaf(-s, t, x) > 0.0f;  // up: x > s t; down: x <= s t
    return beyond == up ? t : s;
}

// The inverse that normalizes a block, x = value * (1/s), for a block scale
// s >= 0: 0 for a zero scale and for one below the smallest normal float
// (whose reciprocal may overflow; 0 * inf would not be 0), so such blocks
// store the code of zero.  For s in [2^-126, 2^126) the hardware reciprocal
// refined by one FMA Newton step equals the IEEE quotient; a wave with a
// larger scale divides.
__device__ __forceinline__ float inv_scale(float s) {
    const bool normal = s >= 0x1p-126f;
    float r;
    if (__builtin_amdgcn_ballot_w64(s >= 0x1p126f) == 0) {
        const float y = __builtin_amdgcn_rcpf(s);
        r = __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
    } else {
        r = 1.0f / s;
    }
    return normal ? r : 0.0f;
}

// ds_bpermute byte addresses of the 8 nibbles of `codes` for lane row + code,
// rb4x4 = 4 * row (the row's first lane) in every byte: byte j of `ev` is
// 4 * nibble(2j) + 4 * row, of `od` 4 * nibble(2j + 1) + 4 * row (the two
// fields share no bit).  ds_bpermute reads only bits 2..7 of an address, so
// element k takes its word shifted right by 8 * (k / 2): two instructions
// per word, then one shift per element.
struct NibbleAddrs {
    uint32_t ev, od;
};
__device__ __forceinline__ NibbleAddrs nibble_addrs(uint32_t codes, uint32_t rb4x4) {
    return {((codes << 2) & 0x3C3C3C3Cu) | rb4x4, ((codes >> 2) & 0x3C3C3C3Cu) | rb4x4};
}
__device__ __forceinline__ int nibble_addr(const NibbleAddrs& a, int k) {
    return (int)(((k & 1) ? a.od : a.ev) >> (8 * (k >> 1)));
}
__device__ __forceinline__ float bperm_addr(float v, int addr) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
}

}  // namespace q4
