// q4_exact.h -- device primitives of the 4-bit AdamW step kernels that
// replace an IEEE operation or a plain lane exchange by a shorter sequence
// and must return exactly the same bits, and the counter-based generator
// whose words the stochastic-rounding rules draw.  The kernels
// (q4_kernels.hip) and their self-test library (q4_selftest.hip) both
// include this header; the self-test sweeps every input in each stated range
// against a check built from the definition of correct rounding, and runs
// the generator on published known-answer vectors.
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
// s >= 0: the IEEE reciprocal, or 0 for a zero scale and for a scale whose
// reciprocal overflows (s <= 2^-128), which has no usable normalization
// (value * inf is infinite, 0 * inf is NaN), so such blocks store the code of
// zero.  For s in [2^-126, 2^126) the hardware reciprocal refined by one FMA
// Newton step equals the IEEE quotient; a wave holding any other non-zero
// scale (subnormal, or 2^126 and up) divides.
__device__ __forceinline__ float inv_scale(float s) {
    const bool fast = (s >= 0x1p-126f && s < 0x1p126f) || s == 0.0f;
    float r;
    if (__builtin_amdgcn_ballot_w64(!fast) == 0) {
        const float y = __builtin_amdgcn_rcpf(s);
        r = __builtin_fmaf(__builtin_fmaf(-s, y, 1.0f), y, y);
    } else {
        r = 1.0f / s;
    }
    // +inf (overflow, or s = 0 divided) and NaN (s = 0 through the Newton
    // step) both fail the compare
    return r <= 0x1.fffffep127f ? r : 0.0f;
}

// The clamp of a normalized second moment, v * (1/s) (+0 or more, or NaN),
// to the level range [0, 1], with NaN sent to 0: the stored second moment
// takes sorted index 0 for a NaN under every rule, and 0 has sorted index 0
// in every unsigned map.  v_med3_f32 with a NaN operand returns the smallest
// of the others, and the compiler folds med3(x, 0, 1) into the clamp bit of
// the multiply that forms x (NaN to 0 in the kernels' clamp mode); checked
// in that form over every input.
__device__ __forceinline__ float clamp_unit(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 1.0f); }
// v * inv clamped as above.  Written as v * inv + 0, which rounds as the
// product does (v * inv >= +0, so adding +0 changes no bit), so that the
// multiply-add carries the clamp even where the plain product is shared.
__device__ __forceinline__ float normalize_v(float v, float inv) { return clamp_unit(__builtin_fmaf(v, inv, 0.0f)); }

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

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies with the published multipliers, the key bumped by the
// published Weyl constants between rounds.  On gfx950 each product is one
// v_mad_u64_u32 and each three-way XOR one v_bitop3_b32 (truth table 0x96).
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// The counter is (x, step, tensor, stream) with x the only word that differs
// between elements.  Round 1 multiplies the tensor word and round 2 the word
// that round 1 made from it and the step, so those two products, and the
// words that only they and the key feed, are the same for every element of
// a tensor; philox_fixed forms them once (scalar registers) and philox_from
// finishes the ten rounds for one x.
struct PhiloxFixed {
    uint32_t y1k;   // round 1's y = lo(M1 tensor), xor round 2's k0
    uint32_t hq0k;  // hi(M0 x1) of round 2, xor round 2's k1
    uint32_t lq0;   // lo(M0 x1): round 2's w
};
__device__ __forceinline__ PhiloxFixed philox_fixed(uint32_t step, uint32_t tid, uint32_t k0, uint32_t k1) {
    const uint64_t p1 = (uint64_t)kPhiloxM1 * tid;
    const uint32_t x1 = (uint32_t)(p1 >> 32) ^ step ^ k0;  // round 1's x
    const uint64_t q0 = (uint64_t)kPhiloxM0 * x1;
    return {(uint32_t)p1 ^ (k0 + kPhiloxW0), (uint32_t)(q0 >> 32) ^ (k1 + kPhiloxW1), (uint32_t)q0};
}
__device__ __forceinline__ uint4 philox_from(uint32_t x, uint32_t stream, const PhiloxFixed& f, uint32_t k0,
                                             uint32_t k1) {
    // round 1: z = hi(M0 x) ^ stream ^ k1, w = lo(M0 x)
    const uint64_t p0 = (uint64_t)kPhiloxM0 * x;
    const uint32_t z1 = (uint32_t)(p0 >> 32) ^ (stream ^ k1);
    // round 2: x = hi(M1 z) ^ y ^ k0', y = lo(M1 z), z = hi(M0 x1) ^ w ^ k1', w = lo(M0 x1)
    const uint64_t p1 = (uint64_t)kPhiloxM1 * z1;
    uint4 c = make_uint4((uint32_t)(p1 >> 32) ^ f.y1k, (uint32_t)p1, (uint32_t)p0 ^ f.hq0k, f.lq0);
    // rounds 3 .. 10 with keys k + r W, r = 2 .. 9
    k0 += 2u * kPhiloxW0;
    k1 += 2u * kPhiloxW1;
#pragma unroll
    for (int r = 2; r < 10; ++r) {
        if (r > 2) { k0 += kPhiloxW0; k1 += kPhiloxW1; }
        const uint64_t q0 = (uint64_t)kPhiloxM0 * c.x;
        const uint64_t q1 = (uint64_t)kPhiloxM1 * c.z;
        c = make_uint4(xor3((uint32_t)(q1 >> 32), c.y, k0), (uint32_t)q1, xor3((uint32_t)(q0 >> 32), c.w, k1),
                       (uint32_t)q0);
    }
    return c;
}

// Element i draws word i mod 4 of Philox(ctr = (i/4, step, tensor, stream)),
// its top 24 bits scaled by 2^-24.  uniforms4 gives the 4 uniforms of
// elements 4c .. 4c+3.
__device__ __forceinline__ void uniforms4(uint32_t c, uint32_t stream, const PhiloxFixed& f, uint32_t k0,
                                          uint32_t k1, float u[4]) {
    const uint4 a = philox_from(c, stream, f, k0, k1);
    const float s = 5.9604644775390625e-8f;  // 2^-24
    u[0] = (float)(a.x >> 8) * s; u[1] = (float)(a.y >> 8) * s;
    u[2] = (float)(a.z >> 8) * s; u[3] = (float)(a.w >> 8) * s;
}

}  // namespace q4
