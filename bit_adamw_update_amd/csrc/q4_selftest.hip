// q4_selftest.hip -- exhaustive checks of the primitives in q4_exact.h, built
// as a library of its own (libq4selftest.so) that only the tests load.
//
// Correct rounding is checked from its definition, not against another
// implementation: a finite y > 0 is the nearest float to a real z > 0 iff z
// lies strictly between the midpoints of y and its two float neighbours
// (neither square roots nor reciprocals of floats ever fall on a midpoint).
// A midpoint has at most 25 significant bits, so its square (50 bits) and
// its product with a float (49 bits) are exact in binary64, and so is each
// comparison below.

#include <stdint.h>

#include "q4_exact.h"

namespace {

constexpr int kWhatSqrt = 0, kWhatInvScale = 1;
constexpr int kFormFast = 0, kFormHardware = 1;

__device__ __forceinline__ double mid_below(uint32_t y) {
    return 0.5 * ((double)__uint_as_float(y - 1u) + (double)__uint_as_float(y));
}
__device__ __forceinline__ double mid_above(uint32_t y) {
    const double up = y + 1u == 0x7F800000u ? 0x1p128 : (double)__uint_as_float(y + 1u);
    return 0.5 * ((double)__uint_as_float(y) + up);
}
__device__ __forceinline__ bool finite_positive(uint32_t y) { return y != 0u && y < 0x7F800000u; }

// y == RN(sqrt(x)) for x = +0, +inf and every finite x > 0
__device__ bool is_sqrt_rn(uint32_t x, uint32_t y) {
    if (x == 0u || x == 0x7F800000u) return y == x;
    if (!finite_positive(y)) return false;
    const double lo = mid_below(y), hi = mid_above(y), xd = (double)__uint_as_float(x);
    return lo * lo < xd && xd < hi * hi;
}
// y == (s >= 2^-126 ? RN(1/s) : +0) for every s >= +0, NaN included (-> +0)
__device__ bool is_inv_scale(uint32_t s, uint32_t y) {
    const float sf = __uint_as_float(s);
    if (!(sf >= 0x1p-126f) || s == 0x7F800000u) return y == 0u;
    if (!finite_positive(y)) return false;
    const double lo = mid_below(y), hi = mid_above(y), sd = (double)sf;
    return lo * sd < 1.0 && 1.0 < hi * sd;
}

template <int WHAT, int FORM>
__global__ void __launch_bounds__(256) k_sweep(uint64_t lo, uint64_t hi, unsigned long long* bad,
                                               uint32_t* first_bad) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t n = 0, first = 0xFFFFFFFFu;
    for (uint64_t i = lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi; i += stride) {
        const uint32_t b = (uint32_t)i;
        const float x = __uint_as_float(b);
        bool ok;
        if constexpr (WHAT == kWhatSqrt) {
            const float r = FORM == kFormFast ? q4::sqrt_rn_normal(x) : __builtin_amdgcn_sqrtf(x);
            ok = is_sqrt_rn(b, __float_as_uint(r));
        } else {
            const float r = FORM == kFormFast ? q4::inv_scale(x) : (x >= 0x1p-126f ? __builtin_amdgcn_rcpf(x) : 0.0f);
            ok = is_inv_scale(b, __float_as_uint(r));
        }
        if (!ok) {
            ++n;
            first = min(first, b);
        }
    }
    if (n != 0) {
        atomicAdd(bad, (unsigned long long)n);
        atomicMin(first_bad, first);
    }
}

// Each lane holds 2 * lane + 1 and a random word of 8 nibbles; element k
// must fetch the value of lane (row's first lane) + nibble k.
template <int FORM>
__global__ void __launch_bounds__(256) k_nibble(uint64_t seed, unsigned long long* bad) {
    const int lane = threadIdx.x & 63;
    const uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // splitmix64 of (seed, thread): the codes, and junk for the upper address bits
    uint64_t z = seed + 0x9E3779B97F4A7C15ull * (2 * gid + 1);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    const uint32_t codes = (uint32_t)z, junk = (uint32_t)(z >> 32);
    const int row_base = lane & 48;
    const float own = (float)(2 * lane + 1);
    const q4::NibbleAddrs a = q4::nibble_addrs(codes, ((uint32_t)row_base << 2) * 0x01010101u);
    uint32_t n = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int src = row_base + (int)((codes >> (4 * k)) & 15u);
        const int addr = FORM == kFormFast ? q4::nibble_addr(a, k)
                                           : (int)(((uint32_t)src << 2) | ((junk >> k) & 0xFFFFFF03u));
        const float got = q4::bperm_addr(own, addr);
        n += got == (float)(2 * src + 1) ? 0u : 1u;
    }
    if (n != 0) atomicAdd(bad, (unsigned long long)n);
}

struct DevCounters {
    unsigned long long* bad = nullptr;
    uint32_t* first = nullptr;
    ~DevCounters() {
        if (bad) (void)hipFree(bad);
        if (first) (void)hipFree(first);
    }
    hipError_t init() {
        hipError_t e = hipMalloc(&bad, sizeof(*bad));
        if (e == hipSuccess) e = hipMalloc(&first, sizeof(*first));
        if (e == hipSuccess) e = hipMemset(bad, 0, sizeof(*bad));
        if (e == hipSuccess) e = hipMemset(first, 0xFF, sizeof(*first));
        return e;
    }
};

constexpr int kGrid = 4096, kThreads = 256;

}  // namespace

extern "C" {

// Checks q4::sqrt_rn_normal (what 0) or q4::inv_scale (what 1) on every
// float bit pattern in [lo, hi) (hi <= 2^32) against the definition above;
// form 1 checks the bare hardware square root or reciprocal instead, which
// is not correctly rounded.  Writes the number of inputs whose result
// differs and the smallest such bit pattern (0xFFFFFFFF if none) to host
// memory.  Returns 0, -1 for invalid arguments, or a HIP error code.
// Synchronous, on the current device's null stream.
int q4st_sweep(int what, int form, uint64_t lo, uint64_t hi, unsigned long long* mismatches,
               uint32_t* first_bad) {
    if (what < 0 || what > 1 || form < 0 || form > 1 || lo > hi || hi > (1ull << 32) || !mismatches ||
        !first_bad)
        return -1;
    DevCounters c;
    hipError_t e = c.init();
    if (e != hipSuccess) return (int)e;
    if (hi > lo) {
        if (what == kWhatSqrt && form == kFormFast)
            k_sweep<kWhatSqrt, kFormFast><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        else if (what == kWhatSqrt)
            k_sweep<kWhatSqrt, kFormHardware><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        else if (form == kFormFast)
            k_sweep<kWhatInvScale, kFormFast><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        else
            k_sweep<kWhatInvScale, kFormHardware><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) return (int)e;
    }
    e = hipMemcpy(mismatches, c.bad, sizeof(*mismatches), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(first_bad, c.first, sizeof(*first_bad), hipMemcpyDeviceToHost);
    return (int)e;
}

// Decodes 8 random nibbles per lane over `waves` full wavefronts through
// q4::nibble_addrs / nibble_addr / bperm_addr (form 0), or through clean
// lane addresses with random bits 0-1 and 8-31 (form 1), and writes the
// number of elements that fetched the wrong lane.  waves must be a
// positive multiple of 4.  Returns 0, -1 for invalid arguments, or a HIP
// error code.  Synchronous.
int q4st_nibble_decode(uint64_t seed, uint32_t waves, int form, unsigned long long* mismatches) {
    if (form < 0 || form > 1 || waves == 0 || waves % 4 != 0 || waves > (1u << 20) || !mismatches) return -1;
    DevCounters c;
    hipError_t e = c.init();
    if (e != hipSuccess) return (int)e;
    if (form == kFormFast)
        k_nibble<kFormFast><<<waves / 4, kThreads>>>(seed, c.bad);
    else
        k_nibble<kFormHardware><<<waves / 4, kThreads>>>(seed, c.bad);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(mismatches, c.bad, sizeof(*mismatches), hipMemcpyDeviceToHost);
    return (int)e;
}

}  // extern "C"
