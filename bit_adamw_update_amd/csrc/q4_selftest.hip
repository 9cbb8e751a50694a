// q4_selftest.hip -- exhaustive checks of the primitives in q4_exact.h and of
// the round-to-nearest tables in q4_quant.h, built as a library of its own
// (libq4selftest.so) that only the tests load.
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
#include "q4_quant.h"

namespace {

constexpr int kWhatSqrt = 0, kWhatInvScale = 1, kWhatSqrtFaithful = 2, kWhatSqrtSmall = 3, kWhatClampUnit = 4;
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
// y is one of the two floats around sqrt(x) (a faithful square root): x = +0
// and +inf give themselves, and otherwise sqrt(x) lies strictly between the
// float neighbours of y, i.e. prev(y)^2 < x < next(y)^2 (exact in binary64).
// Every sqrt(x) of a positive float is a normal float, so prev(y) is too.
__device__ bool is_sqrt_faithful(uint32_t x, uint32_t y) {
    if (x == 0u || x == 0x7F800000u) return y == x;
    if (!finite_positive(y) || y <= 0x00800000u) return false;
    const double lo = (double)__uint_as_float(y - 1u);
    const double hi = y + 1u == 0x7F800000u ? 0x1p128 : (double)__uint_as_float(y + 1u);
    const double xd = (double)__uint_as_float(x);
    return lo * lo < xd && xd < hi * hi;
}

// For a subnormal x: 0 <= y <= 2^-63 (every root of a subnormal is below
// 2^-63), i.e. the hardware root is off by less than 2^-63 in absolute terms.
__device__ bool is_sqrt_small(uint32_t x, uint32_t y) {
    (void)x;
    const float yf = __uint_as_float(y);
    return yf >= 0.0f && yf <= 0x1p-63f;
}

// The clamp of a normalized second moment: y = x for x in (0, 1], 1 above,
// a zero for x <= 0 and for every NaN (the kernels send NaN to 0).
__device__ bool is_clamp_unit(uint32_t x, uint32_t y) {
    const float xf = __uint_as_float(x), yf = __uint_as_float(y);
    if (xf != xf || xf <= 0.0f) return yf == 0.0f;
    if (xf >= 1.0f) return y == 0x3F800000u;
    return y == x;
}

// y == RN(1/s) when s > 0 and RN(1/s) is finite, else +0, for every s >= +0,
// +inf and NaN included (-> +0).  RN(1/s) overflows iff 1/s reaches the
// midpoint 2^128 - 2^103 between the largest float and 2^128, i.e. iff
// s * (2^128 - 2^103) <= 1 (exact in binary64: 24 x 25 significant bits).
__device__ bool is_inv_scale(uint32_t s, uint32_t y) {
    const float sf = __uint_as_float(s);
    if (!(sf > 0.0f) || s == 0x7F800000u) return y == 0u;
    const double sd = (double)sf;
    if (sd * (0x1p128 - 0x1p103) <= 1.0) return y == 0u;
    if (!finite_positive(y)) return false;
    const double lo = mid_below(y), hi = mid_above(y);
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
        } else if constexpr (WHAT == kWhatSqrtFaithful) {
            ok = is_sqrt_faithful(b, __float_as_uint(__builtin_amdgcn_sqrtf(x)));
        } else if constexpr (WHAT == kWhatSqrtSmall) {
            ok = is_sqrt_small(b, __float_as_uint(__builtin_amdgcn_sqrtf(x)));
        } else if constexpr (WHAT == kWhatClampUnit) {
            // in the kernels' forms: the clamp of a product and of the
            // multiply-add (one = 1.0f at run time; the multiply cannot
            // fold away)
            const float one = __uint_as_float(0x3F800000u | (uint32_t)(lo >> 63));
            ok = is_clamp_unit(b, __float_as_uint(q4::clamp_unit(x * one))) &&
                 is_clamp_unit(b, __float_as_uint(q4::normalize_v(x, one)));
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


// ---------------------------------------------------------------------------
// Round-to-nearest tables against plain counts
// ---------------------------------------------------------------------------
//
// Each check takes the lookup the step kernels make (tables staged in LDS as
// they stage them) and compares it with the definition: the RTN index of x
// is the number of FP32 midpoints strictly below x, the floor index the
// number of levels <= x less one.  The 4-bit counts run over the codebook's
// 15 midpoints for every x.  The 8-bit counts keep a pointer into the sorted
// midpoints that follows x through a run of consecutive bit patterns (x
// rises through positive patterns and falls through negative ones); each
// run starts from, and ends checked against, a count over all midpoints.

enum QuantCheck {
    QC_RTN_NF4 = 0, QC_RTN_SDYN4, QC_RTN_DYN4, QC_RTN_DYN4_NZ, QC_RTN_LIN4_NZ,  // compact tables
    QC_FLOOR_DYN4,                  // compact floor table of Dyn4
    QC_FLAT_NF4, QC_FLAT_SDYN4,     // flat m slots
    QC_FLAT_FLOOR,                  // flat Dyn4 floor slots
    QC_RTN8_M, QC_RTN8_V,           // 8-bit bucket counts
    QC_CONTROL_NF4_TIES_UP,         // control: NF4 lookup that rounds midpoints up
    QC_COUNT
};
constexpr int kRun = 4096;  // bit patterns per thread

__host__ __device__ constexpr bool qc_signed(int c) {
    return c == QC_RTN_NF4 || c == QC_RTN_SDYN4 || c == QC_FLAT_NF4 || c == QC_FLAT_SDYN4 || c == QC_RTN8_M ||
           c == QC_CONTROL_NF4_TIES_UP;
}

template <int CB> __device__ __forceinline__ int plain_rtn4(float x) {
    int n = 0;
#pragma unroll
    for (int k = 0; k + 1 < q4::Book<CB>::N; ++k) n += q4::Book<CB>::mid(k) < x ? 1 : 0;
    return n;
}
__device__ __forceinline__ int plain_floor_dyn4(float x) {
    int n = 0;
#pragma unroll
    for (int k = 0; k < q4::Book<Q4_CB_DYN4>::N; ++k) n += q4::Book<Q4_CB_DYN4>::level(k) <= x ? 1 : 0;
    return n - 1;
}

struct QuantLds {
    q4::BucketEntry enc[q4::Enc<Q4_CB_NF4>::SIZE > q4::Enc<Q4_CB_SDYN4>::SIZE ? q4::Enc<Q4_CB_NF4>::SIZE
                                                                                : q4::Enc<Q4_CB_SDYN4>::SIZE];
    q4::FloorEntry floor[q4::Enc<Q4_CB_DYN4>::NPOS];
    alignas(16) q4::BucketEntry flat[q4::kFlatAlloc];
    q4::Step8Lds t8;
    float mids8[256];  // the 8-bit map's midpoints ascending, from its decoded levels
};
static_assert(q4::Enc<Q4_CB_DYN4>::SIZE <= q4::Enc<Q4_CB_NF4>::SIZE && q4::Enc<Q4_CB_DYN4_NZ>::SIZE <= q4::Enc<Q4_CB_NF4>::SIZE &&
                  q4::Enc<Q4_CB_LIN4_NZ>::SIZE <= q4::Enc<Q4_CB_NF4>::SIZE,
              "the staging array must hold every compact table");

// Check one x of a 4-bit map; returns true when the lookup equals the count.
template <int CHECK> __device__ __forceinline__ bool check4(const QuantLds& L, float x) {
    if constexpr (CHECK <= QC_RTN_LIN4_NZ) {
        return q4::rtn_index(q4::bucket_of<CHECK>(L.enc, x), x) == plain_rtn4<CHECK>(x);
    } else if constexpr (CHECK == QC_FLOOR_DYN4 || CHECK == QC_FLAT_FLOOR) {
        float thr;
        int lo;
        if constexpr (CHECK == QC_FLOOR_DYN4) {
            const q4::FloorEntry& f = L.floor[q4::bucket_index<Q4_CB_DYN4>(x)];
            thr = f.thr;
            lo = f.lo;
        } else {
            const q4::BucketEntry& f = L.flat[q4::flat_floor_slot(x)];
            thr = f.thr;
            lo = f.base;
        }
        const int want = plain_floor_dyn4(x);
        // the kernels also take "x is a level" from the entry: x == thr
        return q4::floor_index(thr, lo, x) == want && (x == thr) == (x == q4::Book<Q4_CB_DYN4>::level(want));
    } else if constexpr (CHECK == QC_CONTROL_NF4_TIES_UP) {
        // differs from the count exactly at the 15 midpoints
        const q4::BucketEntry& e = q4::bucket_of<Q4_CB_NF4>(L.enc, x);
        return e.base + (x >= e.thr ? 1 : 0) == plain_rtn4<Q4_CB_NF4>(x);
    } else {
        constexpr int CB = CHECK == QC_FLAT_NF4 ? Q4_CB_NF4 : Q4_CB_SDYN4;
        return q4::rtn_index(L.flat[q4::flat_m_slot(x)], x) == plain_rtn4<CB>(x);
    }
}

template <int CHECK>
__global__ void __launch_bounds__(256) k_quant(uint64_t lo, uint64_t hi, unsigned long long* bad, uint32_t* first_bad) {
    __shared__ QuantLds L;
    const int t = threadIdx.x;
    if constexpr (CHECK <= QC_RTN_LIN4_NZ) {
        for (int i = t; i < q4::Enc<CHECK>::SIZE; i += blockDim.x) L.enc[i] = q4::enc_table_global<CHECK>()[i];
    } else if constexpr (CHECK == QC_CONTROL_NF4_TIES_UP) {
        for (int i = t; i < q4::Enc<Q4_CB_NF4>::SIZE; i += blockDim.x) L.enc[i] = q4::enc_table_global<Q4_CB_NF4>()[i];
    } else if constexpr (CHECK == QC_FLOOR_DYN4) {
        for (int i = t; i < q4::Enc<Q4_CB_DYN4>::NPOS; i += blockDim.x) L.floor[i] = q4::c_floor_dyn4.e[i];
    } else if constexpr (CHECK == QC_FLAT_NF4 || CHECK == QC_FLAT_FLOOR) {
        q4::copy_flat_table<Q4_CB_NF4>(L.flat);     // the copy the step kernels make
    } else if constexpr (CHECK == QC_FLAT_SDYN4) {
        q4::copy_flat_table<Q4_CB_SDYN4>(L.flat);
    }
    constexpr bool EIGHT = CHECK == QC_RTN8_M || CHECK == QC_RTN8_V;
    constexpr int NMID = CHECK == QC_RTN8_M ? 254 : 255;
    if constexpr (EIGHT) {
        q4::step8_tables(L.t8);  // synchronizes the group
        // ascending levels as decoded: SDyn8 from its most negative code
        // (0x80 | 127) through 0x80 | 1, then codes 0 .. 127; Dyn8 codes 0 .. 255
        auto level = [](int j) {
            if constexpr (CHECK == QC_RTN8_M)
                return q4::bits2f(q4::c_cb8[0][j < 127 ? (0x80 | (127 - j)) : (j - 127)]);
            else
                return q4::bits2f(q4::c_cb8[1][j]);
        };
        if (t < NMID) L.mids8[t] = (level(t) + level(t + 1)) * 0.5f;
    }
    __syncthreads();

    const uint64_t r0 = lo + ((uint64_t)blockIdx.x * blockDim.x + t) * kRun;
    if (r0 >= hi) return;
    const uint64_t r1 = r0 + kRun < hi ? r0 + kRun : hi;
    uint32_t n = 0, first = 0xFFFFFFFFu;
    if constexpr (!EIGHT) {
        for (uint64_t i = r0; i < r1; ++i) {
            const uint32_t b = (uint32_t)i;
            if (!check4<CHECK>(L, __uint_as_float(b))) {
                ++n;
                first = min(first, b);
            }
        }
    } else {
        auto full_count = [&](float x) {
            int c = 0;
            for (int j = 0; j < NMID; ++j) c += L.mids8[j] < x ? 1 : 0;
            return c;
        };
        auto code_of = [](int idx) -> uint32_t {
            if constexpr (CHECK == QC_RTN8_M) return idx >= 127 ? (uint32_t)(idx - 127) : 0x80u | (uint32_t)(127 - idx);
            else return (uint32_t)idx;
        };
        const bool neg = ((uint32_t)r0 >> 31) != 0;
        int j = full_count(__uint_as_float((uint32_t)r0));
        for (uint64_t i = r0; i < r1; ++i) {
            const uint32_t b = (uint32_t)i;
            const float x = __uint_as_float(b);
            if (neg) {
                while (j > 0 && !(L.mids8[j - 1] < x)) --j;
            } else {
                while (j < NMID && L.mids8[j] < x) ++j;
            }
            const uint32_t got = CHECK == QC_RTN8_M ? q4::rtn8_m(L.t8, x) : q4::rtn8_v(L.t8, x);
            if (got != code_of(j)) {
                ++n;
                first = min(first, b);
            }
        }
        // the pointer must agree with a fresh count at the end of the run
        if (j != full_count(__uint_as_float((uint32_t)(r1 - 1)))) {
            ++n;
            first = min(first, (uint32_t)(r1 - 1));
        }
    }
    if (n != 0) {
        atomicAdd(bad, (unsigned long long)n);
        atomicMin(first_bad, first);
    }
}

template <int C> void launch_quant(uint64_t lo, uint64_t hi, unsigned long long* bad, uint32_t* first) {
    const uint64_t runs = (hi - lo + kRun - 1) / kRun;
    k_quant<C><<<(unsigned)((runs + 255) / 256), 256>>>(lo, hi, bad, first);
}

__global__ void __launch_bounds__(256) k_philox(const uint32_t* __restrict__ in, uint32_t* __restrict__ out,
                                                uint32_t n) {
    const uint32_t i = blockIdx.x * 256u + threadIdx.x;
    if (i >= n) return;
    const uint32_t* r = in + 6u * i;
    const q4::PhiloxFixed f = q4::philox_fixed(r[1], r[2], r[4], r[5]);
    const uint4 w = q4::philox_from(r[0], r[3], f, r[4], r[5]);
    out[4u * i] = w.x;
    out[4u * i + 1] = w.y;
    out[4u * i + 2] = w.z;
    out[4u * i + 3] = w.w;
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
// is not correctly rounded.  What 2 checks that the bare hardware square
// root is faithful, what 3 that it is in [0, 2^-63] (for subnormal inputs;
// form ignored).  Writes the number of inputs whose result
// differs and the smallest such bit pattern (0xFFFFFFFF if none) to host
// memory.  Returns 0, -1 for invalid arguments, or a HIP error code.
// Synchronous, on the current device's null stream.
int q4st_sweep(int what, int form, uint64_t lo, uint64_t hi, unsigned long long* mismatches,
               uint32_t* first_bad) {
    if (what < 0 || what > 4 || form < 0 || form > 1 || lo > hi || hi > (1ull << 32) || !mismatches ||
        !first_bad)
        return -1;
    DevCounters c;
    hipError_t e = c.init();
    if (e != hipSuccess) return (int)e;
    if (hi > lo) {
        if (what == kWhatClampUnit)
            k_sweep<kWhatClampUnit, kFormFast><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        else if (what == kWhatSqrtFaithful)
            k_sweep<kWhatSqrtFaithful, kFormHardware><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        else if (what == kWhatSqrtSmall)
            k_sweep<kWhatSqrtSmall, kFormHardware><<<kGrid, kThreads>>>(lo, hi, c.bad, c.first);
        else if (what == kWhatSqrt && form == kFormFast)
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

// Checks one round-to-nearest lookup of the step kernels (check: 0-4 the
// compact RTN tables of codebooks 0-4, 5 the compact Dyn4 floor table, 6-7
// the flat m slots of NF4 and SDyn4, 8 the flat Dyn4 floor slots, 9-10 the
// 8-bit SDyn8 and Dyn8 counts; 11 is a control, an NF4 lookup that rounds
// a midpoint up) over every float bit pattern in [lo, hi)
// against the plain count.  [lo, hi) must lie inside the lookup's domain:
// the patterns of [+0, 1] (0 .. 0x3F800001), or for a signed map also those
// of [-1, -0] (0x80000000 .. 0xBF800001).  Writes the number of inputs whose
// lookup differs and the smallest such pattern (0xFFFFFFFF if none).
// Returns 0, -1 for invalid arguments, or a HIP error code.  Synchronous.
int q4st_quant_sweep(int check, uint64_t lo, uint64_t hi, unsigned long long* mismatches, uint32_t* first_bad) {
    if (check < 0 || check >= QC_COUNT || lo > hi || !mismatches || !first_bad) return -1;
    const bool pos = hi <= 0x3F800001ull;
    const bool negr = lo >= 0x80000000ull && hi <= 0xBF800001ull;
    if (!(pos || (negr && qc_signed(check)))) return -1;
    DevCounters c;
    hipError_t e = c.init();
    if (e != hipSuccess) return (int)e;
    if (hi > lo) {
        switch (check) {
        case QC_RTN_NF4: launch_quant<QC_RTN_NF4>(lo, hi, c.bad, c.first); break;
        case QC_RTN_SDYN4: launch_quant<QC_RTN_SDYN4>(lo, hi, c.bad, c.first); break;
        case QC_RTN_DYN4: launch_quant<QC_RTN_DYN4>(lo, hi, c.bad, c.first); break;
        case QC_RTN_DYN4_NZ: launch_quant<QC_RTN_DYN4_NZ>(lo, hi, c.bad, c.first); break;
        case QC_RTN_LIN4_NZ: launch_quant<QC_RTN_LIN4_NZ>(lo, hi, c.bad, c.first); break;
        case QC_FLOOR_DYN4: launch_quant<QC_FLOOR_DYN4>(lo, hi, c.bad, c.first); break;
        case QC_FLAT_NF4: launch_quant<QC_FLAT_NF4>(lo, hi, c.bad, c.first); break;
        case QC_FLAT_SDYN4: launch_quant<QC_FLAT_SDYN4>(lo, hi, c.bad, c.first); break;
        case QC_FLAT_FLOOR: launch_quant<QC_FLAT_FLOOR>(lo, hi, c.bad, c.first); break;
        case QC_RTN8_M: launch_quant<QC_RTN8_M>(lo, hi, c.bad, c.first); break;
        case QC_RTN8_V: launch_quant<QC_RTN8_V>(lo, hi, c.bad, c.first); break;
        default: launch_quant<QC_CONTROL_NF4_TIES_UP>(lo, hi, c.bad, c.first); break;
        }
        e = hipGetLastError();
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) return (int)e;
    }
    e = hipMemcpy(mismatches, c.bad, sizeof(*mismatches), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(first_bad, c.first, sizeof(*first_bad), hipMemcpyDeviceToHost);
    return (int)e;
}

// Philox4x32-10 through q4::philox_fixed / philox_from, the form the step
// kernels use, for n (counter, key) pairs: in (device) holds n rows of
// {ctr0, ctr1, ctr2, ctr3, key0, key1}, out (device) receives n rows of the
// 4 output words.  Returns 0, -1 for invalid arguments, or a HIP error code.
// Synchronous.
int q4st_philox(const uint32_t* in, uint32_t* out, uint32_t n) {
    if (!in || !out || n == 0 || n > (1u << 24)) return -1;
    k_philox<<<(n + 255) / 256, 256>>>(in, out, n);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return (int)e;
}

}  // extern "C"
