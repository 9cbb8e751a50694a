// q4_quant.h -- codebooks and the round-to-nearest machinery of the step
// kernels: the compile-time bucket tables that turn "the number of FP32
// midpoints strictly below x" into one table read and one compare, their
// flat layout for the ZIP-SR kernels, and the 8-bit tables.  Included by
// q4_kernels.hip and by the self-test library (q4_selftest.hip), which
// compares every lookup here with a plain count over every FP32 input in
// [-1, 1] (signed maps) or [0, 1] (unsigned maps).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/q4adamw.h"
#include "q4_codebooks.inc"

namespace q4 {

// ---------------------------------------------------------------------------
// Codebooks
// ---------------------------------------------------------------------------

__host__ __device__ constexpr float bits2f(uint32_t b) { return __builtin_bit_cast(float, b); }

template <int CB> struct CbBits;
template <> struct CbBits<Q4_CB_NF4> { static constexpr uint32_t b[16] = Q4_CB_BITS_NF4; };
template <> struct CbBits<Q4_CB_SDYN4> { static constexpr uint32_t b[16] = Q4_CB_BITS_SDYN4; };
template <> struct CbBits<Q4_CB_DYN4> { static constexpr uint32_t b[16] = Q4_CB_BITS_DYN4; };
template <> struct CbBits<Q4_CB_DYN4_NZ> { static constexpr uint32_t b[16] = Q4_CB_BITS_DYN4_NZ; };
template <> struct CbBits<Q4_CB_LIN4_NZ> { static constexpr uint32_t b[16] = Q4_CB_BITS_LIN4_NZ; };

// Sorted view of a codebook: N distinct levels ascending; code_of maps a
// sorted index to its code (identity except for the sign-magnitude SDyn4,
// whose "-0" code 8 is never produced).
template <int CB> struct Book {
    static constexpr int N = CB == Q4_CB_SDYN4 ? 15 : 16;
    static constexpr int code_of(int k) {
        return CB == Q4_CB_SDYN4 ? (k < 7 ? 15 - k : (k == 7 ? 0 : k - 7)) : k;
    }
    static constexpr float level(int k) { return bits2f(CbBits<CB>::b[code_of(k)]); }
    // FP32 midpoint of adjacent levels; an exact midpoint rounds down.
    static constexpr float mid(int k) { return (level(k) + level(k + 1)) * 0.5f; }
};

static constexpr bool sorted_ok(int cb) {
    // levels strictly increasing and every midpoint strictly inside its cell
    switch (cb) {
#define Q4_CHECK(CB)                                                                             \
    case CB:                                                                                     \
        for (int k = 0; k + 1 < Book<CB>::N; ++k)                                                \
            if (!(Book<CB>::level(k) < Book<CB>::mid(k) && Book<CB>::mid(k) < Book<CB>::level(k + 1))) \
                return false;                                                                    \
        return true;
        Q4_CHECK(Q4_CB_NF4) Q4_CHECK(Q4_CB_SDYN4) Q4_CHECK(Q4_CB_DYN4) Q4_CHECK(Q4_CB_DYN4_NZ)
        Q4_CHECK(Q4_CB_LIN4_NZ)
#undef Q4_CHECK
    }
    return false;
}
static_assert(sorted_ok(Q4_CB_NF4) && sorted_ok(Q4_CB_SDYN4) && sorted_ok(Q4_CB_DYN4) &&
                  sorted_ok(Q4_CB_DYN4_NZ) && sorted_ok(Q4_CB_LIN4_NZ),
              "codebook levels must be strictly increasing with interior midpoints");

// Device copies, indexed at run time when the LDS tables are filled.
__constant__ uint32_t c_decode[5][16] = {Q4_CB_BITS_NF4, Q4_CB_BITS_SDYN4, Q4_CB_BITS_DYN4, Q4_CB_BITS_DYN4_NZ,
                                         Q4_CB_BITS_LIN4_NZ};

template <int CB> __device__ __forceinline__ float sorted_level_rt(int k) {
    return bits2f(c_decode[CB][Book<CB>::code_of(k)]);
}

// ---------------------------------------------------------------------------
// Round-to-nearest by bucket table
// ---------------------------------------------------------------------------
//
// The RTN index of x is the number of FP32 midpoints strictly below x.
// Buckets split |x| by its binary exponent and MB leading mantissa bits;
// every bucket holds at most one midpoint (checked at compile time), so one
// 8-byte table entry {thr, base} gives the exact count: base + (x > thr).  A bucket of a negative x covers (-hi, -lo], one
// of a positive x [lo, hi); magnitudes below 2^(EMIN-127) share bucket 0.

struct alignas(8) BucketEntry {
    float thr;     // the one midpoint inside the bucket, or 3 (never exceeded)
    int32_t base;  // midpoints below every x of the bucket
};

__host__ __device__ constexpr uint32_t f2bits(float f) { return __builtin_bit_cast(uint32_t, f); }

template <int CB> struct Enc {
    static constexpr int MB = 3;
    static constexpr bool SIGNED = CB == Q4_CB_NF4 || CB == Q4_CB_SDYN4;
    static constexpr int N = Book<CB>::N;
    static constexpr int min_mid_exp() {
        int e = 255;
        for (int k = 0; k + 1 < N; ++k) {
            const int ek = (int)((f2bits(Book<CB>::mid(k)) >> 23) & 0xFF);
            if (ek < e) e = ek;
        }
        return e;
    }
    // bucket 0 ends at 2^(EMIN-127) * 1.125, below every midpoint magnitude
    static constexpr int EMIN = min_mid_exp() - 1;
    static constexpr int NPOS = ((127 - EMIN) << MB) + 1;
    static constexpr int pow2ceil(int v) { int p = 1; while (p < v) p <<= 1; return p; }
    static constexpr int PAD = pow2ceil(NPOS);
    static constexpr int SIZE = SIGNED ? 2 * PAD : NPOS;
};

template <int CB> struct EncTable {
    BucketEntry e[Enc<CB>::SIZE];
    bool ok;
    constexpr EncTable() : e(), ok(true) {
        using E = Enc<CB>;
        for (int s = 0; s < (E::SIGNED ? 2 : 1); ++s) {
            for (int b = 0; b < (E::SIGNED ? E::PAD : E::NPOS); ++b) {
                const int bb = b < E::NPOS ? b : E::NPOS - 1;  // padding repeats the last bucket
                const float lo = bb == 0 ? 0.0f : bits2f((uint32_t)((E::EMIN << E::MB) + bb) << (23 - E::MB));
                const float hi = bits2f((uint32_t)((E::EMIN << E::MB) + bb + 1) << (23 - E::MB));
                int base = 0, inside = 0;
                float thr = 3.0f;
                for (int k = 0; k + 1 < E::N; ++k) {
                    const float m = Book<CB>::mid(k);
                    if (s == 0) {          // x in [lo, hi)
                        if (m < lo) ++base;
                        else if (m < hi) { ++inside; thr = m; }
                    } else {               // x in (-hi, -lo]
                        if (m <= -hi) ++base;
                        else if (m <= -lo) { ++inside; thr = m; }
                    }
                }
                if (inside > 1) ok = false;
                BucketEntry& d = e[s * E::PAD + b];
                d.thr = thr;
                d.base = base;
            }
        }
    }
};

static_assert(EncTable<Q4_CB_NF4>().ok && EncTable<Q4_CB_SDYN4>().ok && EncTable<Q4_CB_DYN4>().ok &&
                  EncTable<Q4_CB_DYN4_NZ>().ok && EncTable<Q4_CB_LIN4_NZ>().ok,
              "a bucket holds two midpoints: use more mantissa bits");

// Floor buckets of an unsigned map whose first level is 0: the index of the
// largest level <= x.  Each bucket holds at most one level, so one entry
// {thr, lo} gives it: lo + (x >= thr).  Every level below the bucket lies
// below every x of the bucket, so x sits exactly on a level iff x == thr.
struct alignas(8) FloorEntry {
    float thr;      // the one level inside the bucket, or 3 (never reached)
    int32_t lo;     // index of the largest level below the bucket (-1 below 0)
};

template <int CB> struct FloorTable {
    FloorEntry e[Enc<CB>::NPOS];
    bool ok;
    constexpr FloorTable() : e(), ok(true) {
        using E = Enc<CB>;
        if (Book<CB>::level(0) != 0.0f) ok = false;
        for (int b = 0; b < E::NPOS; ++b) {
            const float lo = b == 0 ? 0.0f : bits2f((uint32_t)((E::EMIN << E::MB) + b) << (23 - E::MB));
            const float hi = bits2f((uint32_t)((E::EMIN << E::MB) + b + 1) << (23 - E::MB));
            int below = 0, inside = 0;
            float thr = 3.0f;
            for (int k = 0; k < E::N; ++k) {
                const float L = Book<CB>::level(k);
                if (L < lo) ++below;
                else if (L < hi) { ++inside; thr = L; }
            }
            if (inside > 1) ok = false;
            FloorEntry& d = e[b];
            d.thr = thr;
            d.lo = below - 1;
        }
    }
};
static_assert(FloorTable<Q4_CB_DYN4>().ok, "floor buckets of Dyn4 must hold one level each");
__constant__ FloorTable<Q4_CB_DYN4> c_floor_dyn4 = FloorTable<Q4_CB_DYN4>();

__constant__ EncTable<Q4_CB_NF4> c_enc_nf4 = EncTable<Q4_CB_NF4>();
__constant__ EncTable<Q4_CB_SDYN4> c_enc_sdyn4 = EncTable<Q4_CB_SDYN4>();
__constant__ EncTable<Q4_CB_DYN4> c_enc_dyn4 = EncTable<Q4_CB_DYN4>();
__constant__ EncTable<Q4_CB_DYN4_NZ> c_enc_dyn4nz = EncTable<Q4_CB_DYN4_NZ>();
__constant__ EncTable<Q4_CB_LIN4_NZ> c_enc_lin4nz = EncTable<Q4_CB_LIN4_NZ>();

template <int CB> __device__ __forceinline__ const BucketEntry* enc_table_global() {
    if constexpr (CB == Q4_CB_NF4) return c_enc_nf4.e;
    else if constexpr (CB == Q4_CB_SDYN4) return c_enc_sdyn4.e;
    else if constexpr (CB == Q4_CB_DYN4) return c_enc_dyn4.e;
    else if constexpr (CB == Q4_CB_DYN4_NZ) return c_enc_dyn4nz.e;
    else return c_enc_lin4nz.e;
}

// Bucket index of x.  NaN or |x| > 1 land in the last bucket, so the
// index never leaves the table.
template <int CB> __device__ __forceinline__ uint32_t bucket_index(float x) {
    using E = Enc<CB>;
    const uint32_t u = __float_as_uint(x);
    uint32_t raw = __builtin_amdgcn_ubfe(u, 23 - E::MB, 8 + E::MB);
    raw = raw < (uint32_t)(E::EMIN << E::MB) ? (uint32_t)(E::EMIN << E::MB) : raw;
    raw = raw > (uint32_t)(127 << E::MB) ? (uint32_t)(127 << E::MB) : raw;
    uint32_t idx = raw - (uint32_t)(E::EMIN << E::MB);
    if constexpr (E::SIGNED) idx += (u >> 31) * (uint32_t)E::PAD;
    return idx;
}
template <int CB>
__device__ __forceinline__ const BucketEntry& bucket_of(const BucketEntry* tab, float x) {
    return tab[bucket_index<CB>(x)];
}

// The RTN index of x (midpoints strictly below x) from its bucket entry.
__device__ __forceinline__ int rtn_index(const BucketEntry& e, float x) { return e.base + (x > e.thr ? 1 : 0); }
// The floor index of x (largest level <= x) from a floor entry's {thr, lo}.
__device__ __forceinline__ int floor_index(float thr, int lo, float x) { return lo + (x >= thr ? 1 : 0); }

// ---------------------------------------------------------------------------
// Flat layout
// ---------------------------------------------------------------------------

// Flat bucket layout, for the ZIP-SR kernels (their VALU issue rate is what
// bounds them): the entry of x in [-1, 1] sits at its bit pattern >> 20
// (sign, exponent, 3 mantissa bits), slots 0 .. 1016 for x >= 0 and
// 2048 .. 3064 for x < 0, so finding it is a shift; the v floor entries of
// x in [0, 1] fill the slots between, at 1017 + (bits >> 20).  Each flat
// bucket lies inside one bucket of the compact tables above (which merge
// the magnitudes below the smallest midpoint), so it takes that entry.
constexpr int kFlatPos = (127 << 3) + 1;          // bits >> 20 of x in [+0, 1]
constexpr int kFlatNeg = 2048;                     // bits >> 20 of x in [-1, -0]
constexpr int kFlatSlots = kFlatNeg + kFlatPos;
constexpr int kFlatAlloc = (kFlatSlots + 1) & ~1;  // slots held, a whole number of 16-byte pieces
static_assert(2 * kFlatPos <= kFlatNeg, "the floor entries must fit between the two halves");

template <int VCB, int VRULE> constexpr bool flat_tables() {
    return VRULE == Q4_RULE_UPDATE_SR && VCB == Q4_CB_DYN4;
}

// Flat slots of x: the m entry of x in [-1, 1], and the v floor entry of
// x in [0, 1] (11 bits: the slot stays below the negative half for any x).
__device__ __forceinline__ uint32_t flat_m_slot(float x) { return __float_as_uint(x) >> 20; }
__device__ __forceinline__ uint32_t flat_floor_slot(float x) {
    return kFlatPos + __builtin_amdgcn_ubfe(__float_as_uint(x), 20, 11);
}
// The compact bucket index of x, as bucket_index computes it, for building
// tables at compile time.
template <int CB> constexpr uint32_t bucket_index_c(float x) {
    using E = Enc<CB>;
    const uint32_t u = f2bits(x);
    uint32_t raw = (u >> (23 - E::MB)) & ((1u << (8 + E::MB)) - 1u);
    raw = raw < (uint32_t)(E::EMIN << E::MB) ? (uint32_t)(E::EMIN << E::MB) : raw;
    raw = raw > (uint32_t)(127 << E::MB) ? (uint32_t)(127 << E::MB) : raw;
    uint32_t idx = raw - (uint32_t)(E::EMIN << E::MB);
    if (E::SIGNED) idx += (u >> 31) * (uint32_t)E::PAD;
    return idx;
}

// The whole flat table of an m map, built at compile time: slot i takes the
// compact entry of a value inside it (m entries of MCB, Dyn4 floor entries
// as {thr, lo}, unused slots never exceeded).  A work-group copies it into
// LDS with 16-byte loads instead of forming its 3,065 slots itself.
template <int MCB> struct alignas(16) FlatTable {
    BucketEntry e[kFlatAlloc];
    constexpr FlatTable() : e() {
        constexpr EncTable<MCB> enc{};
        constexpr FloorTable<Q4_CB_DYN4> fl{};
        for (int i = 0; i < kFlatAlloc; ++i) {
            BucketEntry d{3.0f, 0};
            if (i < kFlatPos) {
                d = enc.e[bucket_index_c<MCB>(bits2f((uint32_t)i << 20))];
            } else if (i >= kFlatNeg) {
                d = enc.e[bucket_index_c<MCB>(bits2f(0x80000000u | ((uint32_t)(i - kFlatNeg) << 20)))];
            } else if (i - kFlatPos < kFlatPos) {
                const FloorEntry& f = fl.e[bucket_index_c<Q4_CB_DYN4>(bits2f((uint32_t)(i - kFlatPos) << 20))];
                d.thr = f.thr;
                d.base = f.lo;
            }
            if (i < kFlatSlots) e[i] = d;
            else e[i] = BucketEntry{3.0f, 0};
        }
    }
};
static_assert(sizeof(BucketEntry) * kFlatAlloc % 16 == 0, "the flat table is copied in 16-byte pieces");
__device__ const FlatTable<Q4_CB_NF4> c_flat_nf4 = FlatTable<Q4_CB_NF4>();
__device__ const FlatTable<Q4_CB_SDYN4> c_flat_sdyn4 = FlatTable<Q4_CB_SDYN4>();

// The flat table of MCB copied into LDS by a 256-thread work-group in two
// halves: each thread loads its pieces (load_flat_table), and only then
// stores them (store_flat_table), so the copy waits for L2 once, not once
// per piece.  The step kernels issue their other setup loads in between.
typedef uint32_t FlatPiece __attribute__((ext_vector_type(4)));
struct FlatPieces {
    FlatPiece a0, a1, a2, a3, a4, a5;
};
constexpr int kFlatPieces = (int)(sizeof(BucketEntry) * kFlatAlloc / 16);
static_assert(kFlatPieces > 5 * 256 && kFlatPieces <= 6 * 256, "five full passes of 256 pieces and a partial sixth");
template <int MCB> __device__ __forceinline__ FlatPieces load_flat_table() {
    const FlatPiece* src = reinterpret_cast<const FlatPiece*>(MCB == Q4_CB_NF4 ? c_flat_nf4.e : c_flat_sdyn4.e);
    const int t = (int)threadIdx.x;
    FlatPieces p;
    p.a0 = src[t];
    p.a1 = src[t + 256];
    p.a2 = src[t + 512];
    p.a3 = src[t + 768];
    p.a4 = src[t + 1024];
    p.a5 = src[t < kFlatPieces - 1280 ? t + 1280 : 0];  // in bounds; stored only where it is a piece
    return p;
}
// `dst`: LDS, 16-byte aligned, kFlatAlloc entries.
__device__ __forceinline__ void store_flat_table(BucketEntry* dst, const FlatPieces& p) {
    FlatPiece* d = reinterpret_cast<FlatPiece*>(dst);
    const int t = (int)threadIdx.x;
    d[t] = p.a0;
    d[t + 256] = p.a1;
    d[t + 512] = p.a2;
    d[t + 768] = p.a3;
    d[t + 1024] = p.a4;
    if (t < kFlatPieces - 1280) d[t + 1280] = p.a5;
}
template <int MCB> __device__ __forceinline__ void copy_flat_table(BucketEntry* dst) {
    store_flat_table(dst, load_flat_table<MCB>());
}

// ---------------------------------------------------------------------------
// 8-bit maps (SDyn8 m, Dyn8 v)
// ---------------------------------------------------------------------------
//
// The nearest level is the number of FP32 midpoints strictly below x.
// Counting them with a binary search over a sorted table in LDS puts every
// probe of one step on the same bank (the probes of a step sit s apart, s a
// power of two), so it is counted with a bucket table instead: a
// non-negative float's bit pattern shifted right (exponent and top mantissa
// bits) names a bucket that holds at most two midpoints; the table gives the
// midpoints below the bucket, one 8-byte read gives the two candidates, and
// two compares finish the count.
//
// SDyn8 is symmetric about zero with 127 positive midpoints P: for x >= 0
// the ascending level index is 127 + #{P < x}, and for x < 0 it is
// 127 - #{P <= |x|}, which is #{P < nextup(|x|)}.  Either count is the
// magnitude part of the code; the sign bit goes on a non-zero magnitude.

__constant__ uint32_t c_cb8[2][256] = {Q4_CB8_BITS_SDYN8, Q4_CB8_BITS_DYN8};


// The 8-bit tables as the step reads them, formed at compile time and
// copied into LDS by each work-group: code-indexed levels; {mid[i],
// mid[i + 1]} over SDyn8's positive midpoints and Dyn8's midpoints,
// ascending and +inf padded (each midpoint the FP32 sum of adjacent levels
// halved, as the definition forms it); and per bucket the number of
// midpoints below it.
struct alignas(16) Step8Lds {
    float dec_m[256], dec_v[256];
    float2 pair_m[128], pair_v[256];
    uint8_t floor_m[Q4_RTN8_M_NB], floor_v[Q4_RTN8_V_NB];
};
static_assert(sizeof(Step8Lds) % 16 == 0, "copied in 16-byte pieces");

// #{midpoints < bits2f(key)} for a non-negative key; keys outside the
// bucketed range clamp to the first or last bucket (in bounds for any key).
template <int SHIFT, int LO, int NB>
__device__ __forceinline__ uint32_t count_below8(const uint8_t* floor_tab, const float2* pair, uint32_t key) {
    const int b = min(max((int)(key >> SHIFT) - LO, 0), NB - 1);
    const uint32_t f = floor_tab[b];
    const float2 pr = pair[f];
    const float a = bits2f(key);
    return f + (pr.x < a ? 1u : 0u) + (pr.y < a ? 1u : 0u);
}

__device__ __forceinline__ uint32_t rtn8_m(const Step8Lds& lds, float x) {
    const uint32_t xb = __float_as_uint(x);
    const uint32_t neg = xb >> 31;
    const uint32_t c = count_below8<Q4_RTN8_M_SHIFT, Q4_RTN8_M_LO, Q4_RTN8_M_NB>(lds.floor_m, lds.pair_m,
                                                                                 (xb & 0x7FFFFFFFu) + neg);
    return c | ((neg != 0u && c != 0u) ? 0x80u : 0u);
}

__device__ __forceinline__ uint32_t rtn8_v(const Step8Lds& lds, float x) {
    return count_below8<Q4_RTN8_V_SHIFT, Q4_RTN8_V_LO, Q4_RTN8_V_NB>(lds.floor_v, lds.pair_v, __float_as_uint(x));
}

// The tables' values, formed once at compile time.
struct Step8Table {
    Step8Lds t;
    constexpr Step8Table() : t() {
        constexpr uint32_t cb_m[256] = Q4_CB8_BITS_SDYN8, cb_v[256] = Q4_CB8_BITS_DYN8;
        const float inf = __builtin_inff();
        float mid_p[128] = {}, mid_v[256] = {};
        for (int i = 0; i < 256; ++i) {
            t.dec_m[i] = bits2f(cb_m[i]);
            t.dec_v[i] = bits2f(cb_v[i]);
        }
        // SDyn8's codes 0..127 ascend from 0; Dyn8's codes 0..255 ascend from 0
        for (int i = 0; i < 128; ++i) mid_p[i] = i < 127 ? (bits2f(cb_m[i]) + bits2f(cb_m[i + 1])) * 0.5f : inf;
        for (int i = 0; i < 256; ++i) mid_v[i] = i < 255 ? (bits2f(cb_v[i]) + bits2f(cb_v[i + 1])) * 0.5f : inf;
        for (int i = 0; i < 128; ++i) t.pair_m[i] = float2{mid_p[i], i < 127 ? mid_p[i + 1] : inf};
        for (int i = 0; i < 256; ++i) t.pair_v[i] = float2{mid_v[i], i < 255 ? mid_v[i + 1] : inf};
        for (int b = 0; b < Q4_RTN8_M_NB; ++b) {
            const float x = bits2f((uint32_t)(b + Q4_RTN8_M_LO) << Q4_RTN8_M_SHIFT);
            int n = 0;
            for (int i = 0; i < 128; ++i) n += mid_p[i] < x ? 1 : 0;
            t.floor_m[b] = (uint8_t)n;
        }
        for (int b = 0; b < Q4_RTN8_V_NB; ++b) {
            const float x = bits2f((uint32_t)(b + Q4_RTN8_V_LO) << Q4_RTN8_V_SHIFT);
            int n = 0;
            for (int i = 0; i < 256; ++i) n += mid_v[i] < x ? 1 : 0;
            t.floor_v[b] = (uint8_t)n;
        }
    }
};
__device__ const Step8Table c_step8 = Step8Table();

// Copies the tables into LDS; every thread of a 256-thread group takes part
// (all of its loads before its first store), and the group synchronizes.
__device__ __forceinline__ void step8_tables(Step8Lds& lds) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int n16 = (int)(sizeof(Step8Lds) / 16);
    static_assert(n16 > 256 && n16 <= 512, "one full pass of 256 pieces and a partial second");
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(&c_step8.t);
    u32x4_t* d = reinterpret_cast<u32x4_t*>(&lds);
    const int t = (int)threadIdx.x;
    const bool second = t < n16 - 256;
    const u32x4_t a0 = src[t];
    u32x4_t a1 = {0u, 0u, 0u, 0u};
    if (second) a1 = src[t + 256];
    d[t] = a0;
    if (second) d[t + 256] = a1;
    __syncthreads();
}

}  // namespace q4
