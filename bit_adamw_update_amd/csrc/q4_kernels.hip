// q4_kernels.hip -- HIP kernels of the fused 4-bit AdamW optimizer step for
// CDNA4 (gfx950).
//
// What is computed follows the pages on 4-bit AdamW state quantization:
//   "Rounding in Preconditioner Space" (paper listing): abstract, Table 1
//   (rounding rules), Table 2 (ZIP-SR and ZE-EDEN recipes, LM-head switch);
//   AReno "4-bit AdamW", section "State representation" (128-element
//   parameter-local blocks; factored v for matrices, packed zero-excluding v
//   for vectors; bounded block-local FP32 work);
//   the news article on the two 4-bit AdamW methods (AdamW description,
//   1.0625 B/param storage).
//
// How it maps onto the chip: the step is an elementwise stream at ~12 bytes
// per parameter, so it is bound by HBM, not by the matrix cores.  A 64-lane
// wavefront owns a chunk of four 128-element blocks; each lane owns 8
// consecutive elements, so a block is one 16-lane DPP row and every block
// statistic (absmax, EDEN sums, the per-level square roots of ZIP-SR) is a
// row-local DPP or ds_bpermute exchange with no LDS traffic.  Each lane
// moves its parameters as two 16-byte loads, its gradients as one 16-byte
// load and each moment's 8 codes as one 4-byte load.  One launch covers
// every tensor: work-groups walk runs of consecutive tensor-aligned chunks
// (so that each 128-byte line of block scales is written by one group) and
// follow a prefix table of chunk offsets.
//
// Arithmetic is FP32, round-to-nearest-even, with IEEE division and square
// root, in the order stated for each operation, so that every code decision
// is reproducible bit for bit on any IEEE implementation.  The compiler
// contracts nothing (-ffp-contract=off); the fused multiply-adds are written
// out: the two moment recurrences, the denominator and the weight update.

#include <atomic>
#include <mutex>

#include "q4_internal.h"
#include "q4_exact.h"
#include "q4_quant.h"

namespace q4 {

void codebook_table(int cb, float* out) {
    static const uint32_t host[5][16] = {Q4_CB_BITS_NF4, Q4_CB_BITS_SDYN4, Q4_CB_BITS_DYN4, Q4_CB_BITS_DYN4_NZ,
                                         Q4_CB_BITS_LIN4_NZ};
    static const uint32_t host8[2][256] = {Q4_CB8_BITS_SDYN8, Q4_CB8_BITS_DYN8};
    if (cb >= Q4_CB_SDYN8) {
        for (int i = 0; i < 256; ++i) out[i] = bits2f(host8[cb - Q4_CB_SDYN8][i]);
        return;
    }
    for (int i = 0; i < 16; ++i) out[i] = bits2f(host[cb][i]);
}

// ---------------------------------------------------------------------------
// Small device primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Philox4x32-10 and the uniforms drawn from it are in q4_exact.h.

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls within a 16-lane row: swap neighbours, swap pairs, mirror
// each half-row, mirror the row.  Applied in that order, each lane ends up
// with the row's pairwise-tree reduction of its 16 lane values.
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

// Maximum over the 16 lanes of a row of values that are +0 or positive (not
// NaN): their bit patterns order like the values, so an unsigned maximum,
// which takes its DPP operand directly, does it.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row_max16(float x) {
    uint32_t u = __float_as_uint(x);
    u = max(u, dpp_u<DPP_QUAD_1032>(u));
    u = max(u, dpp_u<DPP_QUAD_2301>(u));
    u = max(u, dpp_u<DPP_ROW_HALF_MIRROR>(u));
    u = max(u, dpp_u<DPP_ROW_MIRROR>(u));
    return __uint_as_float(u);
}
// Sum over the 16 lanes of a row, combining lanes (0,1),(2,3).. then pairs
// of pairs, then halves: the pairwise tree over the lanes in index order
// (IEEE addition is commutative, so both partners get the same bits).
__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<DPP_QUAD_1032>(x);
    x = x + dpp<DPP_QUAD_2301>(x);
    x = x + dpp<DPP_ROW_HALF_MIRROR>(x);
    x = x + dpp<DPP_ROW_MIRROR>(x);
    return x;
}
__device__ __forceinline__ float tree4(const float* v) {
    return (v[0] + v[1]) + (v[2] + v[3]);
}
__device__ __forceinline__ float bperm(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(lane << 2, __float_as_int(v)));
}
// The IEEE square root and block-scale inverse the rules use, and the
// nibble-addressed lane exchange that decodes codes, are in q4_exact.h.

// ---------------------------------------------------------------------------
// Global-memory views
// ---------------------------------------------------------------------------

// Pointers read from the tensor table are generic; viewing them in the
// global address space lets the compiler issue global_load/global_store
// rather than flat instructions (which also occupy the LDS wait counter).
template <class T> using gptr = __attribute__((address_space(1))) T*;
template <class T> __device__ __forceinline__ gptr<T> G(T* p) { return (gptr<T>)p; }
template <class T> __device__ __forceinline__ gptr<const T> G(const T* p) { return (gptr<const T>)p; }
// clang vector types copy in any address space (HIP's float4 does not)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// K1: the fused step for packed and factored tensors
// ---------------------------------------------------------------------------

// The codebooks, the round-to-nearest bucket tables (compact and flat) and
// the 8-bit tables are in q4_quant.h.

template <int MCB, int VCB, bool FLAT> struct StepLds {
    BucketEntry enc_m[FLAT ? 1 : Enc<MCB>::SIZE];
    BucketEntry enc_v[Enc<VCB>::SIZE];
    FloorEntry floor_v[(VCB == Q4_CB_DYN4 && !FLAT) ? Enc<VCB>::NPOS : 1];
    alignas(16) BucketEntry flat[FLAT ? kFlatAlloc : 1];  // m entries; v floor entries as {thr, lo}
    float lev_m[16], lev_v[16];  // sorted levels (rare SR paths)
};


// Per-lane constants of the codebooks: lane `sub` of each 16-lane row holds
// the code-`sub` level of each map (decode) and the sorted level `sub` of v.
struct LaneBooks {
    float dec_m, dec_v, lev_v;
};

template <int MCB, int VCB, int VRULE, bool FULL, bool PACKED, bool CLIP>
__device__ __forceinline__ void step_chunk(const DevTensor& T, const int64_t lc, const int64_t chunk,
                                           const StepScalars& sc,
                                           const StepLds<MCB, VCB, flat_tables<VCB, VRULE>()>& lds,
                                           const LaneBooks& lb, const int lane, const float gs) {
    constexpr int NM = Book<MCB>::N, NV = Book<VCB>::N;
    constexpr bool FLAT = flat_tables<VCB, VRULE>();
    // the m bucket entry of x in [-1, 1] (the clamps below keep every x,
    // NaN included, in that range, so a flat index stays inside its half)
    auto m_entry = [&](float x) -> const BucketEntry& {
        if constexpr (FLAT) return lds.flat[flat_m_slot(x)];
        else return bucket_of<MCB>(lds.enc_m, x);
    };
    constexpr bool V_SR = VRULE == Q4_RULE_STATE_SR || VRULE == Q4_RULE_UPDATE_SR;
    constexpr bool V_UPD = VRULE == Q4_RULE_UPDATE_SR || VRULE == Q4_RULE_UPDATE_RTN;
    const int sub = lane & 15, row_base = lane & 48;
    const int rb4 = row_base << 2;
    const uint32_t rb4x4 = (uint32_t)rb4 * 0x01010101u;
    const int64_t n = T.numel;
    const int64_t blk = lc * kBlocksPerChunk + (lane >> 4);
    // the chunk's bases are wave-uniform (scalar registers); a lane adds a
    // 32-bit offset, so no per-lane 64-bit address arithmetic
    const int64_t c0 = lc * kChunkElems;
    // Row r of the wave owns block r.  Lane `sub` holds 4 consecutive
    // elements of each half of it: le .. le+3 (values 0..3) and
    // le+64 .. le+67 (values 4..7).  Each load or store instruction of the
    // masters then covers whole 256-byte pieces of the rows, so the
    // streaming (nontemporal) accesses below never split a cache line
    // between two instructions.
    const int le = row_base * 8 + sub * 4;  // the lane's first element within the chunk
    const int64_t e0 = c0 + le;
    int nva = 4, nvb = 4;  // valid elements of the two halves
    bool blk_ok = true;
    if (!FULL) {
        const int64_t ra = n - e0, rb2 = n - (e0 + 64);
        nva = ra >= 4 ? 4 : (ra > 0 ? (int)ra : 0);
        nvb = rb2 >= 4 ? 4 : (rb2 > 0 ? (int)rb2 : 0);
        blk_ok = blk * kBlock < n;
    }
    // all 8 elements present (the second half's 4 imply the first's)
    const bool lane_full = FULL || nvb == 4;
    auto valid = [&](int k) { return FULL || (k < 4 ? k < nva : k - 4 < nvb); };
    constexpr bool packed_v = PACKED;  // packed v; else the factored estimate
    const gptr<float> param = G(T.param) + c0;
    const gptr<const uint16_t> grad = G(T.grad) + c0;
    const gptr<uint8_t> mcodes = G(T.m_codes) + (c0 >> 1);
    const gptr<uint8_t> vcodes = G(T.v_codes) + (c0 >> 1);
    const gptr<float> mscales = G(T.m_scales) + lc * kBlocksPerChunk;
    const gptr<float> vscales = G(T.v_scales) + lc * kBlocksPerChunk;
    const int lb4 = lane >> 4;  // the lane's block within the chunk
    // the element-independent part of the stochastic-rounding draws, and
    // the counter of the lane's first element: its index in the whole tensor
    // (a shard's elements start at elem_offset) over 4, modulo 2^32
    const PhiloxFixed pf = philox_fixed(sc.step, T.tensor_id, sc.key0, sc.key1);
    const uint32_t ctr0 = (uint32_t)(e0 >> 2) + T.ctr_base;

    // ---- loads
    // While a wave issues its loads it runs at raised priority, so the
    // memory pipe is refilled before other waves' arithmetic.  Memory-bound
    // rules gain from it; the VALU-bound flat-table (ZIP-SR) kernel does not.
    if constexpr (!FLAT) __builtin_amdgcn_s_setprio(2);
    // Masters and gradients are read once and written once per step, so
    // they stream past the caches (nontemporal): an in-place rewrite of this
    // byte mix runs about 6% faster that way on gfx950.  The codes keep the
    // default policy: their 16-bit lane pieces share lines between the two
    // halves' instructions.
    float p[8], g[8];
    uint32_t mc = 0, vc = 0;
    const int lh = (le + 64) >> 1;  // byte offset of the second half's codes
    if (lane_full) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(param + le));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(param + le + 64));
        p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w; p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
        const u32x2 ga = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(grad + le));
        const u32x2 gb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(grad + le + 64));
        g[0] = bf16_to_f32(ga.x & 0xFFFFu); g[1] = bf16_to_f32(ga.x >> 16);
        g[2] = bf16_to_f32(ga.y & 0xFFFFu); g[3] = bf16_to_f32(ga.y >> 16);
        g[4] = bf16_to_f32(gb.x & 0xFFFFu); g[5] = bf16_to_f32(gb.x >> 16);
        g[6] = bf16_to_f32(gb.y & 0xFFFFu); g[7] = bf16_to_f32(gb.y >> 16);
        mc = (uint32_t)*reinterpret_cast<const gptr<const uint16_t>>(mcodes + (le >> 1)) |
             ((uint32_t)*reinterpret_cast<const gptr<const uint16_t>>(mcodes + lh) << 16);
        if (packed_v)
            vc = (uint32_t)*reinterpret_cast<const gptr<const uint16_t>>(vcodes + (le >> 1)) |
                 ((uint32_t)*reinterpret_cast<const gptr<const uint16_t>>(vcodes + lh) << 16);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int o = le + (k < 4 ? k : 60 + k);
            p[k] = valid(k) ? param[o] : 0.0f;
            g[k] = valid(k) ? bf16_to_f32(grad[o]) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // code byte j holds values 2j and 2j + 1
            if (valid(2 * j)) {
                const int ob = j < 2 ? (le >> 1) + j : lh + j - 2;
                mc |= (uint32_t)mcodes[ob] << (8 * j);
                if (packed_v) vc |= (uint32_t)vcodes[ob] << (8 * j);
            }
        }
    }
    if constexpr (CLIP) {
        // the clipped gradient (one FP32 product per element)
#pragma unroll
        for (int k = 0; k < 8; ++k) g[k] *= gs;
    }
    const float sm_old = (FULL || blk_ok) ? mscales[lb4] : 0.0f;
    const float sv_old = ((FULL || blk_ok) && packed_v) ? vscales[lb4] : 0.0f;
    if constexpr (!FLAT) __builtin_amdgcn_s_setprio(0);
    // lane `sub` of the row holds level(sub) * old scale: decoding is one
    // ds_bpermute per element (the same product the definition forms)
    const float dm_own = lb.dec_m * sm_old;
    const float dv_own = lb.dec_v * sv_old;

    // ---- factored second moment: v1 = (R_r C_c) / mean(R) over [rows, cols]
    float vf[8];
    if constexpr (!packed_v) {
        const float inv_mean = *T.inv_meanR;
        const gptr<const float> R = G((const float*)T.v_row);
        const gptr<const float> Cv = G((const float*)T.v_col);
        // row of the chunk's first element (wave-uniform; 32-bit division
        // while the offset fits), then a 32-bit division for the lane's
        // offset (cols < 2^31 is validated)
        const uint32_t cols = (uint32_t)T.cols;
        const uint64_t first = (uint64_t)lc * kChunkElems;
        const int64_t rb = (first >> 32) == 0 ? (int64_t)((uint32_t)first / cols) : (int64_t)(first / (uint64_t)T.cols);
        const uint32_t off = (uint32_t)(e0 - rb * T.cols);
        const uint32_t dr = off / cols;
        const uint32_t cc = off - dr * cols;
        if (lane_full && cc + 68u <= cols && (cc & 3u) == 0u) {
            // both halves in one row
            const float Rr = R[rb + dr];
            const f32x4 a = *reinterpret_cast<const gptr<const f32x4>>(Cv + cc);
            const f32x4 b = *reinterpret_cast<const gptr<const f32x4>>(Cv + cc + 64);
            const float cv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) vf[k] = (Rr * cv[k]) * inv_mean;
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // row and column of the half's first element, then along the row
                const uint32_t oh = off + 64u * h;
                const uint32_t drh = oh / cols;
                uint32_t ch = oh - drh * cols;
                int64_t rh = rb + drh;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = 4 * h + kk;
                    vf[k] = 0.0f;
                    if (valid(k)) {
                        vf[k] = (R[rh] * Cv[ch]) * inv_mean;
                        if (++ch == cols) { ch = 0; ++rh; }
                    }
                }
            }
        }
    }

    // ---- AdamW on the unquantized moments
    const NibbleAddrs ma = nibble_addrs(mc, rb4x4);
    const NibbleAddrs va = nibble_addrs(vc, rb4x4);
    float m1[8], v1[8], sv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float gk = g[k];
        const float m0 = bperm_addr(dm_own, nibble_addr(ma, k));
        // each recurrence is one fused multiply-add onto the gradient term
        m1[k] = __builtin_fmaf(sc.beta1, m0, sc.omb1 * gk);
        if constexpr (packed_v) {
            const float v0 = bperm_addr(dv_own, nibble_addr(va, k));
            v1[k] = __builtin_fmaf(sc.beta2, v0, sc.omb2 * (gk * gk));
        } else {
            v1[k] = vf[k];
        }
    }
    // The preconditioner-space rules decide codes from sqrt(v1), so there it
    // is the IEEE square root (the short form unless some element of the
    // wave is below 2^-96); elsewhere it only scales the weight update and
    // the hardware square root (1 ulp) serves.
    if (V_UPD) {
        // some v1 in (0, 2^-96)?  v1 >= +0, and bits - 1 sends +0 to the top
        uint32_t low = 0xFFFFFFFFu;
#pragma unroll
        for (int k = 0; k < 8; ++k) low = min(low, __float_as_uint(v1[k]) - 1u);
        if (__builtin_amdgcn_ballot_w64(low < 0x0F800000u - 1u) != 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) sv[k] = sqrtf(v1[k]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) sv[k] = sqrt_rn_normal(v1[k]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) sv[k] = __builtin_amdgcn_sqrtf(v1[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        // the quotient m1 / denom uses the hardware reciprocal (1 ulp): it
        // moves the weight by far less than one part in 10^6 and no code
        // depends on it
        const float denom = __builtin_fmaf(sv[k], sc.rsbc2, sc.eps);
        p[k] = __builtin_fmaf(-sc.step_size, m1[k] * __builtin_amdgcn_rcpf(denom), p[k] * sc.decay);
        if (!valid(k)) {
            m1[k] = 0.0f;
            v1[k] = 0.0f;
        }
    }
    if (lane_full) {
        __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, reinterpret_cast<gptr<f32x4>>(param + le));
        __builtin_nontemporal_store(f32x4{p[4], p[5], p[6], p[7]}, reinterpret_cast<gptr<f32x4>>(param + le + 64));
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (valid(k)) param[le + (k < 4 ? k : 60 + k)] = p[k];
    }

    // ---- first moment: absmax scale of the block, RTN or state-space SR
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(m1[k]));
    const float s_m = row_max16(am);
    const float inv_m = inv_scale(s_m);
    const bool m_sr = (sc.flags & SF_M_SR_ALL) || ((T.flags & Q4_TF_LM_HEAD) && (sc.flags & SF_LM_HEAD_SR));
    uint32_t mword = 0;
    if (!m_sr) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float x = fminf(fmaxf(m1[k] * inv_m, -1.0f), 1.0f);
            const int idx = rtn_index(m_entry(x), x);
            const int code = MCB == Q4_CB_SDYN4 ? (idx < 7 ? 15 - idx : (idx == 7 ? 0 : idx - 7)) : idx;
            mword |= (uint32_t)code << (4 * k);
        }
    } else {
        float um[4];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if ((k & 3) == 0) uniforms4(ctr0 + 16u * (k >> 2), 0u, pf, sc.key0, sc.key1, um);
            const float x = fminf(fmaxf(m1[k] * inv_m, -1.0f), 1.0f);
            const int idx = rtn_index(m_entry(x), x);
            const float Lidx = lds.lev_m[idx];
            // the lower level is idx or idx - 1; an exact hit or the top level stays
            const bool below = x < Lidx;
            const int lo = below ? (idx > 0 ? idx - 1 : 0) : idx;
            const int hi = lo + 1 < NM ? lo + 1 : NM - 1;
            const float Llo = lds.lev_m[lo], Lhi = lds.lev_m[hi];
            const bool mv = !(below && idx == 0) && !(x == Lidx) && lo != NM - 1;
            const int fin = lo + ((mv && um[k & 3] * (Lhi - Llo) < (x - Llo)) ? 1 : 0);
            const int code = MCB == Q4_CB_SDYN4 ? (fin < 7 ? 15 - fin : (fin == 7 ? 0 : fin - 7)) : fin;
            mword |= (uint32_t)code << (4 * k);
        }
    }
    if (lane_full) {
        *reinterpret_cast<gptr<uint16_t>>(mcodes + (le >> 1)) = (uint16_t)mword;
        *reinterpret_cast<gptr<uint16_t>>(mcodes + lh) = (uint16_t)(mword >> 16);
    } else {
        // nibbles past the end of the tensor stay 0
        mword &= ((1u << (4 * nva)) - 1u) | (((1u << (4 * nvb)) - 1u) << 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (valid(2 * j)) mcodes[j < 2 ? (le >> 1) + j : lh + j - 2] = (uint8_t)(mword >> (8 * j));
    }
    if ((FULL || blk_ok) && sub == 0) mscales[lb4] = s_m;

    if constexpr (!packed_v) return;

    // ---- second moment: max scale, the v rule, EDEN
    float av = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) av = fmaxf(av, v1[k]);
    const float s_v = row_max16(av);
    const float inv_v = inv_scale(s_v);
    // lane `sub` holds sqrt(level_sub * s_v): the square root of the state
    // each level would store, for the preconditioner-space rules (the short
    // IEEE form unless some product of the wave is in (0, 2^-96))
    float root_own = 0.0f;
    if constexpr (V_UPD) {
        const float a = lb.lev_v * s_v;
        if (__builtin_amdgcn_ballot_w64(__float_as_uint(a) - 1u < 0x0F800000u - 1u) != 0) root_own = sqrtf(a);
        else root_own = sqrt_rn_normal(a);
    }
    // uniforms of the v rule, drawn 4 at a time (elements 4h .. 4h+3)
    float uv[4];
    auto draw_v = [&](int k) {
        if (V_SR && (k & 3) == 0)
            uniforms4(ctr0 + 16u * (k >> 2), 1u, pf, sc.key0, sc.key1, uv);
    };
    uint32_t vword = 0;
    float xx[8], xq[8];
    const bool eden = (sc.flags & SF_EDEN) != 0;
    if (VRULE == Q4_RULE_UPDATE_SR && VCB == Q4_CB_DYN4 && !eden) {
        // ZIP-SR.  Per-row tables, lane k: root_k, root_(k+1) + eps_sr and
        // root_(k+1) - root_k (the same FP32 operations the rule forms per
        // element, done once per level).
        const float root_next = bperm(root_own, lane + 1);
        const float rnext_eps = root_next + sc.eps_sr;
        const float rdiff = root_next - root_own;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            draw_v(k);
            const float x = normalize_v(v1[k], inv_v);
            // lower level: the floor bucket gives it directly; an exact level
            // hit needs no draw (the top level 1 can only be hit exactly)
            float fthr;
            int flo;
            if constexpr (FLAT) {
                const BucketEntry& f = lds.flat[flat_floor_slot(x)];
                fthr = f.thr;
                flo = f.base;
            } else {
                const FloorEntry& f = lds.floor_v[bucket_index<VCB>(x)];
                fthr = f.thr;
                flo = f.lo;
            }
            const int lo = floor_index(fthr, flo, x);
            const bool hit = x == fthr;
            // ds_bpermute byte address of lane row_base + lo
            const int src4 = (lo << 2) + rb4;
            const float rlo = bperm_addr(root_own, src4);
            const float rhe = bperm_addr(rnext_eps, src4);
            const float rdf = bperm_addr(rdiff, src4);
            // P(up) = (r(a_lo) - r(v)) / (r(a_lo) - r(a_hi)), r(a) = 1/(sqrt(a) + eps_sr),
            // multiplied out so that nothing cancels next to a_lo = 0
            const float num = (sv[k] - rlo) * rhe;
            const float den = rdf * (sv[k] + sc.eps_sr);
            // both compares in every lane, joined as bits: a short-circuit
            // here becomes a branch per element around the draw's compare
            const bool up = (uv[k & 3] * den < num) & !hit;
            vword |= (uint32_t)(lo + (int)up) << (4 * k);
        }
    } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        draw_v(k);
        // x is the clamped value (a NaN becomes 0, of sorted index 0); the
        // EDEN sums take the unclamped one's NaN through nan0 (+0 or NaN)
        const float xr = v1[k] * inv_v;
        const float x = clamp_unit(xr);
        const float nan0 = xr - xr;
        int idx = rtn_index(bucket_of<VCB>(lds.enc_v, x), x);
        float q = lds.lev_v[idx];  // level(idx)
        if constexpr (VRULE != Q4_RULE_STATE_RTN) {
            const float Lidx = q;
            const bool below = x < Lidx;
            const int lo = below ? (idx > 0 ? idx - 1 : 0) : idx;
            const int hi = lo + 1 < NV ? lo + 1 : NV - 1;
            const bool mv = !(below && idx == 0) && !(x == Lidx) && lo != NV - 1;
            bool up;
            if constexpr (VRULE == Q4_RULE_STATE_SR) {
                const float Llo = lds.lev_v[lo], Lhi = lds.lev_v[hi];
                up = uv[k & 3] * (Lhi - Llo) < (x - Llo);
            } else {
                const float rlo = bperm(root_own, row_base + lo);
                const float rhi = bperm(root_own, row_base + hi);
                if constexpr (VRULE == Q4_RULE_UPDATE_SR) {
                    const float num = (sv[k] - rlo) * (rhi + sc.eps_sr);
                    const float den = (rhi - rlo) * (sv[k] + sc.eps_sr);
                    up = uv[k & 3] * den < num;
                } else {
                    // nearer level in r: r(v) - r(a_hi) < r(a_lo) - r(v)
                    const float left = (rhi - sv[k]) * (rlo + sc.eps_sr);
                    const float right = (sv[k] - rlo) * (rhi + sc.eps_sr);
                    up = left < right;
                }
            }
            idx = lo + ((mv && up) ? 1 : 0);
            if (eden) q = lds.lev_v[idx];
        }
        vword |= (uint32_t)idx << (4 * k);
        xx[k] = __builtin_fmaf(x, x, nan0);
        xq[k] = __builtin_fmaf(x, q, nan0);
    }
    }
    if (lane_full) {
        *reinterpret_cast<gptr<uint16_t>>(vcodes + (le >> 1)) = (uint16_t)vword;
        *reinterpret_cast<gptr<uint16_t>>(vcodes + lh) = (uint16_t)(vword >> 16);
    } else {
        vword &= ((1u << (4 * nva)) - 1u) | (((1u << (4 * nvb)) - 1u) << 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (valid(2 * j)) vcodes[j < 2 ? (le >> 1) + j : lh + j - 2] = (uint8_t)(vword >> (8 * j));
    }
    float stored = s_v;
    if (eden) {
        // EDEN: S = <x,x> / <x,Q(x)> over the block, pairwise tree in index
        // order: the tree over each half (4 values per lane, then the row),
        // then the two halves
        const float sxx = row_sum16(tree4(xx)) + row_sum16(tree4(xx + 4));
        const float sxq = row_sum16(tree4(xq)) + row_sum16(tree4(xq + 4));
        const float S = sxq > 0.0f ? sxx / sxq : 1.0f;
        stored = s_v * S;
    }
    if ((FULL || blk_ok) && sub == 0) vscales[lb4] = stored;
}

// The next chunk of a wavefront in the quantized steps: work-group g walks
// runs of R consecutive slabs (kWavesPerGroup adjacent chunks each), run k
// being slabs (k G + g) R .. (k G + g) R + R - 1, so that each 128-byte line
// of block scales is written whole by one work-group (a line written in
// parts by groups on different XCDs, with their own L2 caches, costs a
// partial write-back: 4% of the GPT-2.7B ZE-EDEN step).  j counts the
// slabs done in the current run.
__device__ __forceinline__ int64_t next_chunk(int64_t c, int& j, int run_slabs, int64_t groups) {
    if (++j < run_slabs) return c + kWavesPerGroup;
    j = 0;
    return c + (groups * run_slabs - (run_slabs - 1)) * kWavesPerGroup;
}

// Last tensor whose first chunk is <= c (binary search over the prefix).
__device__ __forceinline__ int first_tensor(const int64_t* __restrict__ chunk_begin, int n_tensors, int64_t c) {
    int lo = 0, hi = n_tensors - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_begin[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Resident wavefronts per SIMD asked of the register allocator (at most 80
// and 72 VGPRs): the preconditioner-space rules keep more values live than
// the state-space ones.  Measured on the GPT-2.7B set: ZIP-SR 2% faster than
// with the allocator's own choice (91 VGPRs, 5 wavefronts).
template <int VRULE> constexpr int step_waves() {
    return (VRULE == Q4_RULE_UPDATE_SR || VRULE == Q4_RULE_UPDATE_RTN) ? 6 : 7;
}

// Factored matrices come only with the factored recipe, whose maps are
// fixed (NF4 m, Dyn4-NZ v by State-RTN).  MATS: the tensor list holds
// factored matrices; only that recipe's maps are instantiated with it, and
// every other instantiation carries no factored branch (its scalar
// registers then fit without spilling to vector lanes: ZIP-SR 13 -> 5
// spilled, ZE-EDEN 26 -> 0).
template <int MCB, int VCB, int VRULE> constexpr bool factored_maps() {
    return MCB == Q4_CB_NF4 && VCB == Q4_CB_DYN4_NZ && VRULE == Q4_RULE_STATE_RTN;
}

// Instantiations that also come in a form walking a queue of runs instead of
// one work-group per run: those of the ZE-EDEN maps without factored
// matrices, on large sets.  Measured in one process over the same buffers:
// GPT-2.7B ZE-EDEN (about 180 runs of 4 per resident group) 2.0% faster with
// runs of 4 from the queue than with one group per run of 2, runs of 8 4%
// slower; GPT-162M ZE-EDEN (about 8 runs per group) 12% slower, so the
// launch takes the queue only from kQueueMinRunsPerGroup runs per group.
// The queue loop takes this kernel to 72 VGPRs (7 wavefronts per SIMD, its
// target) without spilling; the other instantiations of the compact tables
// spill with it, and ZIP-SR is bound by its arithmetic.
template <int MCB, int VCB, int VRULE, bool MATS> constexpr bool queue_walk() {
    return factored_maps<MCB, VCB, VRULE>() && !MATS;
}

template <int MCB, int VCB, int VRULE, bool CLIP, bool MATS, bool QUEUE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(step_waves<VRULE>())))
void k_fused_step(const DevTensor* __restrict__ tab,
                                                     const int64_t* __restrict__ chunk_begin, int n_tensors,
                                                     int64_t total_chunks, int run_slabs, StepScalars sc) {
    constexpr bool FLAT = flat_tables<VCB, VRULE>();
    __shared__ StepLds<MCB, VCB, FLAT> lds;
    const int lane = threadIdx.x & 63;
    const int sub = lane & 15;
    LaneBooks lb;
    {
        // Stage the bucket tables and sorted levels in LDS.  Every global
        // load of the setup is issued before the first LDS store, so a
        // work-group's setup waits for L2 once (the loads use in-bounds
        // indices in every thread; only the stores are conditional).
        static_assert(Enc<VCB>::SIZE <= 256 && Enc<MCB>::SIZE <= 256 && Enc<VCB>::NPOS <= 256,
                      "one table entry per thread");
        const int t = threadIdx.x;
        const BucketEntry ev = enc_table_global<VCB>()[t < Enc<VCB>::SIZE ? t : 0];
        BucketEntry em{};
        FloorEntry ef{};
        FlatPieces fp{};
        if constexpr (FLAT) {
            // each flat slot takes the compact entry of a value inside it
            // (built at compile time, copied in 16-byte pieces)
            fp = load_flat_table<MCB>();
        } else {
            em = enc_table_global<MCB>()[t < Enc<MCB>::SIZE ? t : 0];
            if constexpr (VCB == Q4_CB_DYN4) ef = c_floor_dyn4.e[t < Enc<VCB>::NPOS ? t : 0];
        }
        // lane `sub`'s levels: lanes 0..15 of the group also fill the sorted
        // level tables
        const float lev_m = sub < Book<MCB>::N ? sorted_level_rt<MCB>(sub) : 1.0f;
        lb.dec_m = bits2f(c_decode[MCB][sub]);
        lb.dec_v = bits2f(c_decode[VCB][sub]);
        lb.lev_v = sub < Book<VCB>::N ? sorted_level_rt<VCB>(sub) : 1.0f;
        if (t < Enc<VCB>::SIZE) lds.enc_v[t] = ev;
        if constexpr (FLAT) {
            store_flat_table(lds.flat, fp);
        } else {
            if (t < Enc<MCB>::SIZE) lds.enc_m[t] = em;
            if constexpr (VCB == Q4_CB_DYN4)
                if (t < Enc<VCB>::NPOS) lds.floor_v[t] = ef;
        }
        if (t < 16) {
            lds.lev_m[t] = lev_m;
            lds.lev_v[t] = lb.lev_v;
        }
    }
    __syncthreads();

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // clipping is a separate instantiation: the unclipped kernel carries no
    // trace of it (its live values are what limits occupancy)
    const float gs = CLIP ? *clip_of_table(tab) : 1.0f;
    auto chunk_of = [&](int64_t c, int t) {
        const DevTensor T = tab[t];
        const int64_t lc = c - chunk_begin[t];
        if (lc * kChunkElems < T.numel) {  // beyond: a chunk that only aligns the next tensor
            const bool full = (lc + 1) * kChunkElems <= T.numel;
            if (!MATS || T.kind == KIND_PACKED) {
                if (full) step_chunk<MCB, VCB, VRULE, true, true, CLIP>(T, lc, c, sc, lds, lb, lane, gs);
                else step_chunk<MCB, VCB, VRULE, false, true, CLIP>(T, lc, c, sc, lds, lb, lane, gs);
            } else {
                if (full) step_chunk<MCB, VCB, VRULE, true, false, CLIP>(T, lc, c, sc, lds, lb, lane, gs);
                else step_chunk<MCB, VCB, VRULE, false, false, CLIP>(T, lc, c, sc, lds, lb, lane, gs);
            }
        }
    };
    static_assert(!QUEUE || queue_walk<MCB, VCB, VRULE, MATS>(), "no queue form for these maps");
    if constexpr (QUEUE) {
        // one round of resident groups taking runs from the workspace's queue
        // word (zeroed just before the launch), in increasing order
        __shared__ unsigned long long next_run;
        unsigned long long* const queue = queue_of_table(tab);
        const int64_t run_chunks = (int64_t)run_slabs * kWavesPerGroup;
        const int64_t runs = (total_chunks + run_chunks - 1) / run_chunks;
        int t = -1;
        for (;;) {
            if (threadIdx.x == 0) next_run = atomicAdd(queue, 1ull);
            __syncthreads();
            const unsigned long long rv = next_run;
            __syncthreads();  // every wave has read the run before thread 0 takes the next
            const int64_t r = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(rv >> 32)) << 32) |
                                        __builtin_amdgcn_readfirstlane((uint32_t)rv));
            if (r >= runs) break;
            int64_t c = r * run_chunks + wave;
            if (t < 0) t = first_tensor(chunk_begin, n_tensors, c);
            for (int s = 0; s < run_slabs && c < total_chunks; ++s, c += kWavesPerGroup) {
                while (t + 1 < n_tensors && chunk_begin[t + 1] <= c) ++t;
                chunk_of(c, t);
            }
        }
    } else {
        const int64_t G = gridDim.x;
        int64_t c = (int64_t)blockIdx.x * run_slabs * kWavesPerGroup + wave;
        int t = first_tensor(chunk_begin, n_tensors, c);
        for (int j = 0; c < total_chunks;) {
            while (t + 1 < n_tensors && chunk_begin[t + 1] <= c) ++t;
            chunk_of(c, t);
            c = next_chunk(c, j, run_slabs, G);
        }
    }
}

// ---------------------------------------------------------------------------
// K1 for the FP32 recipe (quantization off: plain 32-bit AdamW)
// ---------------------------------------------------------------------------

// One element of plain 32-bit AdamW, in the oracle's order of operations.
__device__ __forceinline__ void fp32_adamw(const StepScalars& sc, float g, float& p, float& m, float& v) {
    const float mm = __builtin_fmaf(sc.beta1, m, sc.omb1 * g);
    const float vv = __builtin_fmaf(sc.beta2, v, sc.omb2 * (g * g));
    const float denom = __builtin_fmaf(sqrtf(vv), sc.rsbc2, sc.eps);
    p = __builtin_fmaf(-sc.step_size, mm / denom, p * sc.decay);
    m = mm;
    v = vv;
}

// K1's lane layout (lane s of row r on elements 128r + 4s .. +3 and
// 128r + 64 + 4s .. +3 of the chunk, 16-byte accesses; scalar accesses only
// in a tensor's last partial lane) over the plain chunk prefix, in runs of
// slabs.  Every stream is read once and written once, all of them
// nontemporal.  Per-element loads (lanes 32 bytes apart in every
// instruction) ran the GPT-162M set at 1.9 TB/s.
__global__ __launch_bounds__(256) void k_fp32_step(const DevTensor* __restrict__ tab,
                                                    const int64_t* __restrict__ chunk_begin, int n_tensors,
                                                    int64_t total_chunks, int run_slabs, StepScalars sc) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int le = (lane & 48) * 8 + (lane & 15) * 4;
    const float gs = (sc.flags & SF_CLIP) ? *clip_of_table(tab) : 1.0f;
    const int64_t ngroups = gridDim.x;
    int64_t c = (int64_t)blockIdx.x * run_slabs * kWavesPerGroup + wave;
    int t = first_tensor(chunk_begin, n_tensors, c);
    for (int j = 0; c < total_chunks; c = next_chunk(c, j, run_slabs, ngroups)) {
        while (t + 1 < n_tensors && chunk_begin[t + 1] <= c) ++t;
        const DevTensor T = tab[t];
        const int64_t c0 = (c - T.chunk_begin) * kChunkElems;  // wave-uniform
        const gptr<float> P = G(T.param) + c0;
        const gptr<float> M = G(T.m32) + c0;
        const gptr<float> V = G(T.v32) + c0;
        const gptr<const uint16_t> Gr = G(T.grad) + c0;
        if (c0 + le + 68 <= T.numel) {
            float p[8], m[8], v[8], g[8];
            const f32x4 pa = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(P + le));
            const f32x4 pb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(P + le + 64));
            const f32x4 ma = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(M + le));
            const f32x4 mb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(M + le + 64));
            const f32x4 va = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(V + le));
            const f32x4 vb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(V + le + 64));
            const u32x2 ga = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(Gr + le));
            const u32x2 gb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(Gr + le + 64));
            p[0] = pa.x; p[1] = pa.y; p[2] = pa.z; p[3] = pa.w; p[4] = pb.x; p[5] = pb.y; p[6] = pb.z; p[7] = pb.w;
            m[0] = ma.x; m[1] = ma.y; m[2] = ma.z; m[3] = ma.w; m[4] = mb.x; m[5] = mb.y; m[6] = mb.z; m[7] = mb.w;
            v[0] = va.x; v[1] = va.y; v[2] = va.z; v[3] = va.w; v[4] = vb.x; v[5] = vb.y; v[6] = vb.z; v[7] = vb.w;
            const uint32_t gw[4] = {ga.x, ga.y, gb.x, gb.y};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                g[k] = bf16_to_f32((k & 1) ? gw[k >> 1] >> 16 : gw[k >> 1] & 0xFFFFu) * gs;
                fp32_adamw(sc, g[k], p[k], m[k], v[k]);
            }
            __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, reinterpret_cast<gptr<f32x4>>(P + le));
            __builtin_nontemporal_store(f32x4{p[4], p[5], p[6], p[7]}, reinterpret_cast<gptr<f32x4>>(P + le + 64));
            __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, reinterpret_cast<gptr<f32x4>>(M + le));
            __builtin_nontemporal_store(f32x4{m[4], m[5], m[6], m[7]}, reinterpret_cast<gptr<f32x4>>(M + le + 64));
            __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<gptr<f32x4>>(V + le));
            __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<gptr<f32x4>>(V + le + 64));
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int o = le + (k < 4 ? k : 60 + k);
                if (c0 + o < T.numel) {
                    float p = P[o], m = M[o], v = V[o];
                    fp32_adamw(sc, bf16_to_f32(Gr[o]) * gs, p, m, v);
                    P[o] = p;
                    M[o] = m;
                    V[o] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K1 of the 8-bit recipe: SDyn8 m, Dyn8 v, one byte per code
// ---------------------------------------------------------------------------
//
// Same lane layout as K1 (a 128-block per 16-lane row, lane s on its
// elements 4s .. 4s+3 and 64+4s .. 64+4s+3; masters and gradients
// nontemporal).  A code is one byte, so a lane's 8 codes of a moment are two
// 4-byte accesses.  256-entry maps do not fit ds_bpermute's 64 lanes: decoding
// reads a code-indexed table in LDS, and the nearest level comes from the
// bucket tables of q4_quant.h (Step8Lds, rtn8_m, rtn8_v).

template <bool FULL, bool CLIP>
__device__ __forceinline__ void step8_chunk(const DevTensor& T, const int64_t lc, const StepScalars& sc,
                                            const Step8Lds& lds, const int lane, const float gs) {
    const int sub = lane & 15;
    const int64_t n = T.numel;
    const int64_t blk = lc * kBlocksPerChunk + (lane >> 4);
    const int64_t e0 = blk * kBlock + sub * 4;
    int nva = 4, nvb = 4;  // valid elements of the lane's two halves
    bool blk_ok = true;
    if (!FULL) {
        const int64_t ra = n - e0, rb2 = n - (e0 + 64);
        nva = ra >= 4 ? 4 : (ra > 0 ? (int)ra : 0);
        nvb = rb2 >= 4 ? 4 : (rb2 > 0 ? (int)rb2 : 0);
        blk_ok = blk * kBlock < n;
    }
    const bool lane_full = FULL || nvb == 4;
    auto valid = [&](int k) { return FULL || (k < 4 ? k < nva : k - 4 < nvb); };
    const gptr<float> param = G(T.param);
    const gptr<const uint16_t> grad = G(T.grad);
    const gptr<uint8_t> mcodes = G(T.m_codes);
    const gptr<uint8_t> vcodes = G(T.v_codes);
    const gptr<float> mscales = G(T.m_scales);
    const gptr<float> vscales = G(T.v_scales);

    // loads at raised wave priority, as in the 4-bit step
    __builtin_amdgcn_s_setprio(2);
    float p[8], g[8];
    uint32_t mc[2] = {0u, 0u}, vc[2] = {0u, 0u};
    if (lane_full) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(param + e0));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(param + e0 + 64));
        p[0] = a.x; p[1] = a.y; p[2] = a.z; p[3] = a.w; p[4] = b.x; p[5] = b.y; p[6] = b.z; p[7] = b.w;
        const u32x2 ga = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(grad + e0));
        const u32x2 gb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(grad + e0 + 64));
        g[0] = bf16_to_f32(ga.x & 0xFFFFu); g[1] = bf16_to_f32(ga.x >> 16);
        g[2] = bf16_to_f32(ga.y & 0xFFFFu); g[3] = bf16_to_f32(ga.y >> 16);
        g[4] = bf16_to_f32(gb.x & 0xFFFFu); g[5] = bf16_to_f32(gb.x >> 16);
        g[6] = bf16_to_f32(gb.y & 0xFFFFu); g[7] = bf16_to_f32(gb.y >> 16);
        mc[0] = *reinterpret_cast<const gptr<const uint32_t>>(mcodes + e0);
        mc[1] = *reinterpret_cast<const gptr<const uint32_t>>(mcodes + e0 + 64);
        vc[0] = *reinterpret_cast<const gptr<const uint32_t>>(vcodes + e0);
        vc[1] = *reinterpret_cast<const gptr<const uint32_t>>(vcodes + e0 + 64);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t o = e0 + (k < 4 ? k : 60 + k);
            p[k] = valid(k) ? param[o] : 0.0f;
            g[k] = valid(k) ? bf16_to_f32(grad[o]) : 0.0f;
            if (valid(k)) {
                mc[k >> 2] |= (uint32_t)mcodes[o] << (8 * (k & 3));
                vc[k >> 2] |= (uint32_t)vcodes[o] << (8 * (k & 3));
            }
        }
    }
    if constexpr (CLIP) {
#pragma unroll
        for (int k = 0; k < 8; ++k) g[k] *= gs;
    }
    const float sm_old = (FULL || blk_ok) ? mscales[blk] : 0.0f;
    const float sv_old = (FULL || blk_ok) ? vscales[blk] : 0.0f;
    __builtin_amdgcn_s_setprio(0);

    float m1[8], v1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t cm = (mc[k >> 2] >> (8 * (k & 3))) & 0xFFu;
        const uint32_t cv = (vc[k >> 2] >> (8 * (k & 3))) & 0xFFu;
        const float m0 = lds.dec_m[cm] * sm_old;
        const float v0 = lds.dec_v[cv] * sv_old;
        m1[k] = __builtin_fmaf(sc.beta1, m0, sc.omb1 * g[k]);
        v1[k] = __builtin_fmaf(sc.beta2, v0, sc.omb2 * (g[k] * g[k]));
        const float denom = __builtin_fmaf(__builtin_amdgcn_sqrtf(v1[k]), sc.rsbc2, sc.eps);
        p[k] = __builtin_fmaf(-sc.step_size, m1[k] * __builtin_amdgcn_rcpf(denom), p[k] * sc.decay);
        if (!valid(k)) {
            m1[k] = 0.0f;
            v1[k] = 0.0f;
        }
    }
    if (lane_full) {
        __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, reinterpret_cast<gptr<f32x4>>(param + e0));
        __builtin_nontemporal_store(f32x4{p[4], p[5], p[6], p[7]}, reinterpret_cast<gptr<f32x4>>(param + e0 + 64));
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (valid(k)) param[e0 + (k < 4 ? k : 60 + k)] = p[k];
    }

    float am = 0.0f, av = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        am = fmaxf(am, fabsf(m1[k]));
        av = fmaxf(av, v1[k]);
    }
    const float s_m = row_max16(am), s_v = row_max16(av);
    const float inv_m = inv_scale(s_m);
    const float inv_v = inv_scale(s_v);
    uint32_t mw[2] = {0u, 0u}, vw[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float xm = fminf(fmaxf(m1[k] * inv_m, -1.0f), 1.0f);
        const float xv = normalize_v(v1[k], inv_v);
        mw[k >> 2] |= rtn8_m(lds, xm) << (8 * (k & 3));
        vw[k >> 2] |= rtn8_v(lds, xv) << (8 * (k & 3));
    }
    if (lane_full) {
        *reinterpret_cast<gptr<uint32_t>>(mcodes + e0) = mw[0];
        *reinterpret_cast<gptr<uint32_t>>(mcodes + e0 + 64) = mw[1];
        *reinterpret_cast<gptr<uint32_t>>(vcodes + e0) = vw[0];
        *reinterpret_cast<gptr<uint32_t>>(vcodes + e0 + 64) = vw[1];
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (valid(k)) {
                const int64_t o = e0 + (k < 4 ? k : 60 + k);
                mcodes[o] = (uint8_t)(mw[k >> 2] >> (8 * (k & 3)));
                vcodes[o] = (uint8_t)(vw[k >> 2] >> (8 * (k & 3)));
            }
        }
    }
    if ((FULL || blk_ok) && sub == 0) {
        mscales[blk] = s_m;
        vscales[blk] = s_v;
    }
}

// One round of resident work-groups takes runs of run_slabs slabs from the
// queue word of the workspace (zeroed by k_zero_queue just before the
// launch), in increasing order, until none is left.  Each group builds its
// tables once for all its runs.  For this byte mix the queue moves 6% more
// than one group per run (the bandwidth probes' two forms of the 8-bit mix);
// the step took 3.6% less time with it (GPT-2.7B, one process, same buffers).
// Its registers are held to 8 wavefronts per SIMD: left to itself the
// allocator takes the queue loop to 69 VGPRs and 7.
template <bool CLIP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void k_step8(const DevTensor* __restrict__ tab,
                                                const int64_t* __restrict__ chunk_begin, int n_tensors,
                                                int64_t total_chunks, int run_slabs, StepScalars sc) {
    __shared__ Step8Lds lds;
    __shared__ unsigned long long next_run;
    step8_tables(lds);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float gs = CLIP ? *clip_of_table(tab) : 1.0f;
    unsigned long long* const queue = queue_of_table(tab);
    const int64_t run_chunks = (int64_t)run_slabs * kWavesPerGroup;
    const int64_t runs = (total_chunks + run_chunks - 1) / run_chunks;
    int t = -1;
    for (;;) {
        if (threadIdx.x == 0) next_run = atomicAdd(queue, 1ull);
        __syncthreads();
        const int64_t r = (int64_t)next_run;
        __syncthreads();  // every wave has read the run before thread 0 takes the next
        if (r >= runs) break;  // uniform over the group
        int64_t c = r * run_chunks + wave;
        // the runs a group takes increase, so its tensor index only moves on
        if (t < 0) t = first_tensor(chunk_begin, n_tensors, c);
        for (int s = 0; s < run_slabs && c < total_chunks; ++s, c += kWavesPerGroup) {
            while (t + 1 < n_tensors && chunk_begin[t + 1] <= c) ++t;
            const DevTensor T = tab[t];
            const int64_t lc = c - chunk_begin[t];
            if (lc * kChunkElems < T.numel) {  // beyond: a chunk that only aligns the next tensor
                if ((lc + 1) * kChunkElems <= T.numel) step8_chunk<true, CLIP>(T, lc, sc, lds, lane, gs);
                else step8_chunk<false, CLIP>(T, lc, sc, lds, lane, gs);
            }
        }
    }
}

// The 8-bit step's queue word set to 0 (a kernel, so that a captured graph
// clears it on every replay).
__global__ void k_zero_queue(unsigned long long* q) {
    if (threadIdx.x == 0) *q = 0ull;
}

__global__ __launch_bounds__(256) void k_dequant8(DevTensor T, float* __restrict__ m_out, float* __restrict__ v_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T.numel) return;
    m_out[i] = bits2f(c_cb8[0][T.m_codes[i]]) * T.m_scales[i / kBlock];
    v_out[i] = bits2f(c_cb8[1][T.v_codes[i]]) * T.v_scales[i / kBlock];
}

// ---------------------------------------------------------------------------
// K2 / K3: factored second moment (row and column means of g^2)
// ---------------------------------------------------------------------------

template <int CTRL> __device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum of one double per lane over the wavefront in a fixed order: a DPP
// tree within each 16-lane row, then the four rows in order (wave-uniform
// result).
__device__ __forceinline__ double wave_sum_d(double v) {
    v = v + dpp_d<DPP_QUAD_1032>(v);
    v = v + dpp_d<DPP_QUAD_2301>(v);
    v = v + dpp_d<DPP_ROW_HALF_MIRROR>(v);
    v = v + dpp_d<DPP_ROW_MIRROR>(v);
    return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}

// Sum over the 256 threads of a work-group, tree in LDS in fixed order.
__device__ __forceinline__ double group_sum_d(double v, double* lds) {
    lds[threadIdx.x] = v;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) lds[threadIdx.x] = lds[threadIdx.x] + lds[threadIdx.x + s];
        __syncthreads();
    }
    const double r = lds[0];
    __syncthreads();
    return r;
}

__device__ __forceinline__ int find_matrix(const DevMatrix* mats, int n, int64_t x, int which) {
    // last matrix whose begin (tile / row group / column group) is <= x
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t b = which == 0 ? mats[mid].tile_begin : (which == 1 ? mats[mid].rgroup_begin
                                                                          : mats[mid].cgroup_begin);
        if (b <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// K2: one work-group per (band of 256 rows) x (tile of 512 columns).  Lane
// j of every wave owns columns 8j..8j+7 of the tile; wave w takes rows
// w, w+4, ... of the band.  Column partials stay in registers (binary64)
// and are combined across the 4 waves in LDS; each row's partial over the
// tile is a wavefront butterfly.  No atomics: the order is fixed.
// FP32 -> BF16 bits, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// Two BF16 values packed in a word: acc <- micro (FIRST), bf16(acc + micro)
// (ADD) or acc (statistics only).
template <int MODE> __device__ __forceinline__ uint32_t grad_pair(uint32_t acc, uint32_t micro) {
    if constexpr (MODE == GRAD_STATS_ONLY) return acc;
    if constexpr (MODE == GRAD_FIRST) return micro;
    const uint32_t lo = f32_to_bf16_rne(bf16_to_f32(acc & 0xFFFFu) + bf16_to_f32(micro & 0xFFFFu));
    const uint32_t hi = f32_to_bf16_rne(bf16_to_f32(acc >> 16) + bf16_to_f32(micro >> 16));
    return lo | (hi << 16);
}

// K2 (MODE = GRAD_STATS_ONLY), or the last microbatch's accumulation pass
// for the factored matrices (FIRST / ADD): a band of 256 rows x a tile of 512
// columns per work-group; wave w takes rows w, w+4, ... of the band.  Column
// partials stay in registers (binary64) and are combined across the 4 waves
// in LDS; each row's partial over the tile is a wavefront butterfly.  No
// atomics: the order is fixed.  With sq_part the work-group also leaves the
// binary64 sum of its squares (its rows' partials, wave by wave) at
// sq_part[tile].
template <int MODE>
__global__ __launch_bounds__(256) void k_rowcol_partial(const DevMatrix* __restrict__ mats, int n_mats,
                                                         const uint16_t* __restrict__ micro,
                                                         double* __restrict__ sq_part) {
    __shared__ double lds[kWavesPerGroup][kTileCols];
    const int64_t tile = blockIdx.x;
    const int mi = find_matrix(mats, n_mats, tile, 0);
    const DevMatrix M = mats[mi];
    const int64_t local = tile - M.tile_begin;
    const int64_t band = local / M.n_ctiles, ctile = local % M.n_ctiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = band * kBandRows;
    const int64_t r1 = r0 + kBandRows < M.rows ? r0 + kBandRows : M.rows;
    const int64_t c0 = ctile * kTileCols + lane * 8;
    const int64_t cr = M.cols - c0;
    const int ncv = cr >= 8 ? 8 : (cr > 0 ? (int)cr : 0);
    const bool vec = ncv == 8 && (M.cols & 7) == 0;
    double col[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) col[k] = 0.0;
    double sq_wave = 0.0;
    // rows r0 + wave, r0 + wave + 4, ...; four rows' loads are issued before
    // any of them is reduced, so each wave keeps four loads in flight
    const gptr<uint16_t> grad = G(const_cast<uint16_t*>(M.grad));
    const gptr<const uint16_t> mic = G(micro + (MODE == GRAD_STATS_ONLY ? 0 : M.flat_off));
    constexpr int U = 4;
    for (int64_t rb = r0 + wave; rb < r1; rb += U * kWavesPerGroup) {
        u32x4 q[U], mq[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = rb + (int64_t)u * kWavesPerGroup;
            q[u] = u32x4{0u, 0u, 0u, 0u};
            mq[u] = u32x4{0u, 0u, 0u, 0u};
            if (r < r1) {
                const int64_t off = r * M.cols + c0;
                if (vec) {
                    // 1 KiB of whole lines per instruction: streaming loads
                    if constexpr (MODE != GRAD_FIRST)
                        q[u] = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x4>>(grad + off));
                    if constexpr (MODE != GRAD_STATS_ONLY)
                        mq[u] = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x4>>(mic + off));
                } else {
                    uint32_t w[4] = {0u, 0u, 0u, 0u}, mw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        if (k < ncv) {
                            if constexpr (MODE != GRAD_FIRST) w[k >> 1] |= (uint32_t)grad[off + k] << (16 * (k & 1));
                            if constexpr (MODE != GRAD_STATS_ONLY)
                                mw[k >> 1] |= (uint32_t)mic[off + k] << (16 * (k & 1));
                        }
                    }
                    q[u] = u32x4{w[0], w[1], w[2], w[3]};
                    mq[u] = u32x4{mw[0], mw[1], mw[2], mw[3]};
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = rb + (int64_t)u * kWavesPerGroup;
            if (r >= r1) break;  // wave-uniform
            uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
            if constexpr (MODE != GRAD_STATS_ONLY) {
                const uint32_t mw[4] = {mq[u].x, mq[u].y, mq[u].z, mq[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) w[k] = grad_pair<MODE>(w[k], mw[k]);
                const int64_t off = r * M.cols + c0;
                if (vec) {
                    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<gptr<u32x4>>(grad + off));
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (k < ncv) grad[off + k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
                }
            }
            double d[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float a = bf16_to_f32(w[k] & 0xFFFFu), b = bf16_to_f32(w[k] >> 16);
                d[2 * k] = (double)(a * a);
                d[2 * k + 1] = (double)(b * b);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) col[k] += d[k];
            const double rp = ((d[0] + d[1]) + (d[2] + d[3])) + ((d[4] + d[5]) + (d[6] + d[7]));
            const double rs = wave_sum_d(rp);
            if (lane == 0) M.part_row[ctile * M.rows + r] = rs;
            sq_wave += rs;
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) lds[wave][lane * 8 + k] = col[k];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k < ncv) {
                const int j = lane * 8 + k;
                M.part_col[band * M.cols + c0 + k] = ((lds[0][j] + lds[1][j]) + lds[2][j]) + lds[3][j];
            }
        }
    }
    if (sq_part) {
        __syncthreads();
        if (lane == 0) lds[0][wave] = sq_wave;
        __syncthreads();
        if (threadIdx.x == 0) sq_part[tile] = ((lds[0][0] + lds[0][1]) + lds[0][2]) + lds[0][3];
    }
}

// The accumulation / statistics pass in chunk order over the tensors of
// `tab` (every tensor, or all but the factored matrices when the tile kernel
// above takes them), over tensor-aligned chunks of 512 elements numbered by
// the prefix `chunk_begin`, lane l on elements 8l .. 8l+7.  Work-groups walk
// runs of consecutive slabs as the step kernels do (next_chunk): with no
// block scales to write, the longer runs of adjacent addresses alone made
// the GPT-2.7B pass 3.13 -> 3.01 ms.  micro
// holds the microbatch gradients flat: tensor i at element 512 times its
// chunk_begin in the full prefix (the table entry's own field).  With LAST each lane keeps a binary64 sum
// of its squares over its chunks; the work-group leaves the sum of its four
// waves at sq_part[blockIdx.x].
template <int MODE, bool LAST>
__global__ __launch_bounds__(256) void k_grad_chunks(const DevTensor* __restrict__ tab,
                                                      const int64_t* __restrict__ chunk_begin, int n_tensors,
                                                      int64_t total_chunks, int run_slabs,
                                                      const uint16_t* __restrict__ micro,
                                                      double* __restrict__ sq_part) {
    __shared__ double lds[kWavesPerGroup];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    double sq = 0.0;
    const int64_t groups = gridDim.x;
    int64_t c = (int64_t)blockIdx.x * run_slabs * kWavesPerGroup + wave;
    int t = first_tensor(chunk_begin, n_tensors, c);
    for (int j = 0; c < total_chunks; c = next_chunk(c, j, run_slabs, groups)) {
        while (t + 1 < n_tensors && chunk_begin[t + 1] <= c) ++t;
        const DevTensor T = tab[t];
        const int64_t lc = c - chunk_begin[t];
        const int64_t e0 = lc * kChunkElems + lane * 8;
        const int64_t rem = T.numel - e0;
        const int nv = rem >= 8 ? 8 : (rem > 0 ? (int)rem : 0);
        const gptr<uint16_t> gp = G(const_cast<uint16_t*>(T.grad)) + e0;
        const gptr<const uint16_t> mp = G(micro + (MODE == GRAD_STATS_ONLY ? 0 : T.chunk_begin * kChunkElems)) + e0;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (nv == 8) {
            u32x4 q = u32x4{0u, 0u, 0u, 0u}, m = u32x4{0u, 0u, 0u, 0u};
            // each instruction covers 1 KiB of whole lines, read and written
            // once: streaming (nontemporal) accesses
            if constexpr (MODE != GRAD_FIRST) q = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x4>>(gp));
            if constexpr (MODE != GRAD_STATS_ONLY) m = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x4>>(mp));
            w[0] = grad_pair<MODE>(q.x, m.x);
            w[1] = grad_pair<MODE>(q.y, m.y);
            w[2] = grad_pair<MODE>(q.z, m.z);
            w[3] = grad_pair<MODE>(q.w, m.w);
            if constexpr (MODE != GRAD_STATS_ONLY)
                __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<gptr<u32x4>>(gp));
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (k < nv) {
                    const uint32_t x = MODE != GRAD_FIRST ? (uint32_t)gp[k] : 0u;
                    const uint32_t y = MODE != GRAD_STATS_ONLY ? (uint32_t)mp[k] : 0u;
                    const uint32_t o = grad_pair<MODE>(x, y) & 0xFFFFu;
                    if constexpr (MODE != GRAD_STATS_ONLY) gp[k] = (uint16_t)o;
                    w[k >> 1] |= o << (16 * (k & 1));
                }
            }
        }
        if constexpr (LAST) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float x = bf16_to_f32(w[k] & 0xFFFFu), y = bf16_to_f32(w[k] >> 16);
                sq += (double)(x * x);
                sq += (double)(y * y);
            }
        }
    }
    if constexpr (LAST) {
        const double wsum = wave_sum_d(sq);
        if (lane == 0) lds[wave] = wsum;
        __syncthreads();
        if (threadIdx.x == 0) sq_part[blockIdx.x] = ((lds[0] + lds[1]) + lds[2]) + lds[3];
    }
}

// First stage of the total of the partial sums of squares: group g sums its
// slice of the slots (thread t adds slots t, t+256, ... of the slice in
// order, then a fixed tree over the threads); a slice past the end gives 0.
__global__ __launch_bounds__(256) void k_sq_stage(const double* __restrict__ part, int64_t n,
                                                  double* __restrict__ out) {
    __shared__ double lds[256];
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < n ? lo + per : n;
    double s = 0.0;
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) s += part[i];
    const double tot = group_sum_d(s, lds);
    if (threadIdx.x == 0) out[blockIdx.x] = tot;
}

// Total of the partial sums of squares: thread t adds slots t, t+256, ... in
// order, then a fixed tree over the threads.
__global__ __launch_bounds__(256) void k_sq_total(const double* __restrict__ part, int64_t n,
                                                   double* __restrict__ out) {
    __shared__ double lds[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += part[i];
    const double tot = group_sum_d(s, lds);
    if (threadIdx.x == 0) *out = tot;
}

// Clip factor as torch.nn.utils.clip_grad_norm_ forms it, in binary64 (IEEE
// square root and division), rounded to FP32.
__global__ void k_clip_factor(const double* __restrict__ sq, float max_norm, float* __restrict__ clip) {
    if (threadIdx.x == 0) {
        const double c = (double)max_norm / (sqrt(*sq) + 1e-6);
        *clip = c < 1.0 ? (float)c : 1.0f;
    }
}

// K3a: finalize rows (first total_rgroups groups) and columns (the rest).
// R_r <- b2 R_r + (1-b2) (row sum / cols), C_c likewise with rows; each row
// group also leaves the binary64 sum of its updated R for the mean.
__global__ __launch_bounds__(256) void k_rowcol_finalize(const DevMatrix* __restrict__ mats, int n_mats,
                                                          int64_t total_rgroups, float beta2, float omb2,
                                                          const float* __restrict__ clip) {
    __shared__ double lds[256];
    const int64_t g = blockIdx.x;
    // clipped gradient: its sums of squares are s^2 times the gathered ones
    const double s2 = clip ? (double)*clip * (double)*clip : 1.0;
    if (g < total_rgroups) {
        const int mi = find_matrix(mats, n_mats, g, 1);
        const DevMatrix M = mats[mi];
        const int64_t lg = g - M.rgroup_begin;
        const int64_t r = lg * kGroup + threadIdx.x;
        double mine = 0.0;
        if (r < M.rows) {
            double rs = 0.0;
            for (int64_t ct = 0; ct < M.n_ctiles; ++ct) rs += M.part_row[ct * M.rows + r];
            const float Rn = beta2 * M.R[r] + omb2 * ((float)(rs * s2) / (float)M.cols);
            M.R[r] = Rn;
            mine = (double)Rn;
        }
        const double s = group_sum_d(mine, lds);
        if (threadIdx.x == 0) M.part_mean[lg] = s;
    } else {
        // kColGroup columns, wave w summing bands w, w + 4, ... of each (a
        // wave reads 64 consecutive columns of a band); eight interleaved
        // accumulators per lane keep eight loads in flight; the lane's
        // accumulators and then the four waves combine in a fixed tree
        const int64_t cg = g - total_rgroups;
        const int mi = find_matrix(mats, n_mats, cg, 2);
        const DevMatrix M = mats[mi];
        const int lane = threadIdx.x & 63, slice = threadIdx.x >> 6;
        const int64_t cidx = (cg - M.cgroup_begin) * kColGroup + lane;
        double cs = 0.0;
        if (cidx < M.cols) {
            double a[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
            int64_t b = slice;
            for (; b + 28 < M.n_bands; b += 32) {
#pragma unroll
                for (int j = 0; j < 8; ++j) a[j] += M.part_col[(b + 4 * j) * M.cols + cidx];
            }
            for (int j = 0; b < M.n_bands; b += 4, ++j) a[j] += M.part_col[b * M.cols + cidx];
            cs = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
        }
        lds[threadIdx.x] = cs;
        __syncthreads();
        if (slice == 0 && cidx < M.cols) {
            const double t = (lds[lane] + lds[64 + lane]) + (lds[128 + lane] + lds[192 + lane]);
            M.C[cidx] = beta2 * M.C[cidx] + omb2 * ((float)(t * s2) / (float)M.rows);
        }
    }
}

// 1 / mean(R) from the per-group sums of R: thread t adds groups t, t+256,
// ... in order, then a fixed tree over the threads.  The step and the
// dequantization both use this, so they agree bit for bit.
__device__ __forceinline__ float inv_mean_of(const double* __restrict__ part, int64_t n_groups, int64_t rows,
                                             double* lds) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n_groups; i += 256) s += part[i];
    const double tot = group_sum_d(s, lds);
    const float meanR = (float)(tot / (double)rows);
    return meanR > 0.0f ? 1.0f / meanR : 0.0f;
}

// K3b: one work-group per matrix.
__global__ __launch_bounds__(256) void k_rowcol_mean(const DevMatrix* __restrict__ mats) {
    __shared__ double lds[256];
    const DevMatrix M = mats[blockIdx.x];
    const float inv = inv_mean_of(M.part_mean, M.n_rgroups, M.rows, lds);
    if (threadIdx.x == 0) *M.inv_meanR = inv;
}

// Group sums of the stored R (same tree as K3a), for dequantization.
__global__ __launch_bounds__(256) void k_rsum_groups(const float* __restrict__ R, int64_t rows, double* part) {
    __shared__ double lds[256];
    const int64_t r = (int64_t)blockIdx.x * kGroup + threadIdx.x;
    const double s = group_sum_d(r < rows ? (double)R[r] : 0.0, lds);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}
__global__ __launch_bounds__(256) void k_rsum_final(const double* __restrict__ part, int64_t n_groups, int64_t rows,
                                                    float* inv) {
    __shared__ double lds[256];
    const float v = inv_mean_of(part, n_groups, rows, lds);
    if (threadIdx.x == 0) *inv = v;
}

// ---------------------------------------------------------------------------
// Init fill and dequantization
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_fill(uint8_t* __restrict__ p, size_t bytes, uint8_t value) {
    const uint32_t w = value * 0x01010101u;
    const uint4 q = make_uint4(w, w, w, w);
    const size_t nvec = bytes / 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (size_t)gridDim.x * blockDim.x)
        reinterpret_cast<uint4*>(p)[i] = q;
    if (blockIdx.x == 0 && threadIdx.x < bytes - nvec * 16) p[nvec * 16 + threadIdx.x] = value;
}

template <int MCB, int VCB>
__global__ __launch_bounds__(256) void k_dequant(DevTensor T, float* __restrict__ m_out, float* __restrict__ v_out,
                                                  const float* __restrict__ inv_meanR) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T.numel) return;
    const int64_t blk = i / kBlock;
    const uint32_t mc = (T.m_codes[i >> 1] >> ((i & 1) * 4)) & 15u;
    m_out[i] = bits2f(c_decode[MCB][mc]) * T.m_scales[blk];
    if (T.kind == KIND_PACKED) {
        const uint32_t vc = (T.v_codes[i >> 1] >> ((i & 1) * 4)) & 15u;
        v_out[i] = bits2f(c_decode[VCB][vc]) * T.v_scales[blk];
    } else {
        const int64_t r = i / T.cols, c = i % T.cols;
        v_out[i] = (T.v_row[r] * T.v_col[c]) * *inv_meanR;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// Resident 256-thread work-groups of a kernel on the current device (its
// occupancy per CU, cached by the caller, times the CUs; no dynamic LDS).
template <class K>
static int64_t resident_groups(K kernel, std::atomic<int>& per_cu_cache) {
    static std::atomic<int> cus{0};
    if (cus.load() == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        const bool ok = hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess;
        cus.store(ok && prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256);
    }
    int per_cu = per_cu_cache.load();
    if (per_cu == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1)
            per_cu = 1;
        per_cu_cache.store(per_cu);
    }
    return (int64_t)per_cu * cus.load();
}

// Most work-groups of one launch; a set with more runs loops over them.
constexpr int64_t kMaxRunGroups = int64_t(1) << 22;

// Grid and run length of the quantized steps: one work-group per run of
// slabs.  The dispatcher starts the groups in order as earlier ones finish,
// so it hands out the runs like a queue, the fastest order found for these
// steps' bytes.  Against the earlier grids of a few times the resident
// groups looping over runs (gfx950, alternating processes, one box):
// GPT-2.7B ZIP-SR 6.634 -> 6.425 ms, ZE-EDEN 6.352 -> 6.229 ms, 8-bit
// 7.427 -> 7.331 ms; Llama-1.1B ZIP-SR 2.789 -> 2.699 ms; GPT-162M ZIP-SR
// 0.327 -> 0.316 ms; the Qwen3-0.6B factored step 1.653 -> 1.525 ms (from
// accumulated statistics 1.408 -> 1.265 ms); the FP32 step, whose groups
// had swept the chunks grid-stride, 13.925 -> 13.49 ms.  Grids of 16x-32x
// the resident groups that loop were slower than both (ZIP-SR 6.84 ms).
// Runs are of max_run slabs, shortened while the set has fewer runs than
// resident groups.  The best length depends on the group's setup and on the
// access policy.  Measured with the streaming row-block kernels, each pair in
// one process over the same buffers (GPT-2.7B unless named): the ZIP-SR
// kernels, whose groups each copy a 24.5 KB table, take runs of 8 (4 slabs
// 1.7% slower, Llama-1.1B 1.4%; 16 slabs 2.3% slower); the others take runs
// of 2, which fill one 128-byte line of each scale stream (ZE-EDEN 1.7% and
// FP32 3.6% faster than 4, the factored step alike; 8 slabs 3-4% slower than
// 4).  The 8-bit step, and the ZE-EDEN kernel on large sets, take runs of 4
// from a queue.
struct RunLaunch {
    int grid, run_slabs;
};
constexpr int kRunSlabsFlat = 8, kRunSlabsCompact = 2, kRunSlabs8 = 4, kRunSlabsQueue = 4;
constexpr int64_t kQueueMinRunsPerGroup = 64;
template <class K>
static RunLaunch run_per_group(K kernel, int64_t total_chunks, std::atomic<int>& per_cu_cache, int max_run) {
    const int64_t resident = resident_groups(kernel, per_cu_cache);
    const int64_t slabs = (total_chunks + kWavesPerGroup - 1) / kWavesPerGroup;
    int r = max_run;
    // a set of fewer than 8 rounds of groups takes runs of at most 4 slabs,
    // for a finer last round (GPT-162M ZIP-SR 0.3177 -> 0.3161 ms)
    if (r > 4 && slabs / r < 8 * resident) r = 4;
    while (r > 1 && slabs / r < resident) r >>= 1;
    const int64_t runs = (slabs + r - 1) / r;
    return {(int)(runs < 1 ? 1 : (runs > kMaxRunGroups ? kMaxRunGroups : runs)), r};
}

// One round of resident groups (no more than there are runs) over runs of
// the length run_per_group picks.
template <class K>
static RunLaunch queue_launch(K kernel, int64_t total_chunks, std::atomic<int>& per_cu_cache, int max_run) {
    const RunLaunch L = run_per_group(kernel, total_chunks, per_cu_cache, max_run);
    const int64_t resident = resident_groups(kernel, per_cu_cache);
    return {(int)(L.grid < resident ? L.grid : resident), L.run_slabs};
}

#define Q4_VARIANTS(X)                                              \
    X(Q4_CB_NF4, Q4_CB_DYN4, Q4_RULE_UPDATE_SR)    /* ZIP-SR */    \
    X(Q4_CB_NF4, Q4_CB_DYN4_NZ, Q4_RULE_STATE_RTN) /* ZE-EDEN, factored */ \
    X(Q4_CB_NF4, Q4_CB_DYN4, Q4_RULE_STATE_RTN)                     \
    X(Q4_CB_NF4, Q4_CB_DYN4, Q4_RULE_STATE_SR)                      \
    X(Q4_CB_NF4, Q4_CB_DYN4, Q4_RULE_UPDATE_RTN)                    \
    X(Q4_CB_SDYN4, Q4_CB_LIN4_NZ, Q4_RULE_STATE_RTN) /* TorchAO-style */ \
    X(Q4_CB_SDYN4, Q4_CB_DYN4_NZ, Q4_RULE_STATE_RTN)                \
    X(Q4_CB_SDYN4, Q4_CB_DYN4, Q4_RULE_UPDATE_SR)

bool variant_supported(const Variant& v) {
#define Q4_MATCH(A, B, C) if (v.mcb == A && v.vcb == B && v.vrule == C) return true;
    Q4_VARIANTS(Q4_MATCH)
#undef Q4_MATCH
    return false;
}

template <int A, int B, int C, bool CLIP, bool MATS>
static hipError_t launch_step_kernel(const StepScalars& sc, const DevTensor* d_tab, const int64_t* d_chunk_begin,
                                     int n_tensors, int64_t total_chunks, hipStream_t stream) {
    static std::atomic<int> occ{0};
    if constexpr (queue_walk<A, B, C, MATS>()) {
        static std::atomic<int> occq{0};
        const int64_t resident = resident_groups(k_fused_step<A, B, C, CLIP, MATS, true>, occq);
        const int64_t slabs = (total_chunks + kWavesPerGroup - 1) / kWavesPerGroup;
        if ((slabs + kRunSlabsQueue - 1) / kRunSlabsQueue >= kQueueMinRunsPerGroup * resident) {
            k_zero_queue<<<1, 64, 0, stream>>>(queue_of_table(d_tab));
            const RunLaunch L =
                queue_launch(k_fused_step<A, B, C, CLIP, MATS, true>, total_chunks, occq, kRunSlabsQueue);
            k_fused_step<A, B, C, CLIP, MATS, true><<<L.grid, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors,
                                                                                total_chunks, L.run_slabs, sc);
            return hipGetLastError();
        }
    }
    const RunLaunch L = run_per_group(k_fused_step<A, B, C, CLIP, MATS>, total_chunks, occ,
                                      flat_tables<B, C>() ? kRunSlabsFlat : kRunSlabsCompact);
    k_fused_step<A, B, C, CLIP, MATS><<<L.grid, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors, total_chunks,
                                                                  L.run_slabs, sc);
    return hipGetLastError();
}

template <int A, int B, int C>
static hipError_t launch_variant(const StepScalars& sc, const DevTensor* d_tab, const int64_t* d_chunk_begin,
                                 int n_tensors, int64_t total_chunks, bool has_matrices, hipStream_t stream) {
    const bool clip = (sc.flags & SF_CLIP) != 0;
    if constexpr (factored_maps<A, B, C>()) {
        if (has_matrices)
            return clip ? launch_step_kernel<A, B, C, true, true>(sc, d_tab, d_chunk_begin, n_tensors, total_chunks,
                                                                  stream)
                        : launch_step_kernel<A, B, C, false, true>(sc, d_tab, d_chunk_begin, n_tensors, total_chunks,
                                                                   stream);
    } else {
        if (has_matrices) return hipErrorInvalidValue;  // only the factored recipe's maps take matrices
    }
    return clip ? launch_step_kernel<A, B, C, true, false>(sc, d_tab, d_chunk_begin, n_tensors, total_chunks, stream)
                : launch_step_kernel<A, B, C, false, false>(sc, d_tab, d_chunk_begin, n_tensors, total_chunks, stream);
}

hipError_t launch_fused_step(const Variant& v, const StepScalars& sc, const DevTensor* d_tab,
                             const int64_t* d_chunk_begin, int n_tensors, int64_t total_chunks, bool has_matrices,
                             hipStream_t stream) {
    if (total_chunks <= 0) return hipSuccess;
#define Q4_LAUNCH(A, B, C)                                                                            \
    if (v.mcb == A && v.vcb == B && v.vrule == C)                                                     \
        return launch_variant<A, B, C>(sc, d_tab, d_chunk_begin, n_tensors, total_chunks, has_matrices, stream);
    Q4_VARIANTS(Q4_LAUNCH)
#undef Q4_LAUNCH
    return hipErrorInvalidValue;
}

hipError_t launch_fp32_step(const StepScalars& sc, const DevTensor* d_tab, const int64_t* d_chunk_begin,
                            int n_tensors, int64_t total_chunks, hipStream_t stream) {
    if (total_chunks <= 0) return hipSuccess;
    static std::atomic<int> occ{0};
    const RunLaunch L = run_per_group(k_fp32_step, total_chunks, occ, kRunSlabsCompact);
    k_fp32_step<<<L.grid, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors, total_chunks, L.run_slabs, sc);
    return hipGetLastError();
}

hipError_t launch_factored_stats(const DevMatrix* d_mats, int n_mats, int64_t total_tiles, int64_t total_rgroups,
                                 int64_t total_cgroups, float beta2, float omb2, const float* clip, bool partials_ready,
                                 hipStream_t stream) {
    if (n_mats <= 0) return hipSuccess;
    hipError_t e;
    if (!partials_ready) {
        k_rowcol_partial<GRAD_STATS_ONLY><<<(unsigned)total_tiles, 256, 0, stream>>>(d_mats, n_mats, nullptr, nullptr);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    k_rowcol_finalize<<<(unsigned)(total_rgroups + total_cgroups), 256, 0, stream>>>(d_mats, n_mats, total_rgroups,
                                                                                     beta2, omb2, clip);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_rowcol_mean<<<n_mats, 256, 0, stream>>>(d_mats);
    return hipGetLastError();
}

template <int MODE>
static void launch_grad_mode(bool last, int64_t groups, int run_slabs, const DevTensor* d_tab,
                             const int64_t* d_chunk_begin, int n_tensors, int64_t total_chunks,
                             const uint16_t* micro, double* sq_part, hipStream_t stream) {
    if (last)
        k_grad_chunks<MODE, true><<<(unsigned)groups, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors, total_chunks,
                                                                        run_slabs, micro, sq_part);
    else
        k_grad_chunks<MODE, false><<<(unsigned)groups, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors,
                                                                         total_chunks, run_slabs, micro, sq_part);
}

// One group per run, as the steps launch; against 2,048 groups looping over
// runs of 8 slabs (alternating processes, one box): GPT-2.7B accumulation
// 3.145 -> 3.022 ms, Qwen3-0.6B 0.747 -> 0.743 ms.  The many partial sums
// are totalled in two fixed-order stages (a single 256-thread group over
// 161K slots had cost 0.16 ms).
AccLaunch acc_launch(int64_t total_chunks) {
    const int64_t slabs = (total_chunks + kWavesPerGroup - 1) / kWavesPerGroup;
    if (slabs <= 0) return {0, 1};
    int r = 4;
    while (r > 1 && slabs / r < 2048) r >>= 1;
    const int64_t runs = (slabs + r - 1) / r;
    return {runs < kMaxRunGroups ? runs : kMaxRunGroups, r};
}

hipError_t launch_grad_pass(int mode, bool last, bool tiles_for_matrices, const DevTensor* d_tab,
                            const int64_t* d_chunk_begin, int n_tensors, int64_t total_chunks, const DevMatrix* d_mats,
                            int n_mats, int64_t total_tiles, const DevTensor* d_tab1, const int64_t* d_chunks1,
                            int n_tensors1, int64_t total_chunks1, const uint16_t* micro, double* sq_part, double* sq,
                            hipStream_t stream) {
    const bool tiles = last && tiles_for_matrices && n_mats > 0;
    if (tiles) {
        // the chunk pass covers the other tensors only
        d_tab = d_tab1;
        d_chunk_begin = d_chunks1;
        n_tensors = n_tensors1;
        total_chunks = total_chunks1;
    }
    int64_t groups = 0;
    if (total_chunks > 0) {
        const AccLaunch L = acc_launch(total_chunks);
        groups = L.groups;
        const int r = L.run_slabs;
        if (mode == GRAD_STATS_ONLY)
            launch_grad_mode<GRAD_STATS_ONLY>(last, groups, r, d_tab, d_chunk_begin, n_tensors, total_chunks, micro,
                                              sq_part, stream);
        else if (mode == GRAD_FIRST)
            launch_grad_mode<GRAD_FIRST>(last, groups, r, d_tab, d_chunk_begin, n_tensors, total_chunks, micro,
                                         sq_part, stream);
        else
            launch_grad_mode<GRAD_ADD>(last, groups, r, d_tab, d_chunk_begin, n_tensors, total_chunks, micro,
                                       sq_part, stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (tiles) {
        double* tile_sq = sq_part + groups;
        if (mode == GRAD_STATS_ONLY)
            k_rowcol_partial<GRAD_STATS_ONLY><<<(unsigned)total_tiles, 256, 0, stream>>>(d_mats, n_mats, micro,
                                                                                          tile_sq);
        else if (mode == GRAD_FIRST)
            k_rowcol_partial<GRAD_FIRST><<<(unsigned)total_tiles, 256, 0, stream>>>(d_mats, n_mats, micro, tile_sq);
        else
            k_rowcol_partial<GRAD_ADD><<<(unsigned)total_tiles, 256, 0, stream>>>(d_mats, n_mats, micro, tile_sq);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (last) {
        // slots 0 .. groups-1 from the chunk pass, then one per tile; the
        // first stage of the total writes the kSqStageGroups slots after them
        const int64_t nslots = groups + (tiles ? total_tiles : 0);
        double* stage = sq_part + nslots;
        k_sq_stage<<<kSqStageGroups, 256, 0, stream>>>(sq_part, nslots, stage);
        k_sq_total<<<1, 256, 0, stream>>>(stage, kSqStageGroups, sq);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_clip_factor(const double* sq, float max_norm, float* clip, hipStream_t stream) {
    k_clip_factor<<<1, 64, 0, stream>>>(sq, max_norm, clip);
    return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, uint8_t value, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    size_t nvec = bytes / 16;
    size_t groups = (nvec + 255) / 256;
    if (groups < 1) groups = 1;
    if (groups > 4096) groups = 4096;
    k_fill<<<(unsigned)groups, 256, 0, stream>>>((uint8_t*)p, bytes, value);
    return hipGetLastError();
}

hipError_t launch_block8_step(const StepScalars& sc, const DevTensor* d_tab, const int64_t* d_chunk_begin,
                              int n_tensors, int64_t total_chunks, hipStream_t stream) {
    if (total_chunks <= 0) return hipSuccess;
    k_zero_queue<<<1, 64, 0, stream>>>(queue_of_table(d_tab));
    if (sc.flags & SF_CLIP) {
        static std::atomic<int> occ{0};
        const RunLaunch L = queue_launch(k_step8<true>, total_chunks, occ, kRunSlabs8);
        k_step8<true><<<L.grid, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors, total_chunks, L.run_slabs, sc);
    } else {
        static std::atomic<int> occ{0};
        const RunLaunch L = queue_launch(k_step8<false>, total_chunks, occ, kRunSlabs8);
        k_step8<false><<<L.grid, 256, 0, stream>>>(d_tab, d_chunk_begin, n_tensors, total_chunks, L.run_slabs, sc);
    }
    return hipGetLastError();
}

// Workspace of q4adamw_step_noalloc, for callers that cannot allocate: a
// static device array, one per device the library runs on, held until the
// process ends.  Every such call on a device shares it, so calls that
// overlap on one device race.  Host code never passes the array's name to a
// kernel or a copy (on the host it only stands for the symbol): it takes
// the device address that hipGetSymbolAddress gives, once per device with
// that device current.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_address(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::mutex mu;
    static void* addr[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_dequant(int mcb, int vcb, const DevTensor& t, int64_t rows, float* m_out, float* v_out,
                          double* ws_partials, float* ws_inv, hipStream_t stream) {
    if (t.numel == 0) return hipSuccess;
    if (t.kind == KIND_BYTE8) {
        k_dequant8<<<(unsigned)((t.numel + 255) / 256), 256, 0, stream>>>(t, m_out, v_out);
        return hipGetLastError();
    }
    if (t.kind == KIND_FACTORED) {
        const int64_t ng = (rows + kGroup - 1) / kGroup;
        k_rsum_groups<<<(unsigned)ng, 256, 0, stream>>>(t.v_row, rows, ws_partials);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        k_rsum_final<<<1, 256, 0, stream>>>(ws_partials, ng, rows, ws_inv);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned grid = (unsigned)((t.numel + 255) / 256);
#define Q4_DQ(A, B)                                                                       \
    if (mcb == A && vcb == B) {                                                           \
        k_dequant<A, B><<<grid, 256, 0, stream>>>(t, m_out, v_out, ws_inv);               \
        return hipGetLastError();                                                         \
    }
    Q4_DQ(Q4_CB_NF4, Q4_CB_DYN4) Q4_DQ(Q4_CB_NF4, Q4_CB_DYN4_NZ) Q4_DQ(Q4_CB_NF4, Q4_CB_LIN4_NZ)
    Q4_DQ(Q4_CB_SDYN4, Q4_CB_DYN4) Q4_DQ(Q4_CB_SDYN4, Q4_CB_DYN4_NZ) Q4_DQ(Q4_CB_SDYN4, Q4_CB_LIN4_NZ)
#undef Q4_DQ
    return hipErrorInvalidValue;
}

}  // namespace q4
