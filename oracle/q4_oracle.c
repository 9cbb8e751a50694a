/*
 * q4_oracle.c -- plain, slow, single-threaded CPU oracle of the fused 4-bit
 * AdamW optimizer step (ZIP-SR, ZE-EDEN, factored, and quantization off).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file.  The GPU library
 * never includes, links or calls it, and it shares no header, table or
 * helper with the GPU library: every table below is constructed here from
 * its definition, at run time.
 *
 * Sources (cited by page title and section; the pages are web pages about
 * one method):
 *   [P]  "Rounding in Preconditioner Space: Redesigning 4-bit AdamW
 *        Optimizer-State Quantization" (paper listing page): abstract,
 *        Table 1 (rounding rules near zero), Table 2 (recipes), Table 10/11,
 *        Figure 7 (the 90% switch of the LM-head first moment).
 *   [A]  AReno docs, "4-bit AdamW": section "State representation"
 *        (128-element parameter-local blocks, factored second moment for
 *        matrices viewed as [shape[0], -1], zero-excluding map for vectors,
 *        bounded block-local FP32 work).
 *   [N]  news article on the two 4-bit AdamW methods (globaltechnewsdesk):
 *        the AdamW description paragraph and the storage paragraph
 *        (1.0625 B/param vs 8 B for two FP32 buffers).
 *
 * Arithmetic: every step is IEEE binary32 with round-to-nearest-even, in
 * the order written, because [A] "State representation" fixes the update to
 * block-local FP32 work.  The compiler contracts nothing (build with
 * -ffp-contract=off); where a sum of products is one fused multiply-add,
 * the code calls fmaf: the two moment recurrences, the denominator and the
 * weight update (the pages fix FP32 work, not the rounding of each product
 * within it).  Exceptions, each stated where it happens: the
 * bias-correction scalars (binary64, then rounded), the codebook
 * constructions (binary64, then rounded) and the factored row/column sums
 * (binary64 accumulation).
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes of the repository as well):
 *   - NF4 levels: the published QLoRA NormalFloat construction.
 *   - Dyn4 / Dyn4-NZ / SDyn4 levels: dynamic-tree (base-10 dynamic exponent)
 *     construction; parity unpinned against the authors' own tables, which
 *     the pages do not print.
 *   - AdamW: torch-style bias correction, decoupled multiplicative decay; the
 *     update uses the unquantized m1, v1 (quantization only affects the next
 *     step; [P] Table 11 speaks of the working first moment before storage).
 *   - Preconditioner coordinate r(v) = 1/(sqrt(v) + eps_sr), v the stored
 *     (not bias-corrected) second moment.
 *   - EDEN: per block S = <x,x>/<x,Q(x)> in normalized v space, no rotation,
 *     folded into the stored scale.
 *   - RTN ties go to the lower code; SR draws from Philox4x32-10 keyed on
 *     (seed, step, tensor id, stream, element index).
 *   - Non-finite moments (NaN or infinite gradients): the IEEE operations
 *     written here decide.  Block maxima take a value only when it compares
 *     greater (NaN skipped, +inf kept); an infinite scale has the inverse
 *     1/inf = 0; normalized values are clamped by comparison, which a NaN
 *     fails, and a NaN then lies above no midpoint and no level, so it takes
 *     sorted index 0 under every rule; EDEN's ratio over a block holding one
 *     is 1 (its sums are NaN); the weight follows IEEE arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define OR_BLOCK 128

/* codebook ids */
enum { OR_CB_NF4 = 0, OR_CB_SDYN4 = 1, OR_CB_DYN4 = 2, OR_CB_DYN4_NZ = 3, OR_CB_LIN4_NZ = 4, OR_CB_COUNT = 5 };
/* rounding rules, in the names of [P] Table 1 */
enum { OR_STATE_RTN = 0, OR_STATE_SR = 1, OR_UPDATE_RTN = 2, OR_UPDATE_SR = 3 };
/* recipes, [P] Table 2, plus the factored mode of [A] and FP32 AdamW */
enum { OR_ZIP_SR = 0, OR_ZE_EDEN = 1, OR_FACTORED = 2, OR_FP32 = 3, OR_CUSTOM = 4 };
/* tensor flags */
#define OR_TF_LM_HEAD 1u

/* ------------------------------------------------------------------------ */
/* Codebooks                                                                 */
/* ------------------------------------------------------------------------ */

/* Standard normal CDF from the complementary error function (binary64). */
static double or_norm_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Inverse standard normal CDF by bisection: slow, but plainly correct to
 * the last bit of binary64 that the CDF itself resolves. */
static double or_norm_ppf(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 400; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (or_norm_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/* NF4 ("4-bit NormalFloat", [P] abstract and Table 2): 8 positive quantiles
 * Phi^-1(1/2 + j (d - 1/2)/8), j = 1..8, 7 negative quantiles
 * -Phi^-1(1/2 + j (d - 1/2)/7), j = 1..7, and an exact zero, all divided by
 * Phi^-1(d), with d = 1 - (1/30 + 1/32)/2.  Sorted ascending; code = index. */
static void or_build_nf4(float out[16]) {
    const double d = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
    const double top = or_norm_ppf(d);
    double v[16];
    int k = 0;
    for (int j = 7; j >= 1; --j) v[k++] = -or_norm_ppf(0.5 + j * (d - 0.5) / 7.0);
    v[k++] = 0.0;
    for (int j = 1; j <= 8; ++j) v[k++] = or_norm_ppf(0.5 + j * (d - 0.5) / 8.0);
    for (int i = 0; i < 16; ++i) out[i] = (float)(v[i] / top);
}

/* Unsigned dynamic-exponent map of `bits` bits (base 10): the number E of
 * leading zero bits selects the decade 10^-E, the next bit is an indicator,
 * the remaining F bits f pick a linear fraction 0.1 + 0.9 (f+1)/2^F.  The
 * all-zero code is 0 (zero-inclusive) or 10^-bits (zero-excluding). */
static double or_dyn_magnitude(int code, int bits, int zero_excluding) {
    if (code == 0) return zero_excluding ? pow(10.0, -(double)bits) : 0.0;
    int E = 0;
    while (!(code & (1 << (bits - 1 - E)))) ++E;
    int F = bits - 1 - E;
    int f = code & ((1 << F) - 1);
    return pow(10.0, -(double)E) * (0.1 + 0.9 * (double)(f + 1) / (double)(1 << F));
}

/* Code-indexed decode table of codebook `cb`. */
void or_codebook(int cb, float out[16]) {
    switch (cb) {
    case OR_CB_NF4: or_build_nf4(out); return;
    case OR_CB_DYN4:
        for (int c = 0; c < 16; ++c) out[c] = (float)or_dyn_magnitude(c, 4, 0);
        return;
    case OR_CB_DYN4_NZ:
        for (int c = 0; c < 16; ++c) out[c] = (float)or_dyn_magnitude(c, 4, 1);
        return;
    case OR_CB_SDYN4: /* sign bit (bit 3) + 3-bit dynamic magnitude */
        for (int c = 0; c < 16; ++c) {
            float mag = (float)or_dyn_magnitude(c & 7, 3, 0);
            out[c] = (c & 8) ? -mag : mag;
        }
        out[8] = 0.0f; /* the code "-0" decodes to +0 and is never emitted */
        return;
    case OR_CB_LIN4_NZ:
        for (int c = 0; c < 16; ++c) out[c] = (float)(c + 1) / 16.0f;
        return;
    default:
        for (int c = 0; c < 16; ++c) out[c] = 0.0f;
    }
}

/* Sorted distinct levels of a codebook and the code of each one.  Returns
 * the number of levels (16, or 15 for SDyn4 which has one zero). */
typedef struct { int n; float L[16]; int code[16]; float mid[15]; } or_levels;

static void or_make_levels(int cb, or_levels* lv) {
    float dec[16];
    or_codebook(cb, dec);
    int n = 0;
    for (int c = 0; c < 16; ++c) {
        if (cb == OR_CB_SDYN4 && c == 8) continue;
        lv->L[n] = dec[c]; lv->code[n] = c; ++n;
    }
    /* insertion sort by value (tiny) */
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && lv->L[j - 1] > lv->L[j]; --j) {
            float t = lv->L[j]; lv->L[j] = lv->L[j - 1]; lv->L[j - 1] = t;
            int tc = lv->code[j]; lv->code[j] = lv->code[j - 1]; lv->code[j - 1] = tc;
        }
    lv->n = n;
    /* FP32 midpoints between adjacent levels */
    for (int k = 0; k + 1 < n; ++k) lv->mid[k] = (lv->L[k] + lv->L[k + 1]) * 0.5f;
}

/* Export of the sorted levels and midpoints (for tests). */
int or_sorted_levels(int cb, float L[16], int code[16], float mid[15]) {
    or_levels lv;
    or_make_levels(cb, &lv);
    memcpy(L, lv.L, sizeof(lv.L));
    memcpy(code, lv.code, sizeof(lv.code));
    memcpy(mid, lv.mid, sizeof(lv.mid));
    return lv.n;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As  */
/* Easy as 1, 2, 3", SC'11).                                                 */
/* ------------------------------------------------------------------------ */

void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform of element i of a tensor: counter (i/4, step, tensor id,
 * stream), key (seed low word, seed high word), word i mod 4; the top 24
 * bits scaled by 2^-24 give an exact float in [0, 1 - 2^-24]. */
float or_uniform(uint64_t seed, uint64_t step, uint32_t tensor_id, uint32_t stream, uint64_t i) {
    uint32_t ctr[4] = { (uint32_t)(i >> 2), (uint32_t)step, tensor_id, stream };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t w[4];
    or_philox4x32_10(ctr, key, w);
    return (float)(w[i & 3] >> 8) * (1.0f / 16777216.0f);
}

/* ------------------------------------------------------------------------ */
/* Host scalars of one step                                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    float lr, beta1, beta2, eps, weight_decay, eps_sr;
    uint64_t step, seed;
    uint32_t lm_head_sr;
    float grad_scale; /* clip factor applied to every gradient element (1: no clipping) */
} or_hparams;

typedef struct { float decay, step_size, rsbc2, omb1, omb2; } or_scalars;

/* AdamW with bias correction and decoupled decay ([N] AdamW paragraph; the
 * bias correction itself is a reading): decay = 1 - lr wd; step size
 * lr / (1 - b1^t); the second-moment correction enters as 1/sqrt(1 - b2^t). */
void or_host_scalars(const or_hparams* hp, float out[5]) {
    double t = (double)hp->step;
    double bc1 = 1.0 - pow((double)hp->beta1, t);
    double bc2 = 1.0 - pow((double)hp->beta2, t);
    out[0] = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
    out[1] = (float)((double)hp->lr / bc1);
    out[2] = (float)(1.0 / sqrt(bc2));
    out[3] = 1.0f - hp->beta1;
    out[4] = 1.0f - hp->beta2;
}

/* ------------------------------------------------------------------------ */
/* Rounding rules on one cell ([P] Table 1)                                  */
/* ------------------------------------------------------------------------ */
/* The cell is [L_lo, L_hi] in normalized units, [a_lo, a_hi] = s [L_lo, L_hi]
 * in state units; x is the normalized value, v = the state value (used by
 * the preconditioner-space rules through sv = sqrt(v)).  Each rule returns
 * 1 to round up to L_hi, 0 to round down.  u is the uniform of the element.
 *
 * r(a) = 1 / (sqrt(a) + eps).  Preconditioner-space SR rounds up with
 * P = (r(a_lo) - r(v)) / (r(a_lo) - r(a_hi)), which makes E[r(Q)] = r(v);
 * multiplied out it is (sv - sqrt(a_lo)) (sqrt(a_hi) + eps) over
 * (sqrt(a_hi) - sqrt(a_lo)) (sv + eps), which does not cancel near a_lo = 0. */

int or_cell_round(int rule, float x, float L_lo, float L_hi, float s, float sv, float eps_sr, float u) {
    switch (rule) {
    case OR_STATE_RTN: {
        float mid = (L_lo + L_hi) * 0.5f;
        return x > mid;
    }
    case OR_STATE_SR:
        return u * (L_hi - L_lo) < (x - L_lo);
    case OR_UPDATE_RTN: {
        float rlo = sqrtf(L_lo * s), rhi = sqrtf(L_hi * s);
        /* nearer to the upper level in r:  r(v) - r(a_hi) < r(a_lo) - r(v) */
        float left = (rhi - sv) * (rlo + eps_sr);
        float right = (sv - rlo) * (rhi + eps_sr);
        return left < right;
    }
    case OR_UPDATE_SR: {
        float rlo = sqrtf(L_lo * s), rhi = sqrtf(L_hi * s);
        float num = (sv - rlo) * (rhi + eps_sr);
        float den = (rhi - rlo) * (sv + eps_sr);
        return u * den < num;
    }
    }
    return 0;
}

/* Probability of rounding up (binary64, for the analysis of [P] Table 1). */
double or_cell_prob_up(int rule, double a_lo, double a_hi, double v, double eps) {
    switch (rule) {
    case OR_STATE_RTN: return v > 0.5 * (a_lo + a_hi) ? 1.0 : 0.0;
    case OR_STATE_SR: return (v - a_lo) / (a_hi - a_lo);
    case OR_UPDATE_RTN: {
        double r = 1.0 / (sqrt(v) + eps), rlo = 1.0 / (sqrt(a_lo) + eps), rhi = 1.0 / (sqrt(a_hi) + eps);
        return (r - rhi) < (rlo - r) ? 1.0 : 0.0;
    }
    case OR_UPDATE_SR: {
        double r = 1.0 / (sqrt(v) + eps), rlo = 1.0 / (sqrt(a_lo) + eps), rhi = 1.0 / (sqrt(a_hi) + eps);
        return (rlo - r) / (rlo - rhi);
    }
    }
    return 0.0;
}

/* ------------------------------------------------------------------------ */
/* Block quantizers                                                          */
/* ------------------------------------------------------------------------ */

/* Round-to-nearest code: the number of FP32 midpoints strictly below x (an
 * exact midpoint goes to the lower level). Returns a sorted index. */
static int or_rtn_index(const or_levels* lv, float x) {
    int k = 0;
    for (int j = 0; j + 1 < lv->n; ++j) if (x > lv->mid[j]) ++k;
    return k;
}

/* Bracket of x: the largest sorted index whose level is <= x (0 when x
 * lies below the smallest level, which only a zero-excluding map allows). */
static int or_lower_index(const or_levels* lv, float x) {
    int lo = 0;
    for (int j = 0; j < lv->n; ++j) if (lv->L[j] <= x) lo = j;
    return lo;
}

/* Choose the sorted index of one normalized value x under `rule`. */
static int or_choose(const or_levels* lv, int rule, float x, float s, float sv, float eps_sr, float u) {
    if (rule == OR_STATE_RTN) return or_rtn_index(lv, x);
    int lo = or_lower_index(lv, x);
    if (lv->L[lo] == x || lo == lv->n - 1 || x < lv->L[0]) return lo;
    return lo + or_cell_round(rule, x, lv->L[lo], lv->L[lo + 1], s, sv, eps_sr, u);
}

static void or_put_nibble(uint8_t* codes, int64_t j, int code) {
    if (j & 1) codes[j >> 1] = (uint8_t)((codes[j >> 1] & 0x0F) | (code << 4));
    else codes[j >> 1] = (uint8_t)((codes[j >> 1] & 0xF0) | code);
}
static int or_get_nibble(const uint8_t* codes, int64_t j) {
    return (j & 1) ? (codes[j >> 1] >> 4) : (codes[j >> 1] & 0x0F);
}

/* Pairwise (tree) sum over the 128 slots of a block in index order, with
 * absent tail slots = +0.  Written as recursion so the order is plain. */
static float or_pairwise(const float* x, int n) {
    if (n == 1) return x[0];
    int h = n / 2;
    return or_pairwise(x, h) + or_pairwise(x + h, n - h);
}

/* Inverse of a block scale for normalization, x = value * (1/s), with 1/s
 * the IEEE quotient ([A] "State representation": absmax-normalized blocks).
 * A zero block normalizes to x = 0 (reading of zero blocks).  A positive
 * scale whose reciprocal overflows to +inf (s <= 2^-128, a subnormal) has
 * no usable normalization: value * inf is infinite, and NaN for a zero
 * value, which no level represents.  Such a block is normalized like a zero
 * block (reading of overflowing inverses), so every slot stores the code of
 * zero; the scale itself is stored as computed.  A subnormal scale whose
 * reciprocal is finite normalizes as any other. */
static float or_scale_inverse(float s) {
    if (!(s > 0.0f)) return 0.0f;
    const float inv = 1.0f / s;
    return isinf(inv) ? 0.0f : inv;
}

/* Clamps of a normalized value to the range of the levels, [-1, 1] for a
 * signed map and at most 1 for an unsigned one: x = value * (1/s) can pass
 * the end of the range by a rounding.  Written as comparisons, which a NaN
 * fails, so a NaN (a NaN moment, or an infinite one normalized by 1/inf =
 * 0) passes through and takes sorted index 0 in the quantizers (reading of
 * non-finite moments). */
static float or_clamp_signed(float x) {
    if (x > 1.0f) x = 1.0f;
    if (x < -1.0f) x = -1.0f;
    return x;
}
static float or_clamp_unsigned(float x) {
    if (x > 1.0f) x = 1.0f;
    return x;
}

/* First moment of one block: absmax scale, normalization, then RTN or
 * state-space SR (the LM-head rule of [P] Table 2) over the signed map.
 * m1[0..n) are the unquantized values; writes n nibbles starting at
 * nibble index j0 of `codes` and returns the new scale. */
static float or_requant_m_levels(const or_levels* lvp, int rule, const float* m1, int n, uint64_t seed,
                                uint64_t step, uint32_t tensor_id, uint64_t elem0, uint8_t* codes, int64_t j0) {
    const or_levels lv = *lvp;
    float s = 0.0f;
    for (int k = 0; k < n; ++k) { float a = fabsf(m1[k]); if (a > s) s = a; }
    float inv = or_scale_inverse(s);
    for (int k = 0; k < n; ++k) {
        float x = or_clamp_signed(m1[k] * inv);
        float u = rule == OR_STATE_SR ? or_uniform(seed, step, tensor_id, 0, elem0 + (uint64_t)k) : 0.0f;
        int idx = or_choose(&lv, rule, x, s, 0.0f, 0.0f, u);
        or_put_nibble(codes, j0 + k, lv.code[idx]);
    }
    return s;
}

/* Second moment of one block: max scale, normalization, the v rule (State
 * or Update, RTN or SR, [P] Table 1), then optionally the EDEN rescale of
 * the quantized block ([P] abstract, ZE-EDEN), folded into the scale. */
static float or_requant_v_levels(const or_levels* lvp, int rule, int eden, const float* v1, int n, float eps_sr,
                                uint64_t seed, uint64_t step, uint32_t tensor_id, uint64_t elem0, uint8_t* codes,
                                int64_t j0) {
    const or_levels lv = *lvp;
    float s = 0.0f;
    for (int k = 0; k < n; ++k) if (v1[k] > s) s = v1[k];
    float inv = or_scale_inverse(s);
    float xx[OR_BLOCK], xq[OR_BLOCK];
    for (int k = 0; k < OR_BLOCK; ++k) { xx[k] = 0.0f; xq[k] = 0.0f; }
    for (int k = 0; k < n; ++k) {
        float x = or_clamp_unsigned(v1[k] * inv);
        float sv = sqrtf(v1[k]);
        int needs_u = rule == OR_STATE_SR || rule == OR_UPDATE_SR;
        float u = needs_u ? or_uniform(seed, step, tensor_id, 1, elem0 + (uint64_t)k) : 0.0f;
        int idx = or_choose(&lv, rule, x, s, sv, eps_sr, u);
        or_put_nibble(codes, j0 + k, lv.code[idx]);
        xx[k] = x * x;
        xq[k] = x * lv.L[idx];
    }
    if (!eden) return s;
    float sxx = or_pairwise(xx, OR_BLOCK);
    float sxq = or_pairwise(xq, OR_BLOCK);
    float S = sxq > 0.0f ? sxx / sxq : 1.0f;
    return s * S;
}

/* Block quantizers with the codebook named by id (the tables are built on
 * each call; the step builds them once per window). */
float or_requant_m_block(int cb, int rule, const float* m1, int n, uint64_t seed, uint64_t step,
                         uint32_t tensor_id, uint64_t elem0, uint8_t* codes, int64_t j0) {
    or_levels lv;
    or_make_levels(cb, &lv);
    return or_requant_m_levels(&lv, rule, m1, n, seed, step, tensor_id, elem0, codes, j0);
}

float or_requant_v_block(int cb, int rule, int eden, const float* v1, int n, float eps_sr, uint64_t seed,
                         uint64_t step, uint32_t tensor_id, uint64_t elem0, uint8_t* codes, int64_t j0) {
    or_levels lv;
    or_make_levels(cb, &lv);
    return or_requant_v_levels(&lv, rule, eden, v1, n, eps_sr, seed, step, tensor_id, elem0, codes, j0);
}

/* ------------------------------------------------------------------------ */
/* Factored second moment ([A] "State representation")                      */
/* ------------------------------------------------------------------------ */
/* Matrix viewed as [rows, cols] = [shape[0], numel/shape[0]].  Row and
 * column sums of g^2 accumulate in binary64 and are rounded to float; the
 * row and column means then enter their own exponential averages; mean(R)
 * is a binary64 sum over rows divided by rows.  Writes 1/mean(R) (0 when
 * mean(R) is 0) to *inv_meanR. */
static float or_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* With gradient clipping (grad_scale s != 1) the statistics are those of the
 * clipped gradient, formed as s^2 times the binary64 sums of the squares of
 * the unclipped BF16 gradient (s^2 exact in binary64), so that they can be
 * gathered before s is known. */
void or_factored_update(const or_hparams* hp, int64_t rows, int64_t cols, const uint16_t* grad,
                        float* R, float* C, float* inv_meanR) {
    float sc[5];
    or_host_scalars(hp, sc);
    float omb2 = sc[4];
    const double s2 = (double)hp->grad_scale * (double)hp->grad_scale;
    double* cs = (double*)calloc((size_t)cols, sizeof(double));
    for (int64_t r = 0; r < rows; ++r) {
        double rs = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            float g = or_bf16_to_f32(grad[r * cols + c]);
            float g2 = g * g;
            rs += (double)g2;
            cs[c] += (double)g2;
        }
        R[r] = hp->beta2 * R[r] + omb2 * ((float)(rs * s2) / (float)cols);
    }
    for (int64_t c = 0; c < cols; ++c) C[c] = hp->beta2 * C[c] + omb2 * ((float)(cs[c] * s2) / (float)rows);
    free(cs);
    double sum = 0.0;
    for (int64_t r = 0; r < rows; ++r) sum += (double)R[r];
    float meanR = (float)(sum / (double)rows);
    *inv_meanR = meanR > 0.0f ? 1.0f / meanR : 0.0f;
}

/* ------------------------------------------------------------------------ */
/* The step before: BF16 gradient accumulation, norm and clip factor        */
/* ------------------------------------------------------------------------ */
/* [A] "State representation": microbatches stream into BF16 gradient
 * shards (no FP32 main gradient), and the gradient norm and clipping work
 * on those BF16 shards. */

/* FP32 -> BF16, round to nearest, ties to even (NaN kept quiet). */
static uint16_t or_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* acc <- micro on the first microbatch; otherwise acc <- bf16(f32(acc) +
 * f32(micro)): one FP32 addition (exact for most BF16 pairs), then one
 * rounding to BF16. */
void or_accumulate_bf16(uint16_t* acc, const uint16_t* micro, int64_t n, int first) {
    for (int64_t i = 0; i < n; ++i) {
        if (first) acc[i] = micro[i];
        else acc[i] = or_f32_to_bf16(or_bf16_to_f32(acc[i]) + or_bf16_to_f32(micro[i]));
    }
}

/* Sum of squares of a BF16 gradient: each square formed in FP32 (exact for
 * BF16 inputs short of overflow and underflow), summed in binary64 in index
 * order.  The global squared norm is the binary64 sum of these over the
 * tensors in order; the pages fix no summation order, so another order
 * gives the same value up to binary64 rounding. */
double or_grad_sumsq(const uint16_t* g, int64_t n) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        float x = or_bf16_to_f32(g[i]);
        s += (double)(x * x);
    }
    return s;
}

/* Clip factor from the global squared norm, as torch.nn.utils.clip_grad_norm_
 * forms it: min(1, max_norm / (sqrt(sq) + 1e-6)) in binary64, rounded to
 * FP32; 1 when max_norm <= 0 (clipping off). */
float or_clip_factor(double sq, float max_norm) {
    if (!(max_norm > 0.0f)) return 1.0f;
    double c = (double)max_norm / (sqrt(sq) + 1e-6);
    return c < 1.0 ? (float)c : 1.0f;
}

/* ------------------------------------------------------------------------ */
/* The step                                                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t recipe, m_cb, v_cb, m_rule, v_rule, eden;
} or_config;

/* A window [base, base + len) of one tensor of `numel` elements.  Every
 * array holds only the window: element i sits at index i - base (codes:
 * nibble i - base; scales: block (i - base)/128).  base is a multiple of
 * 128.  cols > 0 marks a factored matrix (R and C are full vectors);
 * cols == 0 a packed (or FP32) second moment. */
typedef struct {
    uint32_t tensor_id, flags;
    int64_t numel, cols, base, len;
    float* param;
    const uint16_t* grad;
    uint8_t* m_codes; float* m_scales;
    uint8_t* v_codes; float* v_scales;
    const float* R; const float* C; float inv_meanR;
    float* m32; float* v32;
    /* optional (NULL: not written): the unquantized m1, v1 of the window,
     * which the parity harness reads to audit a differing code */
    float* m1_out; float* v1_out;
} or_window;

/* One AdamW step over a window ([N] AdamW paragraph; [A] "State
 * representation"; [P] Table 2).  For each 128-block: decode m0, v0 from
 * codes and the old scales (or read the FP32 moments), form m1, v1, update
 * the master weight from the unquantized m1, v1, then requantize. */
int or_step_window(const or_config* cfg, const or_hparams* hp, const or_window* w) {
    if (w->base % OR_BLOCK != 0) return -1;
    float sc[5];
    or_host_scalars(hp, sc);
    const float decay = sc[0], step_size = sc[1], rsbc2 = sc[2], omb1 = sc[3], omb2 = sc[4];
    const float b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps;
    const int fp32 = cfg->recipe == OR_FP32;
    const int factored = w->cols > 0;
    float Lm[16], Lv[16];
    or_codebook(cfg->m_cb, Lm);
    or_codebook(cfg->v_cb, Lv);
    or_levels lvm, lvv;
    or_make_levels(cfg->m_cb, &lvm);
    or_make_levels(cfg->v_cb, &lvv);
    int m_rule = cfg->m_rule;
    if ((w->flags & OR_TF_LM_HEAD) && hp->lm_head_sr) m_rule = OR_STATE_SR;

    float m1[OR_BLOCK], v1[OR_BLOCK];
    for (int64_t off = 0; off < w->len; off += OR_BLOCK) {
        int n = (int)((w->len - off) < OR_BLOCK ? (w->len - off) : OR_BLOCK);
        int64_t blk = off / OR_BLOCK;
        for (int k = 0; k < n; ++k) {
            int64_t j = off + k;            /* index within the window */
            int64_t i = w->base + j;        /* index within the tensor */
            /* the clipped gradient: one FP32 product (exact when s = 1) */
            float g = or_bf16_to_f32(w->grad[j]) * hp->grad_scale;
            float m0, v0 = 0.0f;
            if (fp32) {
                m0 = w->m32[j];
                v0 = w->v32[j];
            } else {
                m0 = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[blk];
                if (!factored) v0 = Lv[or_get_nibble(w->v_codes, j)] * w->v_scales[blk];
            }
            /* m1 = b1 m0 + (1 - b1) g, v1 = b2 v0 + (1 - b2) g^2, each as one
             * fused multiply-add onto the rounded gradient term */
            float mm = fmaf(b1, m0, omb1 * g);
            float vv;
            if (factored) {
                int64_t r = i / w->cols, c = i % w->cols;
                vv = (w->R[r] * w->C[c]) * w->inv_meanR;
            } else {
                vv = fmaf(b2, v0, omb2 * (g * g));
            }
            /* w <- w decay - step_size m1 / (sqrt(v1) rsbc2 + eps) */
            float denom = fmaf(sqrtf(vv), rsbc2, eps);
            w->param[j] = fmaf(-step_size, mm / denom, w->param[j] * decay);
            m1[k] = mm;
            v1[k] = vv;
            if (w->m1_out) w->m1_out[j] = mm;
            if (w->v1_out) w->v1_out[j] = vv;
        }
        if (fp32) {
            for (int k = 0; k < n; ++k) { w->m32[off + k] = m1[k]; w->v32[off + k] = v1[k]; }
            continue;
        }
        uint64_t elem0 = (uint64_t)(w->base + off);
        w->m_scales[blk] = or_requant_m_levels(&lvm, m_rule, m1, n, hp->seed, hp->step, w->tensor_id, elem0,
                                               w->m_codes, off);
        if (!factored)
            w->v_scales[blk] = or_requant_v_levels(&lvv, cfg->v_rule, cfg->eden, v1, n, hp->eps_sr, hp->seed,
                                                   hp->step, w->tensor_id, elem0, w->v_codes, off);
    }
    return 0;
}

/* Fresh state: every code decodes to exactly 0 with scale +0 ("moments
 * start at 0"): NF4/SDyn4 use the code of 0, Dyn4 its zero code, Dyn4-NZ
 * and Lin4-NZ the floor code (decoded with scale 0 it is 0). */
int or_zero_code(int cb) {
    float L[16];
    or_codebook(cb, L);
    for (int c = 0; c < 16; ++c) if (L[c] == 0.0f) return c;
    return 0;
}

/* Dequantization of a window: m = L_m[code] s_m; v = L_v[code] s_v or, for
 * a factored matrix, (R_r C_c) / mean(R). */
void or_dequant_window(const or_config* cfg, const or_window* w, float* m_out, float* v_out) {
    float Lm[16], Lv[16];
    or_codebook(cfg->m_cb, Lm);
    or_codebook(cfg->v_cb, Lv);
    for (int64_t j = 0; j < w->len; ++j) {
        int64_t blk = j / OR_BLOCK, i = w->base + j;
        m_out[j] = Lm[or_get_nibble(w->m_codes, j)] * w->m_scales[blk];
        if (w->cols > 0) {
            int64_t r = i / w->cols, c = i % w->cols;
            v_out[j] = (w->R[r] * w->C[c]) * w->inv_meanR;
        } else {
            v_out[j] = Lv[or_get_nibble(w->v_codes, j)] * w->v_scales[blk];
        }
    }
}

/* Storage of the quantized state ([N] storage paragraph): per quantized
 * buffer one nibble per element plus one FP32 scale per 128-block; the
 * factored row and column vectors count as scale metadata. */
void or_state_bytes(int recipe, int64_t numel, int64_t rows, int is_matrix, uint64_t out[3]) {
    uint64_t nb = (uint64_t)((numel + OR_BLOCK - 1) / OR_BLOCK);
    uint64_t codes = (uint64_t)((numel + 1) / 2);
    uint64_t q = 0, meta = 0;
    if (recipe == OR_FP32) { q = 8ull * (uint64_t)numel; }
    else if (recipe == OR_FACTORED && is_matrix) {
        q = codes; meta = 4 * nb + 4ull * (uint64_t)rows + 4ull * (uint64_t)(numel / rows);
    } else { q = 2 * codes; meta = 2 * 4 * nb; }
    out[0] = q; out[1] = meta; out[2] = q + meta;
}

/* ------------------------------------------------------------------------ */
/* 8-bit blockwise AdamW ([A] names an 8-bit blockwise AdamW, without        */
/* factorization, beside the 4-bit optimizer; the two are mutually           */
/* exclusive)                                                                */
/* ------------------------------------------------------------------------ */
/* Readings (the pages give no maps for it): the 8-bit members of the
 * dynamic-exponent family above, one byte per code.
 *   SDyn8 (m): bit 7 the sign, bits 0..6 the 7-bit dynamic magnitude; the
 *              code 0x80 ("-0") decodes to +0 and is never written.
 *   Dyn8  (v): the 8-bit dynamic map, zero-inclusive.
 * 128-element blocks, absmax scales (FP32), round to nearest level (ties to
 * the lower level) in normalized units, the AdamW arithmetic of the 4-bit
 * step.  Codes: byte i holds element i. */
enum { OR_CB8_SDYN8 = 0, OR_CB8_DYN8 = 1 };

void or_codebook8(int cb8, float out[256]) {
    for (int c = 0; c < 256; ++c) {
        if (cb8 == OR_CB8_DYN8) {
            out[c] = (float)or_dyn_magnitude(c, 8, 0);
        } else {
            float mag = (float)or_dyn_magnitude(c & 127, 7, 0);
            out[c] = (c & 128) ? -mag : mag;
        }
    }
    if (cb8 == OR_CB8_SDYN8) out[128] = 0.0f;
}

typedef struct { int n; float L[256]; int code[256]; float mid[255]; } or_levels8;

static void or_make_levels8(int cb8, or_levels8* lv) {
    float dec[256];
    or_codebook8(cb8, dec);
    int n = 0;
    for (int c = 0; c < 256; ++c) {
        if (cb8 == OR_CB8_SDYN8 && c == 128) continue;
        lv->L[n] = dec[c]; lv->code[n] = c; ++n;
    }
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && lv->L[j - 1] > lv->L[j]; --j) {
            float t = lv->L[j]; lv->L[j] = lv->L[j - 1]; lv->L[j - 1] = t;
            int tc = lv->code[j]; lv->code[j] = lv->code[j - 1]; lv->code[j - 1] = tc;
        }
    lv->n = n;
    for (int k = 0; k + 1 < n; ++k) lv->mid[k] = (lv->L[k] + lv->L[k + 1]) * 0.5f;
}

int or_sorted_levels8(int cb8, float L[256], int code[256], float mid[255]) {
    or_levels8 lv;
    or_make_levels8(cb8, &lv);
    memcpy(L, lv.L, sizeof(lv.L));
    memcpy(code, lv.code, sizeof(lv.code));
    memcpy(mid, lv.mid, sizeof(lv.mid));
    return lv.n;
}

/* Nearest level: the number of midpoints strictly below x (a midpoint goes
 * to the lower level), found by scanning. */
static int or_rtn8(const or_levels8* lv, float x) {
    int idx = 0;
    while (idx + 1 < lv->n && lv->mid[idx] < x) ++idx;
    return lv->code[idx];
}

/* One step over a window of an 8-bit tensor (same window conventions as
 * or_window; m_codes / v_codes hold one byte per element). */
int or_step8_window(const or_hparams* hp, const or_window* w) {
    if (w->base % OR_BLOCK != 0) return -1;
    float sc[5];
    or_host_scalars(hp, sc);
    const float decay = sc[0], step_size = sc[1], rsbc2 = sc[2], omb1 = sc[3], omb2 = sc[4];
    float Lm[256], Lv[256];
    or_codebook8(OR_CB8_SDYN8, Lm);
    or_codebook8(OR_CB8_DYN8, Lv);
    or_levels8 lvm, lvv;
    or_make_levels8(OR_CB8_SDYN8, &lvm);
    or_make_levels8(OR_CB8_DYN8, &lvv);
    float m1[OR_BLOCK], v1[OR_BLOCK];
    for (int64_t off = 0; off < w->len; off += OR_BLOCK) {
        int n = (int)((w->len - off) < OR_BLOCK ? (w->len - off) : OR_BLOCK);
        int64_t blk = off / OR_BLOCK;
        for (int k = 0; k < n; ++k) {
            int64_t j = off + k;
            float g = or_bf16_to_f32(w->grad[j]) * hp->grad_scale;
            float m0 = Lm[w->m_codes[j]] * w->m_scales[blk];
            float v0 = Lv[w->v_codes[j]] * w->v_scales[blk];
            float mm = fmaf(hp->beta1, m0, omb1 * g);
            float vv = fmaf(hp->beta2, v0, omb2 * (g * g));
            float denom = fmaf(sqrtf(vv), rsbc2, hp->eps);
            w->param[j] = fmaf(-step_size, mm / denom, w->param[j] * decay);
            m1[k] = mm;
            v1[k] = vv;
        }
        float sm = 0.0f, sv = 0.0f;
        for (int k = 0; k < n; ++k) {
            float a = fabsf(m1[k]);
            if (a > sm) sm = a;
            if (v1[k] > sv) sv = v1[k];
        }
        float im = or_scale_inverse(sm), iv = or_scale_inverse(sv);
        for (int k = 0; k < n; ++k) {
            float xm = or_clamp_signed(m1[k] * im);
            float xv = or_clamp_unsigned(v1[k] * iv);
            w->m_codes[off + k] = (uint8_t)or_rtn8(&lvm, xm);
            w->v_codes[off + k] = (uint8_t)or_rtn8(&lvv, xv);
        }
        w->m_scales[blk] = sm;
        w->v_scales[blk] = sv;
    }
    return 0;
}

void or_dequant8_window(const or_window* w, float* m_out, float* v_out) {
    float Lm[256], Lv[256];
    or_codebook8(OR_CB8_SDYN8, Lm);
    or_codebook8(OR_CB8_DYN8, Lv);
    for (int64_t j = 0; j < w->len; ++j) {
        m_out[j] = Lm[w->m_codes[j]] * w->m_scales[j / OR_BLOCK];
        v_out[j] = Lv[w->v_codes[j]] * w->v_scales[j / OR_BLOCK];
    }
}
