/*
 * q4adamw.h -- C ABI of the fused 4-bit AdamW optimizer step on MI355X
 * (CDNA4, gfx950).
 *
 * The step follows the pages about 4-bit AdamW optimizer-state quantization:
 *   [P] "Rounding in Preconditioner Space: Redesigning 4-bit AdamW
 *       Optimizer-State Quantization" (paper listing): abstract, Table 1
 *       (rounding rules), Table 2 (recipes ZIP-SR and ZE-EDEN, the LM-head
 *       first-moment switch in the final 10% of training).
 *   [A] AReno docs, "4-bit AdamW": "State representation" (128-element
 *       parameter-local blocks, Adafactor-style factored second moment for
 *       matrices viewed as [shape[0], -1], zero-excluding packed v for 1-D
 *       tensors, no parameter-sized FP32 moment), "Requirements and errors"
 *       (invalid combinations fail before training starts, only the GPU
 *       backend is accepted, 4-bit state resumes only into the 4-bit
 *       optimizer, state bytes reported as quantized / scale metadata /
 *       total).
 *   [N] news article on the two 4-bit AdamW methods: the AdamW description
 *       and the storage figure (1.0625 B/param for packed values plus block
 *       scales, 8 B for two FP32 buffers).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" point to memory on the current HIP device;
 *     "host" pointers to ordinary host memory.  Every device pointer must be
 *     16-byte aligned (Q4_ERR_ALIGNMENT otherwise).
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates no device memory in these calls and keeps no state between
 *     calls.
 *   - Calls validate synchronously.  On any error nothing is enqueued and no
 *     buffer is touched; the status says why and q4adamw_last_error() holds
 *     a message.  Q4_OK means "enqueued on `stream`"; the work is
 *     asynchronous, and a fault inside a kernel surfaces at the caller's
 *     next synchronization.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Buffers of one call must not overlap, except as stated.
 */
#ifndef Q4ADAMW_H
#define Q4ADAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4ADAMW_ABI_VERSION 3u
#define Q4ADAMW_LAYOUT_VERSION 1u
#define Q4ADAMW_BLOCK 128
#define Q4ADAMW_MAX_NDIM 8
#define Q4ADAMW_STATE_MAGIC 0x57444134u /* "4ADW" */

typedef enum {
    Q4_OK = 0,
    Q4_ERR_INVALID_ARG = 1,  /* null pointer, bad enum, block != 128, step == 0, beta outside [0,1),
                                eps <= 0, non-finite hyper-parameter */
    Q4_ERR_SHAPE = 2,        /* numel != prod(shape), ndim outside [1,8], numel >= 2^34, n_tensors <= 0 */
    Q4_ERR_ALIGNMENT = 3,    /* a device pointer not 16-byte aligned */
    Q4_ERR_CONFLICT = 4,     /* option combination outside the supported set (cf. [A] "Requirements and
                                errors": conflicting optimizer options fail before any work) */
    Q4_ERR_STATE_FORMAT = 5, /* state header does not match the configuration ([A]: 4-bit state resumes
                                only into the same 4-bit representation) */
    Q4_ERR_DEVICE = 6,       /* no usable gfx950 device, or a pointer not on the current device */
    Q4_ERR_WORKSPACE = 7,    /* workspace missing or smaller than q4adamw_workspace_bytes() */
    Q4_ERR_HIP = 8           /* a HIP runtime call or kernel launch failed */
} q4_status;

/* Recipes ([P] Table 2; factored mode of [A] "State representation"). */
typedef enum {
    Q4_RECIPE_ZIP_SR = 0,   /* NF4 m (RTN); Dyn4 v (zero-inclusive), Update-SR; no EDEN */
    Q4_RECIPE_ZE_EDEN = 1,  /* NF4 m (RTN); Dyn4-NZ v (zero-excluding), State-RTN; EDEN rescale */
    Q4_RECIPE_FACTORED = 2, /* NF4 m; matrices: row/column means of g^2; 1-D: Dyn4-NZ v, State-RTN */
    Q4_RECIPE_FP32 = 3,     /* quantization off: FP32 m and v (32-bit AdamW) */
    Q4_RECIPE_CUSTOM = 4,   /* codebooks and rules taken from the q4_config fields */
    Q4_RECIPE_BLOCK8 = 5    /* 8-bit blockwise AdamW ([A] names it beside the 4-bit optimizer; the two are
                               mutually exclusive): SDyn8 m, Dyn8 v, one byte per code, State-RTN, no
                               factorization */
} q4_recipe;

typedef enum {
    Q4_CB_NF4 = 0,     /* 4-bit NormalFloat, signed, contains 0 and +-1 */
    Q4_CB_SDYN4 = 1,   /* signed dynamic-exponent map: sign bit + 3-bit magnitude */
    Q4_CB_DYN4 = 2,    /* unsigned dynamic-exponent map, zero-inclusive */
    Q4_CB_DYN4_NZ = 3, /* unsigned dynamic-exponent map, zero-excluding (floor 1e-4) */
    Q4_CB_LIN4_NZ = 4, /* linear zero-excluding map k/16, k = 1..16 */
    Q4_CB_SDYN8 = 5,   /* 8-bit: sign bit + 7-bit dynamic magnitude (Q4_RECIPE_BLOCK8 only) */
    Q4_CB_DYN8 = 6     /* 8-bit unsigned dynamic-exponent map, zero-inclusive (Q4_RECIPE_BLOCK8 only) */
} q4_codebook;

/* Rounding rules ([P] Table 1). State rules round in v; Update rules round
 * in the preconditioner r = 1/(sqrt(v) + eps_sr). */
typedef enum {
    Q4_RULE_STATE_RTN = 0,
    Q4_RULE_STATE_SR = 1,
    Q4_RULE_UPDATE_RTN = 2,
    Q4_RULE_UPDATE_SR = 3
} q4_rule;

typedef struct {
    uint32_t abi_version; /* must be Q4ADAMW_ABI_VERSION */
    int32_t recipe;       /* q4_recipe */
    int32_t block;        /* must be 128 ([A] "State representation") */
    int32_t m_codebook;   /* q4_codebook (Q4_CB_NF4 or Q4_CB_SDYN4) */
    int32_t v_codebook;   /* q4_codebook (Q4_CB_DYN4, Q4_CB_DYN4_NZ or Q4_CB_LIN4_NZ) */
    int32_t m_rule;       /* Q4_RULE_STATE_RTN or Q4_RULE_STATE_SR (all tensors) */
    int32_t v_rule;       /* q4_rule */
    int32_t eden;         /* 1: EDEN block rescale of the quantized v ([P] abstract, ZE-EDEN) */
} q4_config;

/* Hyper-parameters of one step.  The host derives from them, in binary64
 * then rounded to FP32: decay = 1 - lr wd; step_size = lr / (1 - beta1^t);
 * rsbc2 = 1 / sqrt(1 - beta2^t) (torch-style AdamW bias correction). */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    float eps_sr;        /* epsilon of the preconditioner coordinate; <= 0 means "use eps" */
    uint64_t step;       /* 1-based step count t; also a Philox counter word */
    uint64_t seed;       /* Philox key */
    uint32_t lm_head_sr; /* 1 during the final-10% phase: tensors flagged Q4_TF_LM_HEAD round m by SR */
    uint32_t flags;      /* Q4_HP_* */
    float max_grad_norm; /* > 0: clip the gradients to this global L2 norm (see q4adamw_step); 0: off */
    uint32_t reserved;   /* 0 */
} q4_hparams;

#define Q4_HP_REUSE_TABLE 1u      /* the workspace already holds this exact tensor list from the previous
                                     q4adamw_step or q4adamw_accumulate with the same configuration: skip
                                     its upload.  The call then enqueues kernel launches only (no copy, no
                                     allocation, no synchronization), so it may be captured in a HIP graph
                                     once an earlier call on the device has run.  Without it, a call on a
                                     stream that is capturing a graph returns Q4_ERR_INVALID_ARG and
                                     enqueues nothing (the upload's host source would not outlive the
                                     call, so a replay could not read it) */
#define Q4_HP_CHECK_POINTERS 2u   /* also check that every pointer lives on the current device */
#define Q4_HP_GRAD_STATS 4u       /* the workspace holds the statistics of exactly these gradients, left by
                                     q4adamw_accumulate (Q4_ACC_LAST) or q4adamw_grad_stats with this
                                     tensor list and configuration: the step uses them and does not read the
                                     gradients a second time */

#define Q4_TF_LM_HEAD 1u          /* tensor is the LM head (its m switches to SR when lm_head_sr = 1) */

/* One parameter tensor and its state.  All buffers are device memory,
 * contiguous, row-major over `shape`.  Let n = numel, NB = ceil(n/128):
 *   param    float[n]        FP32 master weights, updated in place
 *   grad     uint16[n]       BF16 gradient bits, read only
 *   m_codes  uint8[ceil(n/2)], m_scales float[NB]   packed 4-bit m + block scales (in place)
 *   v_codes  uint8[ceil(n/2)], v_scales float[NB]   packed 4-bit v + block scales (in place;
 *                                                    NULL for a factored matrix)
 *   v_row    float[shape[0]], v_col float[prod(shape[1:])]  factored matrix only: EMA of the row
 *                                                    and column means of g^2 (in place)
 *   m_fp32, v_fp32 float[n]  FP32 recipe only (in place)
 * Codes: element 2j in the low nibble of byte j, element 2j+1 in the high
 * nibble (0 when n is odd).  Q4_RECIPE_BLOCK8: m_codes and v_codes are
 * uint8[n], byte i holding element i.  Blocks are parameter-local: block b
 * covers elements [128 b, min(128 b + 128, n)).
 * A shard (a data-parallel rank's share of a tensor, ZeRO style): blocks
 * [b0, b1) of a tensor passed as a tensor of their own, with every pointer
 * advanced to block b0 (param + 128 b0, m_codes + 64 b0, m_scales + b0, ...;
 * the byte codes of Q4_RECIPE_BLOCK8 + 128 b0), numel the shard's length,
 * elem_offset = 128 b0, and the whole tensor's tensor_id and flags.  b0 is
 * a multiple of 4 (elem_offset of 512), so the advanced pointers keep the
 * 16-byte alignment every pointer needs (a multiple of 32 keeps each
 * shard's scales on whole 128-byte lines, the layout the step runs best
 * on).  The
 * stochastic-rounding draws then use the element's index in the whole
 * tensor, so the shards of a tensor, stepped in one call or in several, give
 * bit for bit what the whole tensor gives.  A shard ends on a block
 * boundary unless it ends the tensor.  Factored matrices (the row and column
 * statistics span the whole matrix) take elem_offset = 0. */
typedef struct {
    uint32_t tensor_id; /* Philox counter word; stable across steps, distinct per tensor */
    uint32_t flags;     /* Q4_TF_* */
    int32_t ndim;
    int32_t reserved;
    int64_t shape[Q4ADAMW_MAX_NDIM];
    int64_t numel;
    float* param;
    const uint16_t* grad;
    uint8_t* m_codes;
    float* m_scales;
    uint8_t* v_codes;
    float* v_scales;
    float* v_row;
    float* v_col;
    float* m_fp32;
    float* v_fp32;
    int64_t elem_offset; /* index of element 0 in the whole tensor: 0, or 128 b0 (a multiple of 512) */
} q4_tensor;

typedef struct {
    uint64_t adam4_quantized_state_bytes; /* packed codes (FP32 recipe: the two FP32 moments) */
    uint64_t adam4_scale_metadata_bytes;  /* block scales, plus factored row/column vectors */
    uint64_t adam4_total_bytes;
} q4_state_bytes;

/* Header a caller stores beside saved state, checked on resume. */
typedef struct {
    uint32_t magic;          /* Q4ADAMW_STATE_MAGIC */
    uint32_t abi_version;
    uint32_t layout_version; /* Q4ADAMW_LAYOUT_VERSION */
    int32_t recipe, m_codebook, v_codebook, m_rule, v_rule, eden, block;
} q4_state_header;

/* ---- helpers (host only, no device work) ------------------------------ */

uint32_t q4adamw_abi_version(void);
const char* q4adamw_status_string(q4_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* q4adamw_last_error(void);

/* Fill *cfg with the recipe's codebooks and rules ([P] Table 2). */
q4_status q4adamw_default_config(int32_t recipe, q4_config* cfg);

/* Validate a configuration, hyper-parameters (hp may be NULL) and tensor
 * list without touching any device: the checks q4adamw_step performs first. */
q4_status q4adamw_validate(const q4_config* cfg, const q4_hparams* hp, const q4_tensor* t, int32_t n_tensors);

/* Bytes of workspace q4adamw_step needs for this tensor list (>= 256). */
q4_status q4adamw_workspace_bytes(const q4_config* cfg, const q4_tensor* t, int32_t n_tensors, size_t* bytes);

/* Persistent state bytes of the tensor list ([A] "Requirements and errors";
 * [N] storage paragraph: 1.0625 B/param whenever 128 divides numel). */
q4_status q4adamw_state_bytes(const q4_config* cfg, const q4_tensor* t, int32_t n_tensors, q4_state_bytes* out);

q4_status q4adamw_make_header(const q4_config* cfg, q4_state_header* out);
/* Q4_ERR_STATE_FORMAT unless `hdr` was made for an identical configuration. */
q4_status q4adamw_check_header(const q4_config* cfg, const q4_state_header* hdr);

/* The FP32 scalars of one step, exactly as passed to the kernels:
 * out = {decay, step_size, rsbc2, 1 - beta1, 1 - beta2}. */
q4_status q4adamw_host_scalars(const q4_hparams* hp, float out[5]);

/* The library's decode table of a codebook, indexed by code (host copy of
 * the table the kernels use): 16 entries, or 256 for the 8-bit maps. */
q4_status q4adamw_codebook(int32_t codebook, float* out);

/* ---- device entry points ---------------------------------------------- */

/* Fresh state, "moments start at 0": every code set to the code that
 * decodes to 0 (NF4/SDyn4: zero; Dyn4: zero; Dyn4-NZ/Lin4-NZ: the floor
 * code, which decodes to 0 under scale 0), every scale +0, v_row = v_col = 0,
 * FP32 moments 0.  Params and grads are not touched (may be NULL). */
q4_status q4adamw_init_state(const q4_config* cfg, const q4_tensor* t, int32_t n_tensors, void* stream);

/* One fused AdamW step over all tensors ([N] AdamW paragraph; [A] "State
 * representation"; [P] Table 1, Table 2).  Per 128-element block: decode m
 * and v, form m1 = b1 m0 + (1-b1) g and v1 = b2 v0 + (1-b2) g^2 (each one
 * fused multiply-add onto the rounded gradient term; or the factored
 * estimate (R_r C_c)/mean(R) for matrices of the factored recipe, after R
 * and C take their own EMA of this step's row/column means of g^2), update
 * the weight p <- p decay - step_size m1 / (sqrt(v1) rsbc2 + eps) from the
 * unquantized m1, v1, then requantize: absmax scales, the m rule (RTN, or
 * SR for the LM head in the final phase), the v rule, EDEN.  A block is
 * normalized by the IEEE reciprocal of its scale (subnormal scales
 * included); a block whose scale is 0, or so small that its reciprocal
 * overflows (s <= 2^-128), stores the code of zero in every slot and keeps
 * its scale as computed.
 * Non-finite gradients (the pages are silent; IEEE operations decide): the
 * block maxima skip NaN and keep +inf; an infinite scale normalizes by 0;
 * a NaN normalized value (a NaN moment, or inf * 0) takes the lowest level
 * of its map; EDEN's ratio over a block holding one is 1; weights follow
 * IEEE arithmetic (NaN where the Adam term is NaN).  Such a block stays
 * poisoned (infinite or zero scales) while its gradients do.
 * Clipping (hp->max_grad_norm > 0): s = min(1, max_grad_norm / (norm +
 * 1e-6)) in binary64, rounded to FP32, from the global norm of the
 * gradients (the statistics in ws with Q4_HP_GRAD_STATS, else gathered
 * first by one read of the gradients); every gradient element is multiplied
 * by s before use and the factored row/column sums of g^2 by s^2.  A NaN
 * norm gives s = 1 (the comparison with 1 fails), an infinite norm s = 0.
 * Stochastic rounding draws Philox4x32-10 with counter (i/4, step,
 * tensor_id, stream 0 for m / 1 for v), key (seed), word i mod 4.
 * `ws` (device, ws_bytes >= q4adamw_workspace_bytes) holds the tensor table,
 * the factored partial sums, the clip statistics and the 8-bit step's run
 * queue (cleared on the stream before each 8-bit launch); it must not be
 * used by another call that overlaps on the device. */
q4_status q4adamw_step(const q4_config* cfg, const q4_hparams* hp, const q4_tensor* t, int32_t n_tensors,
                       void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as q4adamw_step, with the workspace in a static device array of the
 * library (Q4ADAMW_NOALLOC_SCRATCH_BYTES on each device it runs on, held
 * until the process ends) instead of a caller's buffer.  It calls no
 * hipMalloc, hipFree or other allocating routine.  A tensor list whose
 * workspace (q4adamw_workspace_bytes) exceeds the array is refused with
 * Q4_ERR_WORKSPACE before anything is enqueued: every packed and 8-bit set
 * fits (the tensor table takes 128 bytes per tensor), a factored set fits
 * while its row/column partial sums do (e.g. Qwen3-0.6B, 27 MiB).  Every
 * call on a device shares that device's array and leaves the last call's
 * contents there: two calls that overlap on one device (different streams
 * without ordering, or host threads) race.  Q4_HP_REUSE_TABLE means "the
 * previous call on this device, of either entry point's workspace kind,
 * left this exact tensor list in the array". */
#define Q4ADAMW_NOALLOC_SCRATCH_BYTES (32u << 20)
q4_status q4adamw_step_noalloc(const q4_config* cfg, const q4_hparams* hp, const q4_tensor* t, int32_t n_tensors,
                               void* stream);

/* ---- the step before: gradient accumulation, norm, clipping ------------
 * [A] "State representation": microbatches stream into BF16 gradient shards
 * (no FP32 main gradient), and the gradient norm and clipping work on those
 * BF16 shards.  A microbatch's gradients arrive as one flat device buffer
 * of BF16 values in which tensor i starts at element offsets[i] =
 * 512 * sum_{j<i} ceil(numel_j / 512) (q4adamw_flat_offsets); the elements
 * between tensors are not read. */

#define Q4_ACC_FIRST 1        /* first microbatch: grad <- micro (instead of adding) */
#define Q4_ACC_LAST 2         /* last microbatch: also leave the gradients' statistics in ws */
#define Q4_ACC_REUSE_TABLE 4  /* as Q4_HP_REUSE_TABLE */

/* offsets[i] (host, n_tensors entries) and *total (elements of the flat
 * buffer) of the flat microbatch layout above. */
q4_status q4adamw_flat_offsets(const q4_tensor* t, int32_t n_tensors, int64_t* offsets, int64_t* total);

/* Accumulate one microbatch into the BF16 gradient buffers t[i].grad
 * (device, written in place although q4_tensor declares them const): per
 * element g <- bf16(f32(g) + f32(micro)), rounded to nearest even, or
 * g <- micro with Q4_ACC_FIRST.  With Q4_ACC_LAST the same pass leaves in
 * `ws` the statistics of the accumulated gradients: their binary64 sum of
 * squares over all tensors and, for the matrices of the factored recipe,
 * the per-row and per-column partial sums of g^2 that q4adamw_step would
 * otherwise gather with a second read of the gradients.  `micro` (device):
 * the flat microbatch buffer.  `ws`: as for q4adamw_step, the same buffer
 * the step will get. */
q4_status q4adamw_accumulate(const q4_config* cfg, const q4_tensor* t, int32_t n_tensors, const uint16_t* micro,
                             int32_t flags, void* ws, size_t ws_bytes, void* stream);

/* The statistics of Q4_ACC_LAST for gradients accumulated elsewhere (one
 * read of every gradient). */
q4_status q4adamw_grad_stats(const q4_config* cfg, const q4_tensor* t, int32_t n_tensors, void* ws, size_t ws_bytes,
                             void* stream);

/* The global L2 norm sqrt(sum of squares) from the statistics in ws:
 * waits for `stream`, then stores it to *norm (host). */
q4_status q4adamw_grad_norm(const void* ws, size_t ws_bytes, double* norm, void* stream);

/* Decode one tensor's state to FP32 (device m_out, v_out of numel floats,
 * 16-byte aligned): m = L_m[code] s_m; v = L_v[code] s_v, or
 * (R_r C_c)/mean(R) for a factored matrix (the stored second moment, without
 * bias correction).  `ws` (device) is only used for a factored matrix and
 * then needs 256 + 8 ceil(shape[0]/256) bytes, rounded up to 256; it may be
 * NULL otherwise.  FP32 recipe: copies m_fp32 and v_fp32. */
q4_status q4adamw_dequant_state(const q4_config* cfg, const q4_tensor* t, float* m_out, float* v_out,
                                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* Q4ADAMW_H */
