// q4_internal.h -- structures shared by the host ABI (q4_abi.cpp) and the
// HIP kernels (q4_kernels.hip) of the fused 4-bit AdamW step.  Not part of
// the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4 {

constexpr int kBlock = 128;            // elements per quantization block
constexpr int kBlocksPerChunk = 4;     // one wavefront step: 4 blocks = 512 elements
constexpr int kChunkElems = kBlock * kBlocksPerChunk;
constexpr int kWavesPerGroup = 4;      // 256-thread work-groups
constexpr int kBandRows = 256;         // rows per band of the row/column partial kernel
constexpr int kTileCols = 512;         // columns per tile (64 lanes x 8 BF16)
constexpr int kGroup = 256;            // rows per finalize work-group
constexpr int kColGroup = 64;          // columns per finalize work-group (4 band slices of 64 lanes)
// The quantized steps number chunks in a prefix where every tensor starts at
// a multiple of kStepAlignChunks (8 chunks = 32 block scales = one 128-byte
// line of each scale array); a work-group of the steps takes one run of 4
// or 8 consecutive slabs of kWavesPerGroup chunks (at least 2 slabs, 8
// chunks, while the set has a run for every resident group), so each scale
// line is written whole by one work-group.
constexpr int64_t kStepAlignChunks = 8;

// Gradient pass modes: read the gradient for its statistics only, copy the
// microbatch into it, or add the microbatch to it.
enum GradMode : int { GRAD_STATS_ONLY = 0, GRAD_FIRST = 1, GRAD_ADD = 2 };

enum Kind : int32_t { KIND_PACKED = 0, KIND_FACTORED = 1, KIND_FP32 = 2, KIND_BYTE8 = 3 };

// One tensor as the step kernel sees it (128 bytes, read with scalar loads).
struct alignas(16) DevTensor {
    float* param;
    const uint16_t* grad;
    uint8_t* m_codes;
    float* m_scales;
    uint8_t* v_codes;
    float* v_scales;
    float* v_row;
    float* v_col;
    float* m32;
    float* v32;
    int64_t numel;
    int64_t cols;          // factored matrix: numel / shape[0]; else 0
    int64_t chunk_begin;   // first chunk of this tensor in the plain prefix (512 x it = its flat offset)
    const float* inv_meanR;  // factored matrix: slot written by the finalize kernel
    uint32_t tensor_id;
    uint32_t flags;
    int32_t kind;
    uint32_t ctr_base;     // Philox counter of element 0: (elem_offset / 4) mod 2^32
};
static_assert(sizeof(DevTensor) == 128, "DevTensor layout");

// One factored matrix [rows, cols] for the row/column statistics kernels.
struct alignas(16) DevMatrix {
    const uint16_t* grad;
    float* R;
    float* C;
    double* part_row;    // [n_ctiles][rows] partial row sums of g^2
    double* part_col;    // [n_bands][cols] partial column sums of g^2
    double* part_mean;   // [n_rgroups] sums of the updated R over 256-row groups
    float* inv_meanR;    // 1 / mean(R) after the update (0 if mean(R) is 0)
    int64_t rows, cols;
    int64_t tile_begin;  // first tile (band x column tile) of this matrix
    int64_t n_ctiles, n_bands;
    int64_t rgroup_begin, n_rgroups;
    int64_t cgroup_begin, n_cgroups;
    int64_t flat_off;    // element offset of this matrix in a flat microbatch gradient buffer
    int64_t pad[2];
};
static_assert(sizeof(DevMatrix) == 160, "DevMatrix layout");

// Scalars of one step, passed by value.
struct StepScalars {
    float beta1, beta2, omb1, omb2, eps, eps_sr, decay, step_size, rsbc2;
    uint32_t step;        // low 32 bits of the step count (Philox counter word)
    uint32_t key0, key1;  // Philox key (seed)
    uint32_t flags;       // SF_*
};
enum StepFlags : uint32_t {
    SF_LM_HEAD_SR = 1u,  // final phase: LM-head tensors round m by SR
    SF_M_SR_ALL = 2u,    // every tensor rounds m by SR
    SF_EDEN = 4u,        // EDEN rescale of packed v
    SF_CLIP = 8u,        // scale the gradients by the clip factor in the workspace
};

// Workspace layout shared by host and kernels: the first 256 bytes hold the
// gradient statistics' sum of squares (binary64, offset 0), the clip factor
// (FP32, offset 8) and the run queue of the 8-bit step (a 64-bit counter,
// offset 16, zeroed before each launch); the tensor table starts at byte
// 256, so a kernel that has the table finds the others before it.
constexpr size_t kWsOffSq = 0, kWsOffClip = 8, kWsOffQueue = 16, kWsOffTable = 256;
__host__ __device__ inline const float* clip_of_table(const DevTensor* tab) {
    return reinterpret_cast<const float*>(reinterpret_cast<const char*>(tab) - kWsOffTable + kWsOffClip);
}
__host__ __device__ inline unsigned long long* queue_of_table(const DevTensor* tab) {
    return reinterpret_cast<unsigned long long*>(const_cast<char*>(reinterpret_cast<const char*>(tab)) - kWsOffTable +
                                                 kWsOffQueue);
}

// Kernel variants that exist (m codebook, v codebook, v rule).
struct Variant { int mcb, vcb, vrule; };

// has_matrices: the tensor list holds factored matrices (their row/column
// gathers run best at 7 work-groups per CU, which the launch then enforces).
// The fused and 8-bit steps take the aligned step prefix (kStepAlignChunks);
// the FP32 step takes the plain one.
hipError_t launch_fused_step(const Variant& v, const StepScalars& sc, const DevTensor* d_tab,
                             const int64_t* d_chunk_begin, int n_tensors, int64_t total_chunks,
                             bool has_matrices, hipStream_t stream);
hipError_t launch_fp32_step(const StepScalars& sc, const DevTensor* d_tab, const int64_t* d_chunk_begin,
                            int n_tensors, int64_t total_chunks, hipStream_t stream);
hipError_t launch_block8_step(const StepScalars& sc, const DevTensor* d_tab, const int64_t* d_chunk_begin,
                              int n_tensors, int64_t total_chunks, hipStream_t stream);
// K2 (skipped when the partials are already in the workspace), K3a, K3b.
hipError_t launch_factored_stats(const DevMatrix* d_mats, int n_mats, int64_t total_tiles, int64_t total_rgroups,
                                 int64_t total_cgroups, float beta2, float omb2, const float* clip, bool partials_ready,
                                 hipStream_t stream);
// Work-groups and run length of the chunk-order accumulation pass over
// total_chunks chunks: one group per run of up to 4 slabs (shorter runs
// while the set has fewer than 2048 of them), at most 2^22 groups, each
// leaving one partial sum of squares when it is the last pass.
struct AccLaunch {
    int64_t groups;
    int run_slabs;
};
AccLaunch acc_launch(int64_t total_chunks);
constexpr int kSqStageGroups = 256;  // work-groups of the total's first stage
// One pass over the gradients: mode GradMode; with `last` it also leaves the
// factored row/column partials of matrices (when `tiles_for_matrices`) and
// the binary64 sums of squares in sq_part (acc_launch(chunks).groups +
// total_tiles slots, then kSqStageGroups more for the first stage of the
// total), then their total in *sq.
// With last and matrices, the tile kernel takes the matrices and the chunk
// pass runs over d_tab1 / d_chunks1 (the other tensors alone, each entry
// keeping its chunk_begin in the full prefix for the flat offset).
hipError_t launch_grad_pass(int mode, bool last, bool tiles_for_matrices, const DevTensor* d_tab,
                            const int64_t* d_chunk_begin, int n_tensors, int64_t total_chunks, const DevMatrix* d_mats,
                            int n_mats, int64_t total_tiles, const DevTensor* d_tab1, const int64_t* d_chunks1,
                            int n_tensors1, int64_t total_chunks1, const uint16_t* micro, double* sq_part, double* sq,
                            hipStream_t stream);
// *clip = min(1, max_norm / (sqrt(*sq) + 1e-6)) rounded to FP32.
hipError_t launch_clip_factor(const double* sq, float max_norm, float* clip, hipStream_t stream);
hipError_t launch_fill(void* p, size_t bytes, uint8_t value, hipStream_t stream);
hipError_t launch_dequant(int mcb, int vcb, const DevTensor& t, int64_t rows, float* m_out, float* v_out,
                          double* ws_partials, float* ws_inv, hipStream_t stream);
bool variant_supported(const Variant& v);
// The static device scratch of q4adamw_step_noalloc: kScratchBytes on every
// device, its address on the current device in *ptr (looked up once per
// device).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_address(void** ptr);
void codebook_table(int cb, float* out);  // 16 entries, 256 for the 8-bit maps

}  // namespace q4
