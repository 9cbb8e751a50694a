// q4_probe.hip -- bandwidth probes that give the fused step's practical
// ceiling on the machine they run on (libq4probe.so, loaded by the
// benchmark and its tests; the optimizer library does not use it).
//
// k_byte_mix moves exactly the bytes the packed 4-bit step moves per element
// (FP32 master read and written, BF16 gradient read, two 4-bit code streams
// read and written, two FP32 block-scale streams read and written: 12.125
// bytes per element), with the step's lane layout (a 128-element block per
// 16-lane row, lane s on elements 4s .. 4s+3 and 64+4s .. 64+4s+3 of it, two
// 16-byte accesses for masters, two 8-byte ones for gradients, two 16-bit
// ones per moment's codes, the row's scale read by all its lanes and written
// by one), its cache policy (masters and gradients nontemporal) and its work
// distribution (one 4-wavefront group per run of consecutive slabs of 4
// chunks), but only trivial arithmetic.  Its time is what this byte mix
// costs on the memory system, whatever the optimizer computes.
//
// k_byte_mix8 does the same for the 8-bit blockwise step: one code byte per
// element and moment (two 4-byte accesses per lane), 14.125 bytes per
// element.
//
// k_copy is a plain copy (known bytes read and written, 16 bytes per lane
// access), which also calibrates the HBM traffic counters; k_update rewrites
// a buffer in place, as the step rewrites its masters, codes and scales;
// k_read reads only.  Each takes the fastest of the forms measured on
// gfx950, since it stands for what the memory system can do (copy and
// update stream nontemporal: 2% and 3.5% faster than the default policy).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdint.h>

#include "../../include/q4probe.h"

namespace {

// runs of slabs: 8 as the ZIP-SR steps take them (the 4-bit mix), 4 as the
// 8-bit step does
constexpr int kChunk = 512, kWaves = 4, kRun = 8, kRun8 = 4;

template <class T> using gptr = __attribute__((address_space(1))) T*;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int64_t next_chunk(int64_t c, int& j, int run, int64_t groups) {
    if (++j < run) return c + kWaves;
    j = 0;
    return c + (groups * run - (run - 1)) * kWaves;
}

// A lane's codes of one moment in each half of its block: 4 nibbles (4-bit
// codes) or 4 bytes.
template <int BITS> struct LaneCodes;
template <> struct LaneCodes<4> { typedef uint16_t T; };
template <> struct LaneCodes<8> { typedef uint32_t T; };

// One chunk of the byte mix: 512 elements, lane s of row r on elements
// 128r + 4s .. +3 and 128r + 64 + 4s .. +3, BITS-bit codes.
template <int BITS>
__device__ __forceinline__ void mix_chunk(float* __restrict__ param, const uint16_t* __restrict__ grad,
                                          uint8_t* __restrict__ mcodes, uint8_t* __restrict__ vcodes,
                                          float* __restrict__ mscales, float* __restrict__ vscales, int64_t c,
                                          int lane, float a) {
    typedef typename LaneCodes<BITS>::T CodeT;
    const int64_t c0 = c * kChunk;
    const int le = (lane & 48) * 8 + (lane & 15) * 4;
    const gptr<float> p = (gptr<float>)param + c0 + le;
    const gptr<const uint16_t> g = (gptr<const uint16_t>)grad + c0 + le;
    const gptr<CodeT> mc = (gptr<CodeT>)(mcodes + (c0 + le) * BITS / 8);
    const gptr<CodeT> vc = (gptr<CodeT>)(vcodes + (c0 + le) * BITS / 8);
    constexpr int kHalf = 64 * BITS / 8 / sizeof(CodeT);  // the second half's codes, in CodeT units
    const int64_t blk = c * 4 + (lane >> 4);
    f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(p));
    f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const gptr<const f32x4>>(p + 64));
    const u32x2 qa = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(g));
    const u32x2 qb = __builtin_nontemporal_load(reinterpret_cast<const gptr<const u32x2>>(g + 64));
    const CodeT m0 = mc[0], m1 = mc[kHalf], v0 = vc[0], v1 = vc[kHalf];
    const float sm = ((gptr<float>)mscales)[blk], sv = ((gptr<float>)vscales)[blk];
    // trivial, data-dependent arithmetic: nothing can be elided
    const float gq = __uint_as_float(qa.x << 16) + __uint_as_float(qb.y & 0xFFFF0000u);
    x = x * a + gq;
    y = y * a + gq;
    __builtin_nontemporal_store(x, reinterpret_cast<gptr<f32x4>>(p));
    __builtin_nontemporal_store(y, reinterpret_cast<gptr<f32x4>>(p + 64));
    mc[0] = (CodeT)(m0 ^ qa.y);
    mc[kHalf] = (CodeT)(m1 ^ qa.y);
    vc[0] = (CodeT)(v0 ^ qb.x);
    vc[kHalf] = (CodeT)(v1 ^ qb.x);
    if ((lane & 15) == 0) {
        ((gptr<float>)mscales)[blk] = sm * a;
        ((gptr<float>)vscales)[blk] = sv * a;
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void k_byte_mix(float* __restrict__ param, const uint16_t* __restrict__ grad,
                                                   uint8_t* __restrict__ mcodes, uint8_t* __restrict__ vcodes,
                                                   float* __restrict__ mscales, float* __restrict__ vscales,
                                                   int64_t chunks, int run, float a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t groups = gridDim.x;
    int64_t c = (int64_t)blockIdx.x * run * kWaves + wave;
    for (int j = 0; c < chunks; c = next_chunk(c, j, run, groups))
        mix_chunk<BITS>(param, grad, mcodes, vcodes, mscales, vscales, c, lane, a);
}

// The same chunks taken from a queue: one round of resident work-groups,
// each taking the next run of `run` slabs from a counter (zero at launch)
// until none is left, so the groups work on a window of neighbouring runs
// and a group that finishes early takes more.  The fastest way found to
// move this byte mix on gfx950 (5.25 TB/s against 5.07 for the step's own
// walk; runs of 2 slabs 4.08, of 32 slabs 5.04).
template <int BITS>
__global__ __launch_bounds__(256) void k_byte_mix_queue(float* __restrict__ param, const uint16_t* __restrict__ grad,
                                                         uint8_t* __restrict__ mcodes, uint8_t* __restrict__ vcodes,
                                                         float* __restrict__ mscales, float* __restrict__ vscales,
                                                         int64_t chunks, int run, unsigned int* __restrict__ queue,
                                                         float a) {
    __shared__ unsigned int next;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t runs = ((chunks + kWaves - 1) / kWaves + run - 1) / run;
    for (;;) {
        __syncthreads();  // every wave has read the previous run
        if (threadIdx.x == 0) next = atomicAdd(queue, 1u);
        __syncthreads();
        const int64_t r = __builtin_amdgcn_readfirstlane(next);
        if (r >= runs) break;
        for (int64_t c = r * run * kWaves + wave, s = 0; s < run && c < chunks; ++s, c += kWaves)
            mix_chunk<BITS>(param, grad, mcodes, vcodes, mscales, vscales, c, lane, a);
    }
}

// Wave-contiguous segments: a wavefront moves kSegVec consecutive 16-byte
// vectors (16 KiB) with all its loads in flight before its stores, and the
// segments go round the wavefronts; a tail shorter than a segment is done
// vector by vector.  The fastest of the copy forms measured on gfx950:
// 5.59 TB/s, against 5.11 TB/s for a grid-stride sweep with eight loads in
// flight per lane (1x to 8x the resident work-groups, 4 to 16 loads).
constexpr int kSegLoads = 16;
constexpr int64_t kSegVec = 64 * kSegLoads;

__device__ __forceinline__ int64_t wave_id() { return (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); }

__global__ __launch_bounds__(256) void k_copy(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t n16) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * 4;
    const int64_t nseg = n16 / kSegVec;
    for (int64_t sg = wave_id(); sg < nseg; sg += waves) {
        const int64_t b = sg * kSegVec + lane;
        u32x4 v[kSegLoads];
#pragma unroll
        for (int u = 0; u < kSegLoads; ++u) v[u] = __builtin_nontemporal_load((gptr<const u32x4>)src + b + 64 * u);
#pragma unroll
        for (int u = 0; u < kSegLoads; ++u) __builtin_nontemporal_store(v[u], (gptr<u32x4>)dst + b + 64 * u);
    }
    for (int64_t i = nseg * kSegVec + wave_id() * 64 + lane; i < n16; i += waves * 64)
        ((gptr<u32x4>)dst)[i] = ((gptr<const u32x4>)src)[i];
}

// x <- x * a in place, in the copy's wave-contiguous form: the read and the
// write of every byte go to the same address, as the step's updates do.
__global__ __launch_bounds__(256) void k_update(f32x4* __restrict__ x, int64_t n16, float a) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * 4;
    const int64_t nseg = n16 / kSegVec;
    for (int64_t sg = wave_id(); sg < nseg; sg += waves) {
        const int64_t b = sg * kSegVec + lane;
        f32x4 v[kSegLoads];
#pragma unroll
        for (int u = 0; u < kSegLoads; ++u) v[u] = __builtin_nontemporal_load((gptr<const f32x4>)x + b + 64 * u);
#pragma unroll
        for (int u = 0; u < kSegLoads; ++u) __builtin_nontemporal_store(v[u] * a, (gptr<f32x4>)x + b + 64 * u);
    }
    for (int64_t i = nseg * kSegVec + wave_id() * 64 + lane; i < n16; i += waves * 64)
        ((gptr<f32x4>)x)[i] = ((gptr<const f32x4>)x)[i] * a;
}

__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = ((gptr<const u32x4>)src)[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // one store per thread whose value is never 0 for data the caller made
    // non-zero, so the loads stay; a sink of gridDim.x * 256 words
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

int resident_groups(const void* kernel) {
    static std::atomic<int> cus{0};
    if (cus.load() == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        const bool ok = hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess;
        cus.store(ok && prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256);
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    return per_cu * cus.load();
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The queue counter of k_byte_mix_queue: a device word of this library, its
// address looked up once per device.
__device__ unsigned int queue_word;

hipError_t queue_address(unsigned int** ptr) {
    static std::mutex mu;
    static unsigned int* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(queue_word));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<unsigned int*>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

bool mix_args_ok(const float* param, const uint16_t* grad, const uint8_t* m_codes, const uint8_t* v_codes,
                 const float* m_scales, const float* v_scales, int64_t n) {
    if (n <= 0 || n % kChunk != 0) return false;
    if (!param || !grad || !m_codes || !v_codes || !m_scales || !v_scales) return false;
    return a16(param) && a16(grad) && a16(m_codes) && a16(v_codes) && a16(m_scales) && a16(v_scales);
}

// One work-group per run of `max_run` slabs, as the quantized steps launch
// (runs halved while the set has fewer than one per resident group; a set
// with more than 2^22 runs loops over them).
template <int BITS>
int launch_mix(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
               float* v_scales, int64_t n, int max_run, void* stream) {
    if (!mix_args_ok(param, grad, m_codes, v_codes, m_scales, v_scales, n)) return Q4PROBE_ERR_ARG;
    const int64_t chunks = n / kChunk;
    const int64_t slabs = (chunks + kWaves - 1) / kWaves;
    static std::atomic<int> resident{0};
    if (resident.load() == 0) resident.store(resident_groups(reinterpret_cast<const void*>(k_byte_mix<BITS>)));
    int run = max_run;
    while (run > 1 && slabs / run < resident.load()) run >>= 1;
    const int64_t runs = (slabs + run - 1) / run;
    const int64_t max_groups = int64_t(1) << 22;
    const int grid = (int)(runs < max_groups ? runs : max_groups);
    k_byte_mix<BITS><<<grid, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(param, grad, m_codes, v_codes,
                                                                             m_scales, v_scales, chunks, run, 0.999f);
    return hipGetLastError() == hipSuccess ? Q4PROBE_OK : Q4PROBE_ERR_HIP;
}

// One round of resident work-groups taking runs of `max_run` slabs from the
// queue word, zeroed before the launch.
template <int BITS>
int launch_mix_queue(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                     float* v_scales, int64_t n, int max_run, void* stream) {
    if (!mix_args_ok(param, grad, m_codes, v_codes, m_scales, v_scales, n)) return Q4PROBE_ERR_ARG;
    unsigned int* queue = nullptr;
    if (queue_address(&queue) != hipSuccess) return Q4PROBE_ERR_HIP;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int64_t chunks = n / kChunk;
    const int64_t slabs = (chunks + kWaves - 1) / kWaves;
    static std::atomic<int> resident{0};
    if (resident.load() == 0)
        resident.store(resident_groups(reinterpret_cast<const void*>(k_byte_mix_queue<BITS>)));
    const int64_t groups = resident.load();
    int run = max_run;
    while (run > 1 && slabs / run < groups) run >>= 1;
    const int64_t runs = (slabs + run - 1) / run;
    if (hipMemsetAsync(queue, 0, sizeof(unsigned int), st) != hipSuccess) return Q4PROBE_ERR_HIP;
    k_byte_mix_queue<BITS><<<(unsigned)(runs < groups ? runs : groups), 256, 0, st>>>(
        param, grad, m_codes, v_codes, m_scales, v_scales, chunks, run, queue, 0.999f);
    return hipGetLastError() == hipSuccess ? Q4PROBE_OK : Q4PROBE_ERR_HIP;
}

// Work-groups of the wave-contiguous probes: 2x the resident groups (4096
// on gfx950, as fast as 8192 and faster than 2048 or 16384), never more than
// one segment per wavefront.
unsigned segment_grid(int64_t n16, const void* kernel, std::atomic<int>& resident) {
    if (resident.load() == 0) resident.store(resident_groups(kernel));
    const int64_t need = (n16 / kSegVec + 3) / 4 + 1;
    const int64_t cap = 2 * (int64_t)resident.load();
    return (unsigned)(need < cap ? need : cap);
}

}  // namespace

extern "C" {

int64_t q4probe_byte_mix_bytes(int64_t n) { return n <= 0 ? 0 : 10 * n + 2 * n + (n / 128) * 16; }

int q4probe_byte_mix(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                     float* v_scales, int64_t n, void* stream) {
    return launch_mix<4>(param, grad, m_codes, v_codes, m_scales, v_scales, n, kRun, stream);
}

int q4probe_byte_mix_queue(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                           float* v_scales, int64_t n, void* stream) {
    return launch_mix_queue<4>(param, grad, m_codes, v_codes, m_scales, v_scales, n, kRun, stream);
}

int64_t q4probe_byte_mix8_bytes(int64_t n) { return n <= 0 ? 0 : 10 * n + 4 * n + (n / 128) * 16; }

int q4probe_byte_mix8(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                      float* v_scales, int64_t n, void* stream) {
    return launch_mix<8>(param, grad, m_codes, v_codes, m_scales, v_scales, n, kRun8, stream);
}

int q4probe_byte_mix8_queue(float* param, const uint16_t* grad, uint8_t* m_codes, uint8_t* v_codes, float* m_scales,
                            float* v_scales, int64_t n, void* stream) {
    return launch_mix_queue<8>(param, grad, m_codes, v_codes, m_scales, v_scales, n, kRun8, stream);
}

int q4probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || bytes == 0 || bytes % 16 != 0 || !a16(dst) || !a16(src)) return Q4PROBE_ERR_ARG;
    static std::atomic<int> resident{0};
    const int64_t n16 = (int64_t)(bytes / 16);
    k_copy<<<segment_grid(n16, reinterpret_cast<const void*>(k_copy), resident), 256, 0,
             reinterpret_cast<hipStream_t>(stream)>>>(reinterpret_cast<u32x4*>(dst),
                                                      reinterpret_cast<const u32x4*>(src), n16);
    return hipGetLastError() == hipSuccess ? Q4PROBE_OK : Q4PROBE_ERR_HIP;
}

int q4probe_update_in_place(float* x, size_t bytes, void* stream) {
    if (!x || bytes == 0 || bytes % 16 != 0 || !a16(x)) return Q4PROBE_ERR_ARG;
    static std::atomic<int> resident{0};
    const int64_t n16 = (int64_t)(bytes / 16);
    k_update<<<segment_grid(n16, reinterpret_cast<const void*>(k_update), resident), 256, 0,
               reinterpret_cast<hipStream_t>(stream)>>>(reinterpret_cast<f32x4*>(x), n16, 0.999f);
    return hipGetLastError() == hipSuccess ? Q4PROBE_OK : Q4PROBE_ERR_HIP;
}

int64_t q4probe_read_sink_words(void) { return 4 * 1024 * 256; }

int q4probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !a16(src)) return Q4PROBE_ERR_ARG;
    static std::atomic<int> resident{0};
    if (resident.load() == 0) resident.store(resident_groups(reinterpret_cast<const void*>(k_read)));
    // one round of resident groups sweeping the buffer together: the
    // fastest read form measured on gfx950 (more groups, queued behind the
    // first round, start elsewhere in the buffer and read slower)
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t need = (n16 + 255) / 256;
    int64_t cap = (int64_t)resident.load();
    if (cap > q4probe_read_sink_words() / 256) cap = q4probe_read_sink_words() / 256;
    k_read<<<(unsigned)(need < cap ? need : cap), 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError() == hipSuccess ? Q4PROBE_OK : Q4PROBE_ERR_HIP;
}

}  // extern "C"
