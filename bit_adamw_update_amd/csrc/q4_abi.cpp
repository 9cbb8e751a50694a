// q4_abi.cpp -- host side of the C ABI declared in include/q4adamw.h:
// validation, the host scalars of a step, the workspace layout, the tensor
// table upload and the kernel launches.  Every entry point validates first
// and enqueues nothing when it returns an error.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/q4adamw.h"
#include "q4_internal.h"

using namespace q4;

namespace {

thread_local std::string g_last_error;

q4_status fail(q4_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}
q4_status ok() {
    g_last_error.clear();
    return Q4_OK;
}

constexpr int64_t kMaxNumel = int64_t(1) << 34;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Resolved configuration: what the kernels run.
struct Resolved {
    int recipe;
    Variant var;
    int m_sr_all;
    int eden;
};

q4_status resolve(const q4_config* cfg, Resolved* r) {
    if (!cfg) return fail(Q4_ERR_INVALID_ARG, "config is NULL");
    if (cfg->abi_version != Q4ADAMW_ABI_VERSION)
        return fail(Q4_ERR_INVALID_ARG, "config abi_version %u != %u", cfg->abi_version, Q4ADAMW_ABI_VERSION);
    if (cfg->block != Q4ADAMW_BLOCK) return fail(Q4_ERR_INVALID_ARG, "block must be 128 (got %d)", cfg->block);
    if (cfg->recipe < Q4_RECIPE_ZIP_SR || cfg->recipe > Q4_RECIPE_BLOCK8)
        return fail(Q4_ERR_INVALID_ARG, "unknown recipe %d", cfg->recipe);
    if (cfg->recipe == Q4_RECIPE_FP32) {
        *r = Resolved{Q4_RECIPE_FP32, Variant{Q4_CB_NF4, Q4_CB_DYN4, Q4_RULE_STATE_RTN}, 0, 0};
        return ok();
    }
    if (cfg->recipe == Q4_RECIPE_BLOCK8) {
        // the 8-bit optimizer has one configuration; 4-bit and 8-bit options
        // do not mix ([A] "Requirements and errors")
        if (cfg->m_codebook != Q4_CB_SDYN8 || cfg->v_codebook != Q4_CB_DYN8 || cfg->m_rule != Q4_RULE_STATE_RTN ||
            cfg->v_rule != Q4_RULE_STATE_RTN || cfg->eden != 0)
            return fail(Q4_ERR_CONFLICT, "the 8-bit recipe takes SDyn8 m, Dyn8 v, State-RTN and no EDEN");
        *r = Resolved{Q4_RECIPE_BLOCK8, Variant{Q4_CB_SDYN8, Q4_CB_DYN8, Q4_RULE_STATE_RTN}, 0, 0};
        return ok();
    }
    if (cfg->m_codebook < 0 || cfg->m_codebook > Q4_CB_DYN8 || cfg->v_codebook < 0 || cfg->v_codebook > Q4_CB_DYN8)
        return fail(Q4_ERR_INVALID_ARG, "unknown codebook");
    if (cfg->m_codebook >= Q4_CB_SDYN8 || cfg->v_codebook >= Q4_CB_SDYN8)
        return fail(Q4_ERR_CONFLICT, "8-bit codebooks belong to Q4_RECIPE_BLOCK8 only");
    if (cfg->m_rule < 0 || cfg->m_rule > Q4_RULE_UPDATE_SR || cfg->v_rule < 0 || cfg->v_rule > Q4_RULE_UPDATE_SR)
        return fail(Q4_ERR_INVALID_ARG, "unknown rounding rule");
    if (cfg->eden != 0 && cfg->eden != 1) return fail(Q4_ERR_INVALID_ARG, "eden must be 0 or 1");
    if (cfg->recipe != Q4_RECIPE_CUSTOM) {
        q4_config d;
        q4adamw_default_config(cfg->recipe, &d);
        const bool eden_free = cfg->recipe == Q4_RECIPE_FACTORED;
        if (cfg->m_codebook != d.m_codebook || cfg->v_codebook != d.v_codebook || cfg->m_rule != d.m_rule ||
            cfg->v_rule != d.v_rule || (!eden_free && cfg->eden != d.eden))
            return fail(Q4_ERR_CONFLICT, "recipe %d fixes its codebooks and rules; use Q4_RECIPE_CUSTOM to change them",
                        cfg->recipe);
    }
    if (cfg->m_codebook != Q4_CB_NF4 && cfg->m_codebook != Q4_CB_SDYN4)
        return fail(Q4_ERR_CONFLICT, "the first moment needs a signed codebook (NF4 or SDyn4)");
    if (cfg->v_codebook == Q4_CB_NF4 || cfg->v_codebook == Q4_CB_SDYN4)
        return fail(Q4_ERR_CONFLICT, "the second moment needs an unsigned codebook (Dyn4, Dyn4-NZ, Lin4-NZ)");
    if (cfg->m_rule != Q4_RULE_STATE_RTN && cfg->m_rule != Q4_RULE_STATE_SR)
        return fail(Q4_ERR_CONFLICT, "the first moment rounds in state space (STATE_RTN or STATE_SR)");
    const Variant v{cfg->m_codebook, cfg->v_codebook, cfg->v_rule};
    if (!variant_supported(v))
        return fail(Q4_ERR_CONFLICT, "unsupported combination m_codebook=%d v_codebook=%d v_rule=%d", v.mcb, v.vcb,
                    v.vrule);
    *r = Resolved{cfg->recipe, v, cfg->m_rule == Q4_RULE_STATE_SR ? 1 : 0, cfg->eden};
    return ok();
}

bool finite(float x) { return std::isfinite(x); }

q4_status check_hp(const q4_hparams* hp) {
    if (!hp) return fail(Q4_ERR_INVALID_ARG, "hparams is NULL");
    if (!finite(hp->lr) || !finite(hp->beta1) || !finite(hp->beta2) || !finite(hp->eps) ||
        !finite(hp->weight_decay) || !finite(hp->eps_sr))
        return fail(Q4_ERR_INVALID_ARG, "non-finite hyper-parameter");
    if (hp->beta1 < 0.0f || hp->beta1 >= 1.0f || hp->beta2 < 0.0f || hp->beta2 >= 1.0f)
        return fail(Q4_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
    if (!(hp->eps > 0.0f)) return fail(Q4_ERR_INVALID_ARG, "eps must be > 0");
    if (hp->step == 0) return fail(Q4_ERR_INVALID_ARG, "step is 1-based (got 0)");
    if (!finite(hp->max_grad_norm) || hp->max_grad_norm < 0.0f)
        return fail(Q4_ERR_INVALID_ARG, "max_grad_norm must be finite and >= 0");
    return ok();
}

int kind_of(const Resolved& r, const q4_tensor& t) {
    if (r.recipe == Q4_RECIPE_FP32) return KIND_FP32;
    if (r.recipe == Q4_RECIPE_BLOCK8) return KIND_BYTE8;
    if (r.recipe == Q4_RECIPE_FACTORED && t.ndim >= 2) return KIND_FACTORED;
    return KIND_PACKED;
}

q4_status check_tensors(const Resolved& r, const q4_tensor* t, int32_t n, bool need_param_grad) {
    if (n <= 0) return fail(Q4_ERR_SHAPE, "n_tensors must be >= 1 (got %d)", n);
    if (!t) return fail(Q4_ERR_INVALID_ARG, "tensor list is NULL");
    for (int32_t i = 0; i < n; ++i) {
        const q4_tensor& x = t[i];
        if (x.ndim < 1 || x.ndim > Q4ADAMW_MAX_NDIM)
            return fail(Q4_ERR_SHAPE, "tensor %d: ndim %d outside [1, 8]", i, x.ndim);
        int64_t prod = 1;
        for (int d = 0; d < x.ndim; ++d) {
            if (x.shape[d] < 0) return fail(Q4_ERR_SHAPE, "tensor %d: negative extent", i);
            if (x.shape[d] != 0 && prod > kMaxNumel / x.shape[d]) return fail(Q4_ERR_SHAPE, "tensor %d: too large", i);
            prod *= x.shape[d];
        }
        if (prod != x.numel)
            return fail(Q4_ERR_SHAPE, "tensor %d: numel %lld != product of shape %lld", i, (long long)x.numel,
                        (long long)prod);
        if (x.numel >= kMaxNumel) return fail(Q4_ERR_SHAPE, "tensor %d: numel must be < 2^34", i);
        if (x.elem_offset < 0 || x.elem_offset % kChunkElems != 0 || x.elem_offset >= kMaxNumel - x.numel)
            return fail(Q4_ERR_SHAPE, "tensor %d: elem_offset %lld must be a multiple of 512 in [0, 2^34 - numel)", i,
                        (long long)x.elem_offset);
        if (x.numel == 0) continue;
        const int kind = kind_of(r, x);
        if (kind == KIND_FACTORED && (x.numel / x.shape[0]) >= (int64_t(1) << 31))
            return fail(Q4_ERR_SHAPE, "tensor %d: factored matrix needs numel/shape[0] < 2^31", i);
        if (kind == KIND_FACTORED && x.elem_offset != 0)
            return fail(Q4_ERR_SHAPE, "tensor %d: a factored matrix cannot be a shard (elem_offset must be 0)", i);
        struct P { const void* p; const char* name; };
        std::vector<P> need;
        if (need_param_grad) {
            need.push_back({x.param, "param"});
            need.push_back({x.grad, "grad"});
        }
        if (kind == KIND_FP32) {
            need.push_back({x.m_fp32, "m_fp32"});
            need.push_back({x.v_fp32, "v_fp32"});
        } else {
            need.push_back({x.m_codes, "m_codes"});
            need.push_back({x.m_scales, "m_scales"});
            if (kind == KIND_FACTORED) {
                need.push_back({x.v_row, "v_row"});
                need.push_back({x.v_col, "v_col"});
            } else {
                need.push_back({x.v_codes, "v_codes"});
                need.push_back({x.v_scales, "v_scales"});
            }
        }
        for (const P& p : need) {
            if (!p.p) return fail(Q4_ERR_INVALID_ARG, "tensor %d: %s is NULL", i, p.name);
            if (!aligned16(p.p)) return fail(Q4_ERR_ALIGNMENT, "tensor %d: %s is not 16-byte aligned", i, p.name);
        }
    }
    return ok();
}

// Is `p` device memory of the current device?
q4_status check_device_ptr(const void* p, int dev, int i, const char* name) {
    if (!p) return Q4_OK;
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(Q4_ERR_DEVICE, "tensor %d: %s is not a HIP device pointer", i, name);
    }
    if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
        return fail(Q4_ERR_DEVICE, "tensor %d: %s is not device memory", i, name);
    if (a.device != dev) return fail(Q4_ERR_DEVICE, "tensor %d: %s lives on device %d, current is %d", i, name,
                                     a.device, dev);
    return Q4_OK;
}

// A usable gfx950 device must be current.
q4_status check_device(int* dev_out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(Q4_ERR_DEVICE, "no HIP device available");
    }
    static std::mutex mu;
    static int known[64] = {0};  // 0 unknown, 1 ok, -1 not gfx950
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 0 || dev >= 64) return fail(Q4_ERR_DEVICE, "device index %d out of range", dev);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(Q4_ERR_DEVICE, "cannot query device %d", dev);
        }
        known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    if (known[dev] < 0) return fail(Q4_ERR_DEVICE, "device %d is not a gfx950 (MI355X) GPU", dev);
    *dev_out = dev;
    return Q4_OK;
}

q4_status check_all_pointers(const q4_tensor* t, int32_t n) {
    int dev = 0;
    q4_status s = check_device(&dev);
    if (s != Q4_OK) return s;
    for (int32_t i = 0; i < n; ++i) {
        const q4_tensor& x = t[i];
        const void* ps[] = {x.param, x.grad, x.m_codes, x.m_scales, x.v_codes, x.v_scales, x.v_row, x.v_col,
                            x.m_fp32, x.v_fp32};
        const char* nm[] = {"param", "grad", "m_codes", "m_scales", "v_codes", "v_scales", "v_row", "v_col",
                            "m_fp32", "v_fp32"};
        for (int k = 0; k < 10; ++k) {
            s = check_device_ptr(ps[k], dev, i, nm[k]);
            if (s != Q4_OK) return s;
        }
    }
    return Q4_OK;
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout of a step.

struct Plan {
    size_t off_tab, off_chunks, off_mats, off_tab1, off_chunks1, off_schunks, off_inv, off_prow, off_pcol, off_pmean,
        off_sqpart, total;
    int64_t total_chunks = 0;
    // the quantized steps' prefix: each tensor starts at a multiple of
    // kStepAlignChunks (the chunks between only align the next tensor)
    std::vector<int64_t> schunks;
    int64_t total_schunks = 0;
    int n_mats = 0;
    int64_t total_tiles = 0, total_rgroups = 0, total_cgroups = 0;
    std::vector<DevTensor> tab;
    std::vector<int64_t> chunks;
    std::vector<DevMatrix> mats;
    // with matrices: the other tensors alone and their chunk prefix, for
    // the chunk-order pass that runs beside the tile kernel
    std::vector<DevTensor> tab1;
    std::vector<int64_t> chunks1;
    int64_t total_chunks1 = 0;
};

void plan_layout(const Resolved& r, const q4_tensor* t, int32_t n, Plan& P, uint8_t* ws) {
    P.tab.assign(n, DevTensor{});
    P.chunks.assign(n + 1, 0);
    P.schunks.assign(n + 1, 0);
    P.total_schunks = 0;
    P.mats.clear();
    int64_t prow = 0, pcol = 0, pmean = 0;
    for (int32_t i = 0; i < n; ++i) {
        const q4_tensor& x = t[i];
        DevTensor& d = P.tab[i];
        d.param = x.param;
        d.grad = x.grad;
        d.m_codes = x.m_codes;
        d.m_scales = x.m_scales;
        d.v_codes = x.v_codes;
        d.v_scales = x.v_scales;
        d.v_row = x.v_row;
        d.v_col = x.v_col;
        d.m32 = x.m_fp32;
        d.v32 = x.v_fp32;
        d.numel = x.numel;
        d.kind = kind_of(r, x);
        d.cols = (d.kind == KIND_FACTORED && x.numel > 0) ? x.numel / x.shape[0] : 0;
        d.tensor_id = x.tensor_id;
        d.flags = x.flags;
        d.ctr_base = (uint32_t)((uint64_t)x.elem_offset >> 2);
        d.chunk_begin = P.total_chunks;
        P.chunks[i] = P.total_chunks;
        const int64_t nch = (x.numel + kChunkElems - 1) / kChunkElems;
        P.total_chunks += nch;
        P.schunks[i] = P.total_schunks;
        P.total_schunks += (nch + kStepAlignChunks - 1) / kStepAlignChunks * kStepAlignChunks;
        if (d.kind == KIND_FACTORED && x.numel > 0) {
            DevMatrix m{};
            m.grad = x.grad;
            m.R = x.v_row;
            m.C = x.v_col;
            m.rows = x.shape[0];
            m.cols = d.cols;
            m.n_ctiles = (m.cols + kTileCols - 1) / kTileCols;
            m.n_bands = (m.rows + kBandRows - 1) / kBandRows;
            m.tile_begin = P.total_tiles;
            m.flat_off = d.chunk_begin * kChunkElems;
            P.total_tiles += m.n_ctiles * m.n_bands;
            m.n_rgroups = (m.rows + kGroup - 1) / kGroup;
            m.rgroup_begin = P.total_rgroups;
            P.total_rgroups += m.n_rgroups;
            m.n_cgroups = (m.cols + kColGroup - 1) / kColGroup;
            m.cgroup_begin = P.total_cgroups;
            P.total_cgroups += m.n_cgroups;
            // offsets (in doubles) filled into pointers below
            m.part_row = reinterpret_cast<double*>(prow);
            m.part_col = reinterpret_cast<double*>(pcol);
            m.part_mean = reinterpret_cast<double*>(pmean);
            prow += m.n_ctiles * m.rows;
            pcol += m.n_bands * m.cols;
            pmean += m.n_rgroups;
            d.inv_meanR = reinterpret_cast<const float*>((intptr_t)P.mats.size());
            P.mats.push_back(m);
        }
    }
    P.chunks[n] = P.total_chunks;
    P.schunks[n] = P.total_schunks;
    P.n_mats = (int)P.mats.size();
    P.tab1.clear();
    P.chunks1.clear();
    P.total_chunks1 = 0;
    if (P.n_mats > 0) {
        for (int32_t i = 0; i < n; ++i) {
            if (P.tab[i].kind == KIND_FACTORED && P.tab[i].numel > 0) continue;
            P.chunks1.push_back(P.total_chunks1);
            P.tab1.push_back(P.tab[i]);  // keeps its chunk_begin in the full prefix (the flat offset)
            P.total_chunks1 += P.chunks[i + 1] - P.chunks[i];
        }
        P.chunks1.push_back(P.total_chunks1);
    }
    size_t o = kWsOffTable;
    P.off_tab = o;       o = round256(o + sizeof(DevTensor) * n);
    P.off_chunks = o;    o = round256(o + sizeof(int64_t) * (n + 1));
    P.off_mats = o;      o = round256(o + sizeof(DevMatrix) * P.mats.size());
    P.off_tab1 = o;      o = round256(o + sizeof(DevTensor) * P.tab1.size());
    P.off_chunks1 = o;   o = round256(o + sizeof(int64_t) * P.chunks1.size());
    P.off_schunks = o;   o = round256(o + sizeof(int64_t) * (n + 1));
    P.off_inv = o;       o = round256(o + sizeof(float) * P.mats.size());
    P.off_prow = o;      o = round256(o + sizeof(double) * prow);
    P.off_pcol = o;      o = round256(o + sizeof(double) * pcol);
    P.off_pmean = o;     o = round256(o + sizeof(double) * pmean);
    // the chunk pass runs over all tensors, or over the non-matrix ones when
    // the tile kernel takes the matrices: room for the larger launch
    const int64_t acc_groups = std::max(acc_launch(P.total_chunks).groups, acc_launch(P.total_chunks1).groups);
    P.off_sqpart = o;    o = round256(o + sizeof(double) * (size_t)(acc_groups + P.total_tiles + kSqStageGroups));
    P.total = o;
    if (ws) {  // resolve offsets into device addresses
        for (DevMatrix& m : P.mats) {
            m.part_row = reinterpret_cast<double*>(ws + P.off_prow) + reinterpret_cast<intptr_t>(m.part_row);
            m.part_col = reinterpret_cast<double*>(ws + P.off_pcol) + reinterpret_cast<intptr_t>(m.part_col);
            m.part_mean = reinterpret_cast<double*>(ws + P.off_pmean) + reinterpret_cast<intptr_t>(m.part_mean);
        }
        for (size_t k = 0; k < P.mats.size(); ++k)
            P.mats[k].inv_meanR = reinterpret_cast<float*>(ws + P.off_inv) + k;
        for (DevTensor& d : P.tab)
            if (d.kind == KIND_FACTORED && d.numel > 0)
                d.inv_meanR = reinterpret_cast<float*>(ws + P.off_inv) + reinterpret_cast<intptr_t>(d.inv_meanR);
    }
}

void scalars_of(const q4_hparams* hp, float out[5]) {
    const double t = (double)hp->step;
    const double bc1 = 1.0 - std::pow((double)hp->beta1, t);
    const double bc2 = 1.0 - std::pow((double)hp->beta2, t);
    out[0] = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
    out[1] = (float)((double)hp->lr / bc1);
    out[2] = (float)(1.0 / std::sqrt(bc2));
    out[3] = 1.0f - hp->beta1;
    out[4] = 1.0f - hp->beta2;
}

int codebook_size(int cb) { return cb >= Q4_CB_SDYN8 ? 256 : 16; }

int zero_code(int cb) {
    float L[256];
    codebook_table(cb, L);
    for (int c = 0; c < codebook_size(cb); ++c)
        if (L[c] == 0.0f) return c;
    return 0;  // zero-excluding maps: the floor code, decoded with scale 0
}

q4_status hip_fail(hipError_t e, const char* what) {
    return fail(Q4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Tensor table, chunk prefix and matrix table form one contiguous upload.
// From pageable host memory HIP performs the copy synchronously, so the
// temporary source may go away on return; the cost (a host wait for the
// stream) is why callers that pass the same tensor list again set
// Q4_HP_REUSE_TABLE / Q4_ACC_REUSE_TABLE.  A stream under graph capture
// would record the copy with a pointer to that temporary, which is gone by
// the time the graph replays, so the upload is refused there: a captured
// call must reuse a table that an eager call left in the workspace.
q4_status upload_tables(const Plan& P, int32_t n, uint8_t* wsb, hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
        (void)hipGetLastError();
        cs = hipStreamCaptureStatusNone;  // the copy below reports whatever is wrong with the stream
    }
    if (cs != hipStreamCaptureStatusNone)
        return fail(Q4_ERR_INVALID_ARG,
                    "the stream is capturing a graph: the tensor table upload cannot be captured; run one eager "
                    "call first and capture with Q4_HP_REUSE_TABLE / Q4_ACC_REUSE_TABLE");
    const size_t upload = P.off_inv - P.off_tab;
    std::vector<uint8_t> host(upload, 0);
    std::memcpy(host.data(), P.tab.data(), sizeof(DevTensor) * n);
    std::memcpy(host.data() + (P.off_chunks - P.off_tab), P.chunks.data(), sizeof(int64_t) * (n + 1));
    if (!P.mats.empty())
        std::memcpy(host.data() + (P.off_mats - P.off_tab), P.mats.data(), sizeof(DevMatrix) * P.mats.size());
    if (!P.tab1.empty())
        std::memcpy(host.data() + (P.off_tab1 - P.off_tab), P.tab1.data(), sizeof(DevTensor) * P.tab1.size());
    if (!P.chunks1.empty())
        std::memcpy(host.data() + (P.off_chunks1 - P.off_tab), P.chunks1.data(), sizeof(int64_t) * P.chunks1.size());
    std::memcpy(host.data() + (P.off_schunks - P.off_tab), P.schunks.data(), sizeof(int64_t) * (n + 1));
    const hipError_t e = hipMemcpyAsync(wsb + P.off_tab, host.data(), upload, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "tensor table upload");
    return Q4_OK;
}

// Common checks and layout of the calls that take a workspace.
q4_status prepare(const q4_config* cfg, const q4_tensor* t, int32_t n, bool need_param, void* ws, size_t ws_bytes,
                  Resolved& r, Plan& P) {
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if ((s = check_tensors(r, t, n, need_param)) != Q4_OK) return s;
    int dev = 0;
    if ((s = check_device(&dev)) != Q4_OK) return s;
    if (!ws) return fail(Q4_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned16(ws)) return fail(Q4_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    plan_layout(r, t, n, P, reinterpret_cast<uint8_t*>(ws));
    if (ws_bytes < P.total)
        return fail(Q4_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", ws_bytes, P.total);
    return Q4_OK;
}

}  // namespace

extern "C" {

uint32_t q4adamw_abi_version(void) { return Q4ADAMW_ABI_VERSION; }

const char* q4adamw_status_string(q4_status s) {
    switch (s) {
    case Q4_OK: return "ok";
    case Q4_ERR_INVALID_ARG: return "invalid argument";
    case Q4_ERR_SHAPE: return "bad shape";
    case Q4_ERR_ALIGNMENT: return "misaligned pointer";
    case Q4_ERR_CONFLICT: return "conflicting options";
    case Q4_ERR_STATE_FORMAT: return "incompatible state format";
    case Q4_ERR_DEVICE: return "device error";
    case Q4_ERR_WORKSPACE: return "workspace too small";
    case Q4_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* q4adamw_last_error(void) { return g_last_error.c_str(); }

q4_status q4adamw_default_config(int32_t recipe, q4_config* cfg) {
    if (!cfg) return fail(Q4_ERR_INVALID_ARG, "config is NULL");
    q4_config c{};
    c.abi_version = Q4ADAMW_ABI_VERSION;
    c.recipe = recipe;
    c.block = Q4ADAMW_BLOCK;
    c.m_codebook = Q4_CB_NF4;
    c.m_rule = Q4_RULE_STATE_RTN;
    switch (recipe) {
    case Q4_RECIPE_ZIP_SR: c.v_codebook = Q4_CB_DYN4; c.v_rule = Q4_RULE_UPDATE_SR; c.eden = 0; break;
    case Q4_RECIPE_ZE_EDEN: c.v_codebook = Q4_CB_DYN4_NZ; c.v_rule = Q4_RULE_STATE_RTN; c.eden = 1; break;
    case Q4_RECIPE_FACTORED: c.v_codebook = Q4_CB_DYN4_NZ; c.v_rule = Q4_RULE_STATE_RTN; c.eden = 0; break;
    case Q4_RECIPE_FP32: c.v_codebook = Q4_CB_DYN4; c.v_rule = Q4_RULE_STATE_RTN; c.eden = 0; break;
    case Q4_RECIPE_CUSTOM: c.v_codebook = Q4_CB_DYN4; c.v_rule = Q4_RULE_UPDATE_SR; c.eden = 0; break;
    case Q4_RECIPE_BLOCK8:
        c.m_codebook = Q4_CB_SDYN8; c.v_codebook = Q4_CB_DYN8; c.v_rule = Q4_RULE_STATE_RTN; c.eden = 0; break;
    default: return fail(Q4_ERR_INVALID_ARG, "unknown recipe %d", recipe);
    }
    *cfg = c;
    return ok();
}

q4_status q4adamw_validate(const q4_config* cfg, const q4_hparams* hp, const q4_tensor* t, int32_t n) {
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if (hp && (s = check_hp(hp)) != Q4_OK) return s;
    return check_tensors(r, t, n, true);
}

q4_status q4adamw_workspace_bytes(const q4_config* cfg, const q4_tensor* t, int32_t n, size_t* bytes) {
    if (!bytes) return fail(Q4_ERR_INVALID_ARG, "bytes is NULL");
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if (n <= 0) return fail(Q4_ERR_SHAPE, "n_tensors must be >= 1");
    if (!t) return fail(Q4_ERR_INVALID_ARG, "tensor list is NULL");
    Plan P;
    plan_layout(r, t, n, P, nullptr);
    *bytes = P.total;
    return ok();
}

q4_status q4adamw_state_bytes(const q4_config* cfg, const q4_tensor* t, int32_t n, q4_state_bytes* out) {
    if (!out) return fail(Q4_ERR_INVALID_ARG, "out is NULL");
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if (n <= 0 || !t) return fail(Q4_ERR_SHAPE, "empty tensor list");
    uint64_t q = 0, meta = 0;
    for (int32_t i = 0; i < n; ++i) {
        const q4_tensor& x = t[i];
        const uint64_t numel = (uint64_t)x.numel;
        const uint64_t nb = (numel + 127) / 128, codes = (numel + 1) / 2;
        const int kind = kind_of(r, x);
        if (kind == KIND_FP32) {
            q += 8 * numel;
        } else if (kind == KIND_BYTE8) {
            q += 2 * numel;
            meta += 8 * nb;
        } else if (kind == KIND_FACTORED && numel > 0) {
            q += codes;
            meta += 4 * nb + 4 * (uint64_t)x.shape[0] + 4 * (numel / (uint64_t)x.shape[0]);
        } else {
            q += 2 * codes;
            meta += 8 * nb;
        }
    }
    out->adam4_quantized_state_bytes = q;
    out->adam4_scale_metadata_bytes = meta;
    out->adam4_total_bytes = q + meta;
    return ok();
}

q4_status q4adamw_make_header(const q4_config* cfg, q4_state_header* out) {
    if (!out) return fail(Q4_ERR_INVALID_ARG, "out is NULL");
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    q4_state_header h{};
    h.magic = Q4ADAMW_STATE_MAGIC;
    h.abi_version = Q4ADAMW_ABI_VERSION;
    h.layout_version = Q4ADAMW_LAYOUT_VERSION;
    h.recipe = cfg->recipe;
    h.m_codebook = cfg->m_codebook;
    h.v_codebook = cfg->v_codebook;
    h.m_rule = cfg->m_rule;
    h.v_rule = cfg->v_rule;
    h.eden = cfg->eden;
    h.block = cfg->block;
    *out = h;
    return ok();
}

q4_status q4adamw_check_header(const q4_config* cfg, const q4_state_header* hdr) {
    if (!hdr) return fail(Q4_ERR_INVALID_ARG, "header is NULL");
    q4_state_header mine;
    q4_status s = q4adamw_make_header(cfg, &mine);
    if (s != Q4_OK) return s;
    if (hdr->magic != Q4ADAMW_STATE_MAGIC) return fail(Q4_ERR_STATE_FORMAT, "not a 4-bit AdamW state header");
    if (hdr->layout_version != Q4ADAMW_LAYOUT_VERSION)
        return fail(Q4_ERR_STATE_FORMAT, "state layout version %u, this library reads %u", hdr->layout_version,
                    Q4ADAMW_LAYOUT_VERSION);
    if (hdr->recipe != mine.recipe || hdr->m_codebook != mine.m_codebook || hdr->v_codebook != mine.v_codebook ||
        hdr->m_rule != mine.m_rule || hdr->v_rule != mine.v_rule || hdr->eden != mine.eden ||
        hdr->block != mine.block)
        return fail(Q4_ERR_STATE_FORMAT, "saved state was made with a different recipe, codebook, rule or block");
    return ok();
}

q4_status q4adamw_host_scalars(const q4_hparams* hp, float out[5]) {
    if (!out) return fail(Q4_ERR_INVALID_ARG, "out is NULL");
    q4_status s = check_hp(hp);
    if (s != Q4_OK) return s;
    scalars_of(hp, out);
    return ok();
}

q4_status q4adamw_codebook(int32_t cb, float* out) {
    if (!out) return fail(Q4_ERR_INVALID_ARG, "out is NULL");
    if (cb < 0 || cb > Q4_CB_DYN8) return fail(Q4_ERR_INVALID_ARG, "unknown codebook %d", cb);
    codebook_table(cb, out);
    return ok();
}

q4_status q4adamw_init_state(const q4_config* cfg, const q4_tensor* t, int32_t n, void* stream) {
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if ((s = check_tensors(r, t, n, false)) != Q4_OK) return s;
    if ((s = check_all_pointers(t, n)) != Q4_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const uint8_t zm = (uint8_t)zero_code(r.var.mcb), zv = (uint8_t)zero_code(r.var.vcb);
    for (int32_t i = 0; i < n; ++i) {
        const q4_tensor& x = t[i];
        if (x.numel == 0) continue;
        const size_t numel = (size_t)x.numel, nb = (numel + 127) / 128, codes = (numel + 1) / 2;
        const int kind = kind_of(r, x);
        hipError_t e = hipSuccess;
        auto fill = [&](void* p, size_t bytes, uint8_t val) {
            if (e == hipSuccess && p && bytes) e = launch_fill(p, bytes, val, st);
        };
        if (kind == KIND_FP32) {
            fill(x.m_fp32, 4 * numel, 0);
            fill(x.v_fp32, 4 * numel, 0);
        } else if (kind == KIND_BYTE8) {
            fill(x.m_codes, numel, zm);
            fill(x.v_codes, numel, zv);
            fill(x.m_scales, 4 * nb, 0);
            fill(x.v_scales, 4 * nb, 0);
        } else {
            fill(x.m_codes, codes, (uint8_t)(zm | (zm << 4)));
            if (numel & 1) fill(x.m_codes + codes - 1, 1, zm);
            fill(x.m_scales, 4 * nb, 0);
            if (kind == KIND_FACTORED) {
                fill(x.v_row, 4 * (size_t)x.shape[0], 0);
                fill(x.v_col, 4 * (numel / (size_t)x.shape[0]), 0);
            } else {
                fill(x.v_codes, codes, (uint8_t)(zv | (zv << 4)));
                if (numel & 1) fill(x.v_codes + codes - 1, 1, zv);
                fill(x.v_scales, 4 * nb, 0);
            }
        }
        if (e != hipSuccess) return hip_fail(e, "init_state fill");
    }
    return ok();
}

}  // extern "C"

namespace {

// The step after validation and layout, on workspace `wsb` (planned in P).
q4_status run_step(const Resolved& r, const q4_hparams* hp, int32_t n, const Plan& P, uint8_t* wsb, void* stream) {
    q4_status s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (!(hp->flags & Q4_HP_REUSE_TABLE) && (s = upload_tables(P, n, wsb, st)) != Q4_OK) return s;
    float hs[5];
    scalars_of(hp, hs);
    StepScalars sc{};
    sc.beta1 = hp->beta1;
    sc.beta2 = hp->beta2;
    sc.omb1 = hs[3];
    sc.omb2 = hs[4];
    sc.eps = hp->eps;
    sc.eps_sr = hp->eps_sr > 0.0f ? hp->eps_sr : hp->eps;
    sc.decay = hs[0];
    sc.step_size = hs[1];
    sc.rsbc2 = hs[2];
    sc.step = (uint32_t)hp->step;
    sc.key0 = (uint32_t)hp->seed;
    sc.key1 = (uint32_t)(hp->seed >> 32);
    sc.flags = (hp->lm_head_sr ? SF_LM_HEAD_SR : 0u) | (r.m_sr_all ? SF_M_SR_ALL : 0u) | (r.eden ? SF_EDEN : 0u);
    const float* clip = nullptr;

    const DevTensor* d_tab = reinterpret_cast<const DevTensor*>(wsb + P.off_tab);
    const int64_t* d_chunks = reinterpret_cast<const int64_t*>(wsb + P.off_chunks);
    const int64_t* d_schunks = reinterpret_cast<const int64_t*>(wsb + P.off_schunks);
    const DevMatrix* d_mats = reinterpret_cast<const DevMatrix*>(wsb + P.off_mats);
    bool stats_ready = (hp->flags & Q4_HP_GRAD_STATS) != 0;
    if (hp->max_grad_norm > 0.0f) {
        double* sq = reinterpret_cast<double*>(wsb + kWsOffSq);
        float* clipw = reinterpret_cast<float*>(wsb + kWsOffClip);
        if (!stats_ready) {
            // one read of the gradients: their norm and, for factored
            // matrices, the row/column partials the step needs anyway
            e = launch_grad_pass(GRAD_STATS_ONLY, true, P.n_mats > 0, d_tab, d_chunks, n, P.total_chunks, d_mats,
                                 P.n_mats, P.total_tiles, reinterpret_cast<const DevTensor*>(wsb + P.off_tab1),
                                 reinterpret_cast<const int64_t*>(wsb + P.off_chunks1), (int)P.tab1.size(),
                                 P.total_chunks1, nullptr, reinterpret_cast<double*>(wsb + P.off_sqpart), sq, st);
            if (e != hipSuccess) return hip_fail(e, "gradient statistics launch");
            stats_ready = true;
        }
        e = launch_clip_factor(sq, hp->max_grad_norm, clipw, st);
        if (e != hipSuccess) return hip_fail(e, "clip factor launch");
        sc.flags |= SF_CLIP;
        clip = clipw;
    }
    if (r.recipe == Q4_RECIPE_FP32) {
        e = launch_fp32_step(sc, d_tab, d_chunks, n, P.total_chunks, st);
        if (e != hipSuccess) return hip_fail(e, "fp32 step launch");
        return ok();
    }
    if (r.recipe == Q4_RECIPE_BLOCK8) {
        e = launch_block8_step(sc, d_tab, d_schunks, n, P.total_schunks, st);
        if (e != hipSuccess) return hip_fail(e, "8-bit step launch");
        return ok();
    }
    if (P.n_mats > 0) {
        e = launch_factored_stats(d_mats, P.n_mats, P.total_tiles, P.total_rgroups, P.total_cgroups, sc.beta2, sc.omb2,
                                  clip, stats_ready, st);
        if (e != hipSuccess) return hip_fail(e, "factored statistics launch");
    }
    e = launch_fused_step(r.var, sc, d_tab, d_schunks, n, P.total_schunks, P.n_mats > 0, st);
    if (e != hipSuccess) return hip_fail(e, "fused step launch");
    return ok();
}

}  // namespace

extern "C" {

q4_status q4adamw_step(const q4_config* cfg, const q4_hparams* hp, const q4_tensor* t, int32_t n, void* ws,
                       size_t ws_bytes, void* stream) {
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if ((s = check_hp(hp)) != Q4_OK) return s;
    if ((s = check_tensors(r, t, n, true)) != Q4_OK) return s;
    int dev = 0;
    if ((s = check_device(&dev)) != Q4_OK) return s;
    if ((hp->flags & Q4_HP_CHECK_POINTERS) && (s = check_all_pointers(t, n)) != Q4_OK) return s;
    if (!ws) return fail(Q4_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned16(ws)) return fail(Q4_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    Plan P;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    plan_layout(r, t, n, P, wsb);
    if (ws_bytes < P.total)
        return fail(Q4_ERR_WORKSPACE, "workspace has %zu bytes, the step needs %zu", ws_bytes, P.total);
    return run_step(r, hp, n, P, wsb, stream);
}

q4_status q4adamw_step_noalloc(const q4_config* cfg, const q4_hparams* hp, const q4_tensor* t, int32_t n,
                               void* stream) {
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if ((s = check_hp(hp)) != Q4_OK) return s;
    if ((s = check_tensors(r, t, n, true)) != Q4_OK) return s;
    {
        Plan sizing;
        plan_layout(r, t, n, sizing, nullptr);
        if (sizing.total > kScratchBytes)
            return fail(Q4_ERR_WORKSPACE,
                        "the step needs %zu workspace bytes, the library's static scratch holds %zu; use "
                        "q4adamw_step with a workspace of q4adamw_workspace_bytes",
                        sizing.total, kScratchBytes);
    }
    int dev = 0;
    if ((s = check_device(&dev)) != Q4_OK) return s;
    if ((hp->flags & Q4_HP_CHECK_POINTERS) && (s = check_all_pointers(t, n)) != Q4_OK) return s;
    void* ptr = nullptr;
    const hipError_t e = scratch_address(&ptr);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
    Plan P;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ptr);
    plan_layout(r, t, n, P, wsb);
    return run_step(r, hp, n, P, wsb, stream);
}

q4_status q4adamw_dequant_state(const q4_config* cfg, const q4_tensor* t, float* m_out, float* v_out, void* ws,
                                size_t ws_bytes, void* stream) {
    Resolved r;
    q4_status s = resolve(cfg, &r);
    if (s != Q4_OK) return s;
    if ((s = check_tensors(r, t, 1, false)) != Q4_OK) return s;
    if (!m_out || !v_out) return fail(Q4_ERR_INVALID_ARG, "m_out / v_out is NULL");
    if (!aligned16(m_out) || !aligned16(v_out)) return fail(Q4_ERR_ALIGNMENT, "m_out / v_out not 16-byte aligned");
    if ((s = check_all_pointers(t, 1)) != Q4_OK) return s;
    const q4_tensor& x = *t;
    const int kind = kind_of(r, x);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (x.numel == 0) return ok();
    if (kind == KIND_FP32) {
        hipError_t e = hipMemcpyAsync(m_out, x.m_fp32, 4 * (size_t)x.numel, hipMemcpyDeviceToDevice, st);
        if (e == hipSuccess) e = hipMemcpyAsync(v_out, x.v_fp32, 4 * (size_t)x.numel, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_fail(e, "dequant copy");
        return ok();
    }
    const int64_t rows = x.shape[0];
    const size_t need = kind == KIND_FACTORED ? 256 + round256(8 * (size_t)((rows + kGroup - 1) / kGroup)) : 0;
    if (need && (!ws || ws_bytes < need))
        return fail(Q4_ERR_WORKSPACE, "dequant of a factored matrix needs %zu workspace bytes", need);
    if (ws && !aligned16(ws)) return fail(Q4_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    DevTensor d{};
    d.m_codes = x.m_codes;
    d.m_scales = x.m_scales;
    d.v_codes = x.v_codes;
    d.v_scales = x.v_scales;
    d.v_row = x.v_row;
    d.v_col = x.v_col;
    d.numel = x.numel;
    d.kind = kind;
    d.cols = kind == KIND_FACTORED ? x.numel / rows : 0;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    hipError_t e = launch_dequant(r.var.mcb, r.var.vcb, d, rows, m_out, v_out,
                                  need ? reinterpret_cast<double*>(wsb + 256) : nullptr,
                                  need ? reinterpret_cast<float*>(wsb) : nullptr, st);
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    return ok();
}

q4_status q4adamw_flat_offsets(const q4_tensor* t, int32_t n, int64_t* offsets, int64_t* total) {
    if (!t || !offsets || !total) return fail(Q4_ERR_INVALID_ARG, "tensor list, offsets or total is NULL");
    if (n <= 0) return fail(Q4_ERR_SHAPE, "n_tensors must be >= 1 (got %d)", n);
    int64_t o = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (t[i].numel < 0 || t[i].numel >= kMaxNumel) return fail(Q4_ERR_SHAPE, "tensor %d: bad numel", i);
        offsets[i] = o;
        o += (t[i].numel + kChunkElems - 1) / kChunkElems * kChunkElems;
    }
    *total = o;
    return ok();
}

q4_status q4adamw_accumulate(const q4_config* cfg, const q4_tensor* t, int32_t n, const uint16_t* micro,
                             int32_t flags, void* ws, size_t ws_bytes, void* stream) {
    if (!micro) return fail(Q4_ERR_INVALID_ARG, "micro is NULL");
    if (!aligned16(micro)) return fail(Q4_ERR_ALIGNMENT, "micro is not 16-byte aligned");
    if (flags & ~(Q4_ACC_FIRST | Q4_ACC_LAST | Q4_ACC_REUSE_TABLE))
        return fail(Q4_ERR_INVALID_ARG, "unknown accumulate flags 0x%x", flags);
    Resolved r;
    Plan P;
    q4_status s = prepare(cfg, t, n, true, ws, ws_bytes, r, P);
    if (s != Q4_OK) return s;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!(flags & Q4_ACC_REUSE_TABLE) && (s = upload_tables(P, n, wsb, st)) != Q4_OK) return s;
    const int mode = (flags & Q4_ACC_FIRST) ? GRAD_FIRST : GRAD_ADD;
    const hipError_t e = launch_grad_pass(mode, (flags & Q4_ACC_LAST) != 0, P.n_mats > 0,
                                          reinterpret_cast<const DevTensor*>(wsb + P.off_tab),
                                          reinterpret_cast<const int64_t*>(wsb + P.off_chunks), n, P.total_chunks,
                                          reinterpret_cast<const DevMatrix*>(wsb + P.off_mats), P.n_mats,
                                          P.total_tiles, reinterpret_cast<const DevTensor*>(wsb + P.off_tab1),
                                          reinterpret_cast<const int64_t*>(wsb + P.off_chunks1),
                                          (int)P.tab1.size(), P.total_chunks1, micro,
                                          reinterpret_cast<double*>(wsb + P.off_sqpart),
                                          reinterpret_cast<double*>(wsb + kWsOffSq), st);
    if (e != hipSuccess) return hip_fail(e, "accumulate launch");
    return ok();
}

q4_status q4adamw_grad_stats(const q4_config* cfg, const q4_tensor* t, int32_t n, void* ws, size_t ws_bytes,
                             void* stream) {
    Resolved r;
    Plan P;
    q4_status s = prepare(cfg, t, n, true, ws, ws_bytes, r, P);
    if (s != Q4_OK) return s;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if ((s = upload_tables(P, n, wsb, st)) != Q4_OK) return s;
    const hipError_t e = launch_grad_pass(GRAD_STATS_ONLY, true, P.n_mats > 0,
                                          reinterpret_cast<const DevTensor*>(wsb + P.off_tab),
                                          reinterpret_cast<const int64_t*>(wsb + P.off_chunks), n, P.total_chunks,
                                          reinterpret_cast<const DevMatrix*>(wsb + P.off_mats), P.n_mats,
                                          P.total_tiles, reinterpret_cast<const DevTensor*>(wsb + P.off_tab1),
                                          reinterpret_cast<const int64_t*>(wsb + P.off_chunks1),
                                          (int)P.tab1.size(), P.total_chunks1, nullptr,
                                          reinterpret_cast<double*>(wsb + P.off_sqpart),
                                          reinterpret_cast<double*>(wsb + kWsOffSq), st);
    if (e != hipSuccess) return hip_fail(e, "gradient statistics launch");
    return ok();
}

q4_status q4adamw_grad_norm(const void* ws, size_t ws_bytes, double* norm, void* stream) {
    if (!ws || !norm) return fail(Q4_ERR_INVALID_ARG, "workspace or norm is NULL");
    if (ws_bytes < 256) return fail(Q4_ERR_WORKSPACE, "workspace has %zu bytes", ws_bytes);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    double sq = 0.0;
    hipError_t e = hipMemcpyAsync(&sq, reinterpret_cast<const uint8_t*>(ws) + kWsOffSq, sizeof(double),
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "gradient norm copy");
    *norm = std::sqrt(sq);
    return ok();
}

}  // extern "C"
