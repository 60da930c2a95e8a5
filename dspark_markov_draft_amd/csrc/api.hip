// The extern "C" entry points of libdspark.so: argument validation on the host (before any
// HIP call, so that invalid calls are rejected with no device and no side effect), device
// checks, and dispatch to the kernels' launchers.
#include <string.h>

#include <mutex>

#include "internal.hpp"

namespace dspark {

DebugKnobs& debug_knobs() {
    static DebugKnobs knobs;
    return knobs;
}

static DeviceInfo g_dev_cache[64];

int current_device_info(DeviceInfo* info) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return DSPARK_ERR_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DSPARK_ERR_NO_DEVICE;
    DeviceInfo& c = g_dev_cache[dev];
    if (c.device != dev) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSPARK_ERR_NO_DEVICE;
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return DSPARK_ERR_NO_DEVICE;
        c.cus = prop.multiProcessorCount;
        c.max_lds = prop.sharedMemPerBlock;
        if (prop.maxSharedMemoryPerMultiProcessor > c.max_lds)
            c.max_lds = prop.maxSharedMemoryPerMultiProcessor;
        c.cooperative = prop.cooperativeLaunch != 0;
        c.device = dev;
    }
    *info = c;
    return DSPARK_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape checks shared by the walks. Non-positive sizes are invalid arguments; sizes above the
// supported envelope (vLLM PR #62958, Details) are unsupported.
static int check_walk_shape(int64_t bs, int64_t T, int64_t V, int64_t rank, int w1_dtype) {
    if (bs < 1 || T < 1 || V < 1 || rank < 1) return DSPARK_ERR_INVALID_ARG;
    if (rank != DSPARK_RANK) return DSPARK_ERR_UNSUPPORTED;
    if (bs > DSPARK_MAX_BS || T > DSPARK_MAX_STEPS || V > DSPARK_MAX_V) return DSPARK_ERR_UNSUPPORTED;
    if (w1_dtype != DSPARK_F32 && w1_dtype != DSPARK_BF16 && w1_dtype != DSPARK_F16)
        return DSPARK_ERR_UNSUPPORTED;
    return DSPARK_OK;
}

static int check_walk_common(const int8_t* q, const float* s, const void* w1, const float* base,
                             const int32_t* start, const int32_t* tokens, void* ws,
                             size_t ws_bytes, int64_t bs, int64_t T, int64_t V, int64_t k) {
    if (!q || !s || !w1 || !base || !start || !tokens || !ws) return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(w1) || !aligned4(s) || !aligned4(base) || !aligned4(start) ||
        !aligned4(tokens) || !aligned16(ws))
        return DSPARK_ERR_INVALID_ARG;
    if (ws_bytes < dspark_walk_workspace_bytes(bs, T, V, k)) return DSPARK_ERR_WORKSPACE;
    return DSPARK_OK;
}

// ---- library-held scratch of the no-allocation greedy walk ---------------------------------
// For callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation): dspark_walk_greedy_noalloc keeps the walk's
// workspace in this file-scope device array instead of a caller workspace. It is sized for the
// largest dense walk (64 requests, 16 steps); every GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` names a host-side stand-in, so its device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever handed to kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES =
    (WS_SLOTS + (size_t)DSPARK_MAX_STEPS * MAX_WORKGROUPS * DSPARK_MAX_BS * 8 + WS_ALIGN - 1) /
    WS_ALIGN * WS_ALIGN;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

static void* g_scratch_ptr[64];
static std::mutex g_scratch_mutex;

// The device address of this device's copy of `scratch` (looked up on the first call per
// device); NULL if the lookup failed.
static void* scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Zeroes n16 16-byte words from p (the part of the scratch a call uses; a kernel rather than a
// memset node, so that the call stays safe to capture into a graph).
__global__ void clear_scratch_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace dspark

using namespace dspark;

extern "C" {

const char* dspark_status_string(int status) {
    switch (status) {
        case DSPARK_OK: return "ok";
        case DSPARK_ERR_INVALID_ARG: return "invalid argument (null, non-positive size or misaligned pointer)";
        case DSPARK_ERR_UNSUPPORTED: return "unsupported (outside rank 256, T <= 16, bs <= 64, V <= 270336, k <= 2048, f32/bf16/f16)";
        case DSPARK_ERR_WORKSPACE: return "workspace missing or too small";
        case DSPARK_ERR_NO_DEVICE: return "no gfx950 HIP device";
        case DSPARK_ERR_LAUNCH: return "HIP launch or copy failed";
        case DSPARK_ERR_NONFINITE: return "W2 holds a NaN or infinity";
        case DSPARK_ERR_TIMEOUT: return "grid-wide wait hit its time bound";
        default: return "unknown status";
    }
}

int dspark_quantize_w2(const void* w2, int w2_dtype, int64_t V, int64_t rank, int8_t* w2_q,
                       float* w2_scale, void* stream) {
    if (!w2 || !w2_q || !w2_scale) return DSPARK_ERR_INVALID_ARG;
    if (V < 1 || rank < 1) return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(w2) || !aligned16(w2_q) || !aligned4(w2_scale)) return DSPARK_ERR_INVALID_ARG;
    if (rank != DSPARK_RANK) return DSPARK_ERR_UNSUPPORTED;
    if (w2_dtype != DSPARK_F32 && w2_dtype != DSPARK_BF16 && w2_dtype != DSPARK_F16)
        return DSPARK_ERR_UNSUPPORTED;
    if (V > (int64_t)1 << 31) return DSPARK_ERR_UNSUPPORTED;
    DeviceInfo dev;
    const int st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    return launch_quantize(w2, w2_dtype, V, w2_q, w2_scale, static_cast<hipStream_t>(stream));
}

size_t dspark_walk_workspace_bytes(int64_t bs, int64_t T, int64_t V, int64_t k) {
    (void)V;
    if (bs < 1 || T < 1) return WS_SLOTS;
    if (bs > DSPARK_MAX_BS) bs = DSPARK_MAX_BS;
    if (T > DSPARK_MAX_STEPS) T = DSPARK_MAX_STEPS;
    const size_t dense = dense_slot_bytes(bs, T);
    const size_t top = topk_bytes(bs, T, k);
    const size_t n = WS_SLOTS + (dense > top ? dense : top);
    return (n + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN;
}

int dspark_walk_plan_query(int64_t bs, int64_t T, int64_t V, dspark_walk_plan* plan) {
    if (!plan) return DSPARK_ERR_INVALID_ARG;
    const int st = check_walk_shape(bs, T, V, DSPARK_RANK, DSPARK_BF16);
    if (st != DSPARK_OK) return st;
    DeviceInfo dev;
    const int d = current_device_info(&dev);
    if (d != DSPARK_OK) return d;
    return plan_walk(dev, bs, T, V, 0, plan);
}

int dspark_walk_plan_for(int32_t cus, int64_t max_lds, int64_t bs, int64_t T, int64_t V,
                         dspark_walk_plan* plan) {
    if (!plan || cus < 1 || max_lds < 1) return DSPARK_ERR_INVALID_ARG;
    const int st = check_walk_shape(bs, T, V, DSPARK_RANK, DSPARK_BF16);
    if (st != DSPARK_OK) return st;
    DeviceInfo dev;
    dev.device = 0;
    dev.cus = cus;
    dev.max_lds = (size_t)max_lds;
    dev.cooperative = true;
    return plan_walk(dev, bs, T, V, 0, plan);
}

static int dense_walk(const WalkLaunch& a, int64_t rank, size_t ws_bytes, void* stream) {
    int st = check_walk_shape(a.bs, a.T, a.V, rank, a.w1_dtype);
    if (st != DSPARK_OK) return st;
    st = check_walk_common(a.q, a.scale, a.w1, a.base, a.start, a.tokens, a.workspace, ws_bytes,
                           a.bs, a.T, a.V, 0);
    if (st != DSPARK_OK) return st;
    if (a.sample) {
        if (!a.seeds || !a.temps || !a.draft_logits) return DSPARK_ERR_INVALID_ARG;
        if (((uintptr_t)a.seeds & 7u) || ((uintptr_t)a.positions & 7u) || !aligned4(a.temps) ||
            ((uintptr_t)a.draft_logits & 1u))
            return DSPARK_ERR_INVALID_ARG;
    } else if (a.out_logits && !aligned4(a.out_logits)) {
        return DSPARK_ERR_INVALID_ARG;
    }
    DeviceInfo dev;
    st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    dspark_walk_plan plan;
    st = plan_walk(dev, a.bs, a.T, a.V, a.sample, &plan);
    if (st != DSPARK_OK) return st;
    return launch_dense_walk(a, plan, static_cast<hipStream_t>(stream));
}

int dspark_walk_greedy(const int8_t* w2_q, const float* w2_scale, const void* w1, int w1_dtype,
                       const float* base_logits, const int32_t* start_tokens, int64_t bs,
                       int64_t T, int64_t V, int64_t rank, int32_t* draft_tokens,
                       float* out_logits, void* workspace, size_t workspace_bytes, void* stream) {
    WalkLaunch a = {};
    a.q = w2_q;
    a.scale = w2_scale;
    a.w1 = w1;
    a.w1_dtype = w1_dtype;
    a.base = base_logits;
    a.start = start_tokens;
    a.tokens = draft_tokens;
    a.out_logits = out_logits;
    a.workspace = workspace;
    a.sample = 0;
    if (bs > DSPARK_MAX_BS || T > DSPARK_MAX_STEPS || V > DSPARK_MAX_V) {
        return (bs < 1 || T < 1 || V < 1) ? DSPARK_ERR_INVALID_ARG : DSPARK_ERR_UNSUPPORTED;
    }
    a.bs = (int)bs;
    a.T = (int)T;
    a.V = (int)V;
    return dense_walk(a, rank, workspace_bytes, stream);
}

int dspark_walk_greedy_noalloc(const int8_t* w2_q, const float* w2_scale, const void* w1,
                               int w1_dtype, const float* base_logits,
                               const int32_t* start_tokens, int64_t bs, int64_t T, int64_t V,
                               int64_t rank, int32_t* draft_tokens, float* out_logits,
                               uint32_t* error_word, void* stream) {
    if (bs < 1 || T < 1 || V < 1) return DSPARK_ERR_INVALID_ARG;
    if (bs > DSPARK_MAX_BS || T > DSPARK_MAX_STEPS || V > DSPARK_MAX_V) return DSPARK_ERR_UNSUPPORTED;
    const size_t need = dspark_walk_workspace_bytes(bs, T, V, 0);
    if (need > NOALLOC_SCRATCH_BYTES) return DSPARK_ERR_UNSUPPORTED;
    WalkLaunch a = {};
    a.q = w2_q;
    a.scale = w2_scale;
    a.w1 = w1;
    a.w1_dtype = w1_dtype;
    a.base = base_logits;
    a.start = start_tokens;
    a.tokens = draft_tokens;
    a.out_logits = out_logits;
    a.error_word = error_word;
    a.sample = 0;
    a.bs = (int)bs;
    a.T = (int)T;
    a.V = (int)V;
    // every check of the greedy walk, before any device work
    int st = check_walk_shape(bs, T, V, rank, w1_dtype);
    if (st != DSPARK_OK) return st;
    if (!w2_q || !w2_scale || !w1 || !base_logits || !start_tokens || !draft_tokens)
        return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(w2_q) || !aligned16(w1) || !aligned4(w2_scale) || !aligned4(base_logits) ||
        !aligned4(start_tokens) || !aligned4(draft_tokens))
        return DSPARK_ERR_INVALID_ARG;
    if (error_word && !aligned4(error_word)) return DSPARK_ERR_INVALID_ARG;
    if (out_logits && !aligned4(out_logits)) return DSPARK_ERR_INVALID_ARG;
    DeviceInfo dev;
    st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    void* ws = scratch_address(dev.device);
    if (ws == nullptr) return DSPARK_ERR_LAUNCH;
    a.workspace = ws;
    st = check_walk_common(a.q, a.scale, a.w1, a.base, a.start, a.tokens, ws,
                           NOALLOC_SCRATCH_BYTES, bs, T, V, 0);
    if (st != DSPARK_OK) return st;
    dspark_walk_plan plan;
    st = plan_walk(dev, bs, T, V, 0, &plan);
    if (st != DSPARK_OK) return st;
    // the walk needs the words it uses zeroed; one that timed out may have left keys behind
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t n16 = need / 16;
    const size_t blocks = (n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024;
    clear_scratch_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint4*>(ws), n16);
    if (hipGetLastError() != hipSuccess) return DSPARK_ERR_LAUNCH;
    return launch_dense_walk(a, plan, s);
}

int dspark_walk_sample(const int8_t* w2_q, const float* w2_scale, const void* w1, int w1_dtype,
                       const float* base_logits, const int32_t* start_tokens, int64_t bs,
                       int64_t T, int64_t V, int64_t rank, const uint64_t* seeds,
                       const int64_t* positions, const float* temperature,
                       int32_t* draft_tokens, uint16_t* draft_logits, void* workspace,
                       size_t workspace_bytes, void* stream) {
    WalkLaunch a = {};
    a.q = w2_q;
    a.scale = w2_scale;
    a.w1 = w1;
    a.w1_dtype = w1_dtype;
    a.base = base_logits;
    a.start = start_tokens;
    a.tokens = draft_tokens;
    a.draft_logits = draft_logits;
    a.seeds = seeds;
    a.positions = positions;
    a.temps = temperature;
    a.workspace = workspace;
    a.sample = 1;
    if (bs > DSPARK_MAX_BS || T > DSPARK_MAX_STEPS || V > DSPARK_MAX_V) {
        return (bs < 1 || T < 1 || V < 1) ? DSPARK_ERR_INVALID_ARG : DSPARK_ERR_UNSUPPORTED;
    }
    a.bs = (int)bs;
    a.T = (int)T;
    a.V = (int)V;
    return dense_walk(a, rank, workspace_bytes, stream);
}

int dspark_walk_sample_icdf(const int8_t* w2_q, const float* w2_scale, const void* w1,
                            int w1_dtype, const float* base_logits, const int32_t* start_tokens,
                            int64_t bs, int64_t T, int64_t V, int64_t rank,
                            const uint64_t* seeds, const int64_t* positions,
                            const float* temperature, int32_t* draft_tokens,
                            uint16_t* draft_logits, void* workspace, size_t workspace_bytes,
                            void* stream) {
    WalkLaunch a = {};
    a.q = w2_q;
    a.scale = w2_scale;
    a.w1 = w1;
    a.w1_dtype = w1_dtype;
    a.base = base_logits;
    a.start = start_tokens;
    a.tokens = draft_tokens;
    a.draft_logits = draft_logits;
    a.seeds = seeds;
    a.positions = positions;
    a.temps = temperature;
    a.workspace = workspace;
    a.sample = 2;
    if (bs > DSPARK_MAX_BS || T > DSPARK_MAX_STEPS || V > DSPARK_MAX_V) {
        return (bs < 1 || T < 1 || V < 1) ? DSPARK_ERR_INVALID_ARG : DSPARK_ERR_UNSUPPORTED;
    }
    a.bs = (int)bs;
    a.T = (int)T;
    a.V = (int)V;
    return dense_walk(a, rank, workspace_bytes, stream);
}

int dspark_walk_topk(const int8_t* w2_q, const float* w2_scale, const void* w1, int w1_dtype,
                     const float* base_logits, const int32_t* start_tokens, int64_t bs,
                     int64_t T, int64_t V, int64_t rank, int64_t k, int sample,
                     const uint64_t* seeds, const int64_t* positions, const float* temperature,
                     int32_t* draft_tokens, void* draft_logits, void* workspace,
                     size_t workspace_bytes, void* stream) {
    int st = check_walk_shape(bs, T, V, rank, w1_dtype);
    if (st != DSPARK_OK) return st;
    if (k < 1 || k > V) return DSPARK_ERR_INVALID_ARG;
    if (k > DSPARK_MAX_TOPK) return DSPARK_ERR_UNSUPPORTED;
    if (sample != 0 && sample != 1) return DSPARK_ERR_INVALID_ARG;
    st = check_walk_common(w2_q, w2_scale, w1, base_logits, start_tokens, draft_tokens, workspace,
                           workspace_bytes, bs, T, V, k);
    if (st != DSPARK_OK) return st;
    if (sample) {
        if (!seeds || !temperature || !draft_logits) return DSPARK_ERR_INVALID_ARG;
        if (((uintptr_t)seeds & 7u) || ((uintptr_t)positions & 7u) || !aligned4(temperature) ||
            !aligned16(draft_logits))
            return DSPARK_ERR_INVALID_ARG;
    } else if (draft_logits && !aligned16(draft_logits)) {
        return DSPARK_ERR_INVALID_ARG;
    }
    DeviceInfo dev;
    st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    TopkLaunch a = {};
    a.w.q = w2_q;
    a.w.scale = w2_scale;
    a.w.w1 = w1;
    a.w.w1_dtype = w1_dtype;
    a.w.base = base_logits;
    a.w.start = start_tokens;
    a.w.tokens = draft_tokens;
    a.w.seeds = seeds;
    a.w.positions = positions;
    a.w.temps = temperature;
    a.w.workspace = workspace;
    a.w.bs = (int)bs;
    a.w.T = (int)T;
    a.w.V = (int)V;
    a.w.sample = sample;
    if (sample)
        a.w.draft_logits = static_cast<uint16_t*>(draft_logits);
    else
        a.w.out_logits = static_cast<float*>(draft_logits);
    a.k = (int)k;
    return launch_topk_walk(a, static_cast<hipStream_t>(stream));
}

int dspark_w2_prune_bound(const int8_t* w2_q, const float* w2_scale, int64_t V, int64_t rank,
                          float* bound, void* stream) {
    if (!w2_q || !w2_scale || !bound || V < 1 || rank < 1) return DSPARK_ERR_INVALID_ARG;
    if (!aligned16(w2_q) || !aligned4(w2_scale) || !aligned4(bound)) return DSPARK_ERR_INVALID_ARG;
    if (rank != DSPARK_RANK || V > DSPARK_MAX_V) return DSPARK_ERR_UNSUPPORTED;
    DeviceInfo dev;
    const int st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    return launch_w2_bound(w2_q, w2_scale, V, bound, static_cast<hipStream_t>(stream));
}

int dspark_walk_greedy_pruned(const int8_t* w2_q, const float* w2_scale, const void* w1,
                              int w1_dtype, const float* base_logits,
                              const int32_t* start_tokens, int64_t bs, int64_t T, int64_t V,
                              int64_t rank, int64_t k, const float* w2_bound,
                              int32_t* draft_tokens, float* out_logits, int32_t* dense_steps,
                              void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_walk_shape(bs, T, V, rank, w1_dtype);
    if (st != DSPARK_OK) return st;
    if (k < 1 || k > V) return DSPARK_ERR_INVALID_ARG;
    if (k > DSPARK_MAX_TOPK) return DSPARK_ERR_UNSUPPORTED;
    if (!w2_bound || !aligned4(w2_bound)) return DSPARK_ERR_INVALID_ARG;
    st = check_walk_common(w2_q, w2_scale, w1, base_logits, start_tokens, draft_tokens, workspace,
                           workspace_bytes, bs, T, V, k);
    if (st != DSPARK_OK) return st;
    if ((out_logits && !aligned16(out_logits)) || (dense_steps && !aligned4(dense_steps)))
        return DSPARK_ERR_INVALID_ARG;
    DeviceInfo dev;
    st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    TopkLaunch a = {};
    a.w.q = w2_q;
    a.w.scale = w2_scale;
    a.w.w1 = w1;
    a.w.w1_dtype = w1_dtype;
    a.w.base = base_logits;
    a.w.start = start_tokens;
    a.w.tokens = draft_tokens;
    a.w.out_logits = out_logits;
    a.w.workspace = workspace;
    a.w.bs = (int)bs;
    a.w.T = (int)T;
    a.w.V = (int)V;
    a.w.sample = 0;
    a.k = (int)k;
    a.w2_bound = w2_bound;
    a.dense_steps = dense_steps;
    return launch_topk_walk(a, static_cast<hipStream_t>(stream));
}

size_t dspark_verify_workspace_bytes(int64_t bs, int64_t T, int64_t V) {
    if (bs < 1 || T < 1 || V < 1) return WS_ALIGN;
    if (bs > DSPARK_MAX_BS) bs = DSPARK_MAX_BS;
    if (T > DSPARK_MAX_STEPS) T = DSPARK_MAX_STEPS;
    if (V > DSPARK_MAX_V) V = DSPARK_MAX_V;
    return verify_workspace_bytes(bs, T, V);
}

int dspark_verify(const uint16_t* draft_logits, const int32_t* draft_tokens,
                  const float* target_logits, const float* temperature, const float* uniforms,
                  int64_t bs, int64_t T, int64_t V, int mode, int32_t* accepted,
                  int32_t* out_tokens, float* accept_prob, void* workspace,
                  size_t workspace_bytes, void* stream) {
    if (bs < 1 || T < 1 || V < 1) return DSPARK_ERR_INVALID_ARG;
    if (bs > DSPARK_MAX_BS || T > DSPARK_MAX_STEPS || V > DSPARK_MAX_V) return DSPARK_ERR_UNSUPPORTED;
    if (mode != DSPARK_VERIFY_TOKEN && mode != DSPARK_VERIFY_BLOCK) return DSPARK_ERR_INVALID_ARG;
    if (!draft_logits || !draft_tokens || !target_logits || !temperature || !uniforms ||
        !accepted || !out_tokens || !workspace)
        return DSPARK_ERR_INVALID_ARG;
    if (((uintptr_t)draft_logits & 1u) || !aligned4(draft_tokens) || !aligned4(target_logits) ||
        !aligned4(temperature) || !aligned4(uniforms) || !aligned4(accepted) ||
        !aligned4(out_tokens) || (accept_prob && !aligned4(accept_prob)) || !aligned16(workspace))
        return DSPARK_ERR_INVALID_ARG;
    if (workspace_bytes < dspark_verify_workspace_bytes(bs, T, V)) return DSPARK_ERR_WORKSPACE;
    DeviceInfo dev;
    const int st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    VerifyLaunch a;
    a.draft_logits = draft_logits;
    a.draft_tokens = draft_tokens;
    a.target_logits = target_logits;
    a.temperature = temperature;
    a.uniforms = uniforms;
    a.accepted = accepted;
    a.out_tokens = out_tokens;
    a.accept_prob = accept_prob;
    a.workspace = workspace;
    a.bs = (int)bs;
    a.T = (int)T;
    a.V = (int)V;
    a.mode = mode;
    return launch_verify(a, static_cast<hipStream_t>(stream));
}

int dspark_workspace_status(void* workspace, void* stream) {
    if (!workspace || !aligned16(workspace)) return DSPARK_ERR_INVALID_ARG;
    DeviceInfo dev;
    int st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    uint32_t* err = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + WS_ERR);
    if (hipMemcpyAsync(&word, err, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess)
        return DSPARK_ERR_LAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return DSPARK_ERR_LAUNCH;
    if (word != 0) {
        const uint32_t zero = 0;
        if (hipMemcpyAsync(err, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess)
            return DSPARK_ERR_LAUNCH;
        if (hipStreamSynchronize(s) != hipSuccess) return DSPARK_ERR_LAUNCH;
        return -(int)word;
    }
    return DSPARK_OK;
}

int dspark_philox_words(uint64_t seed, uint64_t position, int64_t v0, int64_t n, uint32_t* out,
                        void* stream) {
    if (!out || n < 0 || v0 < 0 || v0 + n > ((int64_t)1 << 32)) return DSPARK_ERR_INVALID_ARG;
    if (!aligned4(out)) return DSPARK_ERR_INVALID_ARG;
    if (n == 0) return DSPARK_OK;
    DeviceInfo dev;
    const int st = current_device_info(&dev);
    if (st != DSPARK_OK) return st;
    return launch_philox_words(seed, position, v0, n, out, static_cast<hipStream_t>(stream));
}

int dspark_debug_set(int key, int64_t value) {
    if (value < 0) return DSPARK_ERR_INVALID_ARG;
    DebugKnobs& k = debug_knobs();
    switch (key) {
        case DSPARK_DEBUG_MAX_WORKGROUPS: k.max_workgroups = (int)value; return DSPARK_OK;
        case DSPARK_DEBUG_SPIN_LIMIT:
            if (value > 0xFFFFFFFFll) return DSPARK_ERR_INVALID_ARG;
            k.spin_ticks = (uint32_t)value;
            return DSPARK_OK;
        case DSPARK_DEBUG_WAIT_UNSET_FLAG: k.wait_unset = (uint32_t)value; return DSPARK_OK;
        case DSPARK_DEBUG_FORCE_PATH:
            if (value != 0 && value != DSPARK_PATH_DOT4 && value != DSPARK_PATH_MFMA &&
                value != DSPARK_PATH_MFMA1)
                return DSPARK_ERR_INVALID_ARG;
            k.force_path = (int)value;
            return DSPARK_OK;
        case DSPARK_DEBUG_KERNEL_TIMING: return set_kernel_timing(value);
        case DSPARK_DEBUG_MFMA_WAVES:
            if (value != 0 && value != 4 && value != 8) return DSPARK_ERR_INVALID_ARG;
            k.mfma_waves = (int)value;
            return DSPARK_OK;
        case DSPARK_DEBUG_TOPK_SPLIT: k.topk_split = value != 0; return DSPARK_OK;
        case DSPARK_DEBUG_STAMPS:
            if (value & 7) return DSPARK_ERR_INVALID_ARG;
            k.stamps = (uintptr_t)value;
            return DSPARK_OK;
        default: return DSPARK_ERR_INVALID_ARG;
    }
}

int dspark_kernel_times(float* us, int max, int* count) {
    if (us == nullptr || count == nullptr || max < 0) return DSPARK_ERR_INVALID_ARG;
    return read_kernel_times(us, max, count);
}

}  // extern "C"
