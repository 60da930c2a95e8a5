// Host-side declarations shared by the translation units of libdspark.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

// Workspace layout of a walk call (bytes from the start of the caller's workspace). A walk
// leaves every word it uses at zero when it exits, so the caller zeroes the workspace once.
constexpr size_t WS_ERR = 0;          // u32 error word (DSPARK_ERR_TIMEOUT / INVALID_ARG)
constexpr size_t WS_ICDF_DONE = 2048; // u64 [256]: inverse-CDF walks' end-of-walk flags
constexpr int RESULT_REPLICAS = 16;   // copies of the result words, read by disjoint workgroups
constexpr size_t WS_RESULT = 4096;    // u64 [8 copies][16 steps][64 requests]: each step's winner
constexpr size_t WS_SLOTS = WS_RESULT + (size_t)RESULT_REPLICAS * 16 * 64 * 8;  // then
                                      // u64 [T][256 workgroups x slot stride]: workgroup keys
constexpr size_t WS_TOPK = WS_SLOTS;  // top-k calls use the same region for candidate lists
constexpr size_t WS_ALIGN = 256;
constexpr int MAX_WORKGROUPS = 256;

// the key region of one step holds 256 x slot_stride(bs) keys, laid out request-major
// ([request][workgroup]; for one or two requests as replicas of that)
inline int slot_stride(int64_t bs) { return (int)((bs + 15) / 16 * 16); }
inline size_t dense_slot_bytes(int64_t bs, int64_t T) {
    return (size_t)T * MAX_WORKGROUPS * (size_t)slot_stride(bs) * 8;
}
inline size_t topk_bytes(int64_t bs, int64_t T, int64_t k) {
    return k > 0 ? (size_t)bs * (size_t)T * ((size_t)k + 1) * 4 : 0;
}

// Process-wide test hooks (dspark_debug_set).
struct DebugKnobs {
    int max_workgroups = 0;
    uint32_t spin_ticks = 0;
    uint32_t wait_unset = 0;
    uintptr_t stamps = 0;
    int force_path = 0;
    int mfma_waves = 0;
    int topk_split = 0;
};
DebugKnobs& debug_knobs();

struct DeviceInfo {
    int device = -1;
    int cus = 0;
    size_t max_lds = 0;
    bool cooperative = false;
};
// Query (cached per device) of the current device; returns a dspark_status.
int current_device_info(DeviceInfo* info);

int plan_walk(const DeviceInfo& dev, int64_t bs, int64_t T, int64_t V, int sample,
              dspark_walk_plan* plan);

struct WalkLaunch {
    const int8_t* q;
    const float* scale;
    const void* w1;
    int w1_dtype;
    const float* base;
    const int32_t* start;
    int32_t* tokens;
    float* out_logits;        // greedy, optional
    uint16_t* draft_logits;   // sample, required
    const uint64_t* seeds;
    const int64_t* positions;
    const float* temps;
    void* workspace;
    uint32_t* error_word;     // where errors are recorded; NULL: the workspace's error word
    int bs, T, V;
    int sample;               // 0 greedy, 1 Gumbel-max, 2 inverse CDF
};
int launch_dense_walk(const WalkLaunch& a, const dspark_walk_plan& plan, hipStream_t stream);

int launch_quantize(const void* w2, int dtype, int64_t V, int8_t* q, float* s, hipStream_t stream);

int launch_philox_words(uint64_t seed, uint64_t position, int64_t v0, int64_t n, uint32_t* out,
                        hipStream_t stream);

struct TopkLaunch {
    WalkLaunch w;
    int k;
    const float* w2_bound;    // non-null: the lossless pruned greedy walk
    int32_t* dense_steps;     // pruned walk: per request, steps computed over the whole row
};
int launch_w2_bound(const int8_t* q, const float* s, int64_t V, float* bound, hipStream_t stream);
int launch_topk_walk(const TopkLaunch& a, hipStream_t stream);

// Verification of drafted blocks (csrc/verify.hip). Workspace: the error word at WS_ERR, then
// one state slot per request from VERIFY_WS_STATE, then per-chunk partial results.
constexpr size_t VERIFY_WS_STATE = 256;
constexpr size_t VERIFY_STATE_BYTES = 512;
struct VerifyLaunch {
    const uint16_t* draft_logits;
    const int32_t* draft_tokens;
    const float* target_logits;
    const float* temperature;
    const float* uniforms;
    int32_t* accepted;
    int32_t* out_tokens;
    float* accept_prob;
    void* workspace;
    int bs, T, V, mode;
};
size_t verify_workspace_bytes(int64_t bs, int64_t T, int64_t V);
int launch_verify(const VerifyLaunch& a, hipStream_t stream);

// Kernel launch (walks and verification): plain, or with dispatch-recorded events while kernel
// timing is on.
hipError_t launch_walk_kernel(const void* fn, dim3 grid, dim3 block, void** args, size_t lds,
                              hipStream_t stream);
int set_kernel_timing(int64_t ring_size);
int read_kernel_times(float* us, int max, int* count);

}  // namespace dspark
