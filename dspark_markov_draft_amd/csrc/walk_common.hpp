// Pieces shared by the two dense-walk kernels (lane-per-row v_dot4 for one request, MFMA for
// several): launch parameters, clock stamps, the per-step W1 gather, and the grid-wide combine.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace dspark {

constexpr int WALK_THREADS = 256;
constexpr int WALK_WAVES = WALK_THREADS / WAVE;  // 4: one wave per SIMD
constexpr int W1Q_BYTES = MAX_BS * RANK;         // high digits of the gathered W1 rows (LDS)
constexpr int W1L_BYTES = MAX_BS * RANK;         // their low digits, one byte each
constexpr int W1N_BYTES = MAX_BS * RANK / 2;     // or two per byte (the multi-request MFMA kernel)
constexpr int LDS_MIN_BYTES = 96 * 1024;         // > half a CU's LDS: one workgroup per CU
// Bound of every grid-wide wait, in ticks of the 100 MHz constant clock: 10 ms, some thousand
// times the longest healthy wait (the first step's, behind the W2 fill). A walk whose
// workgroups are not all resident at once (other work holds compute units) thus gives up within
// milliseconds per wait and reports DSPARK_ERR_TIMEOUT.
constexpr uint32_t DEFAULT_SPIN_TICKS = 1000000u;
constexpr int DOT4_REG_SETS = 3;  // lane-per-row kernel: row sets of 256 rows held in registers
constexpr int MFMA1_TILES = 10;      // one-request MFMA kernel: 16-row tiles per wave in registers
// Smaller register-slot counts for smaller slices: the kernel multiplies and finishes every slot
// it has (no branch per tile), so a slice of at most 4 or 8 tiles per wave runs an instantiation
// with that many slots.
__host__ __device__ constexpr int mfma1_reg_slots(int tiles_per_wave) {
    return tiles_per_wave <= 4 ? 4 : tiles_per_wave <= 8 ? 8 : MFMA1_TILES;
}
constexpr int MFMA1_LDS_TILES = 8;   // and at most this many more in LDS (4 KB each)
constexpr int MFMA1_MAX_ROWS = (MFMA1_TILES + MFMA1_LDS_TILES) * WALK_WAVES * 16;   // 1152
// rows each lane of the one-request kernel finishes per step, at most (4 tile slots per row)
constexpr int MFMA1_MAX_GROUPS = (MFMA1_TILES + MFMA1_LDS_TILES + 3) / 4;
// MFMA kernel, slices of up to MFMA_STATIC_ROWS rows: all LDS in static arrays (see the kernel):
// two staging buffers for 16 rows of at most MFMA_STATIC_STRIDE floats (157 odd 16-byte units),
// up to mfma_static_lds_slots() LDS tiles per wave, W1 codes and scales, row scales, lane keys,
// tokens. Its workgroup has 4 waves (one per SIMD) or 8 (two per SIMD, half the registers
// each). Every wave has mfma_static_slots() tile slots (registers first, then LDS), at most
// MFMA_STATIC_SLOT_ROWS rows per workgroup; the row-scale array and the staging buffers are
// sized for reads of all of them. A staging buffer also holds whole 64-lane copy instructions
// (64 units each). The kernel multiplies and finishes every slot it has, with no branch per
// tile, so a slice that needs fewer slots runs a build with fewer.
constexpr int MFMA_STATIC_ROWS = 624;
constexpr int MFMA_STATIC_STRIDE = 628;
constexpr int MFMA_STATIC_SLOT_ROWS = 640;
// tile slots per wave of the builds with `waves` waves: the most a wave has (MFMA_STATIC_SLOT_ROWS
// rows), or, for slices of at most 512 rows, the fewer that hold them
__host__ __device__ constexpr int mfma_static_max_slots(int waves) {
    return MFMA_STATIC_SLOT_ROWS / (16 * waves);
}
__host__ __device__ constexpr int mfma_static_small_slots(int waves) { return 512 / (16 * waves); }
__host__ __device__ constexpr int mfma_static_slots(int tiles_per_wave, int waves) {
    return tiles_per_wave <= mfma_static_small_slots(waves) ? mfma_static_small_slots(waves)
                                                            : mfma_static_max_slots(waves);
}
// tile slots per wave held in registers: 8 with 4 waves, 5 with 8 (the sampling kernels finish
// their slots in two halves, which leaves them the registers); the rest of a build's slots are
// in LDS
__host__ __device__ constexpr int mfma_static_reg_slots(int waves) { return waves == 4 ? 8 : 5; }
__host__ __device__ constexpr int mfma_static_lds_slots(int slots, int waves) {
    return slots > mfma_static_reg_slots(waves) ? slots - mfma_static_reg_slots(waves) : 0;
}
constexpr int MFMA_STATIC_COPY_UNITS = (16 * MFMA_STATIC_STRIDE / 4 + WAVE - 1) / WAVE * WAVE;
constexpr int MFMA_STATIC_STAGE_FLOATS =
    MFMA_STATIC_COPY_UNITS * 4 > 15 * MFMA_STATIC_STRIDE + MFMA_STATIC_SLOT_ROWS
        ? MFMA_STATIC_COPY_UNITS * 4
        : 15 * MFMA_STATIC_STRIDE + MFMA_STATIC_SLOT_ROWS;
// per-request sampling constants, loaded once per call: seed, position offset, 1 / temperature
constexpr int MFMA_REQ_CONST_BYTES = MAX_BS * (8 + 8 + 4);
__host__ __device__ constexpr int mfma_static_lds_bytes(int sample, int slots, int waves) {
    return 2 * MFMA_STATIC_STAGE_FLOATS * 4 + mfma_static_lds_slots(slots, waves) * waves * 4 * WAVE * 16 +
           W1Q_BYTES + W1N_BYTES + MAX_BS * 4 + MFMA_STATIC_SLOT_ROWS * 4 +
           (sample == 2 ? waves : 1) * MAX_BS * 8 + MAX_BS * 4 + MFMA_REQ_CONST_BYTES;
}
static_assert(mfma_static_lds_bytes(0, 10, 4) <= 160 * 1024 && mfma_static_lds_bytes(1, 10, 4) <= 160 * 1024 &&
                  mfma_static_lds_bytes(2, 10, 4) <= 160 * 1024 && mfma_static_lds_bytes(2, 5, 8) <= 160 * 1024,
              "static LDS fits a CU");
// more than half a CU's LDS, so that one workgroup runs per CU with every build
static_assert(mfma_static_lds_bytes(0, 8, 4) > 80 * 1024 && mfma_static_lds_bytes(0, 4, 8) > 80 * 1024,
              "one workgroup per CU");
static_assert(mfma_static_max_slots(4) == 10 && mfma_static_small_slots(4) == 8 &&
                  mfma_static_max_slots(8) == 5 && mfma_static_small_slots(8) == 4,
              "slot builds");
// The kernel with dynamic LDS has small static arrays too (the request constants and the
// unused forms of the static buffers): its dynamic LDS leaves this much of the CU's LDS free.
constexpr int MFMA_DYN_STATIC_RESERVE = 2048;
static_assert(MFMA_STATIC_SLOT_ROWS >= MFMA_STATIC_ROWS, "static slices fit in the tile slots");

struct WalkParams {
    const int8_t* q;
    const float* scale;
    const void* w1;
    const float* base;
    const int32_t* start;
    int32_t* tokens;
    float* out_logits;
    uint16_t* draft_logits;
    const uint64_t* seeds;
    const int64_t* positions;
    const float* temps;
    uint64_t* result;       // [16][64] winning keys
    uint64_t* slots;        // [T][num workgroups][stride] per-workgroup keys
    uint32_t* err;
    const uint32_t* never;  // a workspace word nothing writes (test hook)
    uint64_t* stamps;       // instrumented builds: [num workgroups][STAMPS_PER_WG]
    uint64_t* done;         // inverse-CDF walks: [256] end-of-walk flags (workspace)
    int bs, T, V;
    int rows_per_wg;        // contiguous W2 rows per workgroup (the last may own fewer)
    int reg_units;          // register-resident row sets (dot4) or tiles per wave (MFMA)
    int lds_units;          // LDS-resident row sets (dot4) or tiles per wave (MFMA)
    int total_units;        // all row sets / tiles per wave; the rest beyond reg+lds stream
    int stride;             // keys per workgroup slot
    int vec_ok;             // base / draft_logits rows allow float4 and 4 x bf16 accesses
    int stage_bufs;         // MFMA: LDS buffers for the base logits of a 16-request tile (0-2)
    int stage_stride;       // MFMA: floats per request row in a staging buffer
    uint32_t spin_ticks;    // bound of each grid-wide wait (100 MHz clock ticks)
    int wait_unset;
    int w1_row_bytes;       // bytes of one W1 row (RANK elements of its type)
};

// Elapsed-time bound of one grid-wide wait on the constant 100 MHz clock (s_memrealtime). Each
// pass of a wait loop reads the clock first (now()) and compares it last (expired()): the scalar
// read returns while the pass's polls are in flight, and the loop keeps the shape of a plain
// counted loop. (A check only every n-th pass made the compiler copy the poll registers across
// the back edge, waiting for every load in flight on each pass.)
struct WaitBound {
    uint64_t t0;
    __device__ __forceinline__ WaitBound() : t0(__builtin_amdgcn_s_memrealtime()) {}
    __device__ __forceinline__ static uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }
    __device__ __forceinline__ bool expired(uint64_t t, uint32_t ticks) const {
        return t - t0 > (uint64_t)ticks;
    }
};

// Instrumented builds record the constant-rate device clock (s_memrealtime, 100 MHz) per
// workgroup: kernel start, W2 resident, then per step: W1 codes ready, slice argmax done, own
// slot stored, reductions done, result words seen.
constexpr int STAMP_STEP0 = 2;
constexpr int STAMPS_PER_STEP = 5;
// the multi-request MFMA kernel adds two words per step and 16-request tile: the tile's base
// logits landed (every wave past the barrier), the tile finished
constexpr int STAMP_TILE0 = STAMP_STEP0 + MAX_STEPS * STAMPS_PER_STEP;   // 82
constexpr int STAMP_TILES = MAX_BS / 16;
constexpr int STAMPS_PER_WG = STAMP_TILE0 + MAX_STEPS * STAMP_TILES * 2;   // 210

template <int TIMED>
__device__ __forceinline__ void stamp(const WalkParams& p, int slot) {
    if constexpr (TIMED) {
        if (threadIdx.x == 0)
            p.stamps[(size_t)blockIdx.x * STAMPS_PER_WG + slot] = __builtin_amdgcn_s_memrealtime();
    }
}

__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_error(uint32_t* err, int status) {
    __hip_atomic_store(err, (uint32_t)(-status), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// W1 codes. The gathered row is coded per step as C[k] = rint(w[k] * 2032 / absmax), an integer
// in [-2032, 2032] (2032 = 16 * 127), with the step s1 = absmax / 2032. C is held as two int8
// digits, C = 16 * hi + lo with hi in [-127, 127] and lo in [-8, 7], so that the int8 dot
// products give the exact int32 sum_k q[v,k] C[k] = 16 * sum q hi + sum q lo (at most
// 256 * 127 * 2032 < 2^27 in magnitude). Every kernel forms the same integer and hence the same
// logit. The coding error of a W1 element is at most s1 / 2 = absmax / 4064, 1/16 of that of a
// plain int8 code, so a row with a few large entries still meets the logit tolerance.
constexpr float W1_CODE_RANGE = 2032.0f;

// The digits of request b's row in LDS: 256 bytes per request (high digits, and low digits in
// the byte form), whose 16-byte chunk ch sits at position ch ^ (b & 15). A broadcast read of one
// chunk is unaffected; a read of chunk ch for 16 consecutive requests (the MFMA B operand)
// spreads over all LDS banks.
__device__ __forceinline__ int w1q_chunk_dword(int b, int ch) { return b * (RANK / 4) + ((ch ^ (b & 15)) << 2); }
// The nibble form of the low digits (lo + 8 in 4 bits): 128 bytes per request, whose 8-byte
// chunk ch (16 elements) sits at position ch ^ (b & 15).
__device__ __forceinline__ int w1n_chunk_dword(int b, int ch) { return b * (RANK / 8) + ((ch ^ (b & 15)) << 1); }

// 2032 / absmax, the factor that maps a W1 row onto its codes; 0 for rows whose absmax is at
// most 2^-100 (zero rows, and denormal ones whose 2032 / absmax would overflow): their codes are
// 0, dropping a bias below 2^-90.
__device__ __forceinline__ float w1_code_scale(float absmax) {
    return absmax > 0x1p-100f ? W1_CODE_RANGE / absmax : 0.0f;
}
// the code step s1 of a row with this absmax
__device__ __forceinline__ float w1_code_step(float absmax) { return absmax * (1.0f / W1_CODE_RANGE); }

// The code of one element, offset: D = C + 8 (round half to even). With inv = 2032 / absmax,
// |w * inv| <= 2032 * (1 + 2^-23)^2 < 2032.5, so C lies in [-2032, 2032] without a clamp. The
// rounding: for |x| < 2^22, the fp32 sum x + 1.5 * 2^23 is rounded to an integer (its unit in
// the last place is 1) half to even, and as 1.5 * 2^23 is even that integer is
// 1.5 * 2^23 + rint(x), with bit pattern 0x4B400000 + rint(x). The product is rounded before the
// sum: the empty asm makes it a value of its own, so the compiler cannot contract the two into
// one fused multiply-add, which would round w * inv + 1.5 * 2^23 once and could differ from rint
// of the rounded product. From D: hi = D >> 4 (arithmetic; bits 4..11 of D are its two's
// complement byte) and lo = (D & 15) - 8.
__device__ __forceinline__ uint32_t code_plus8(float w, float inv) {
    float x = w * inv;
    asm volatile("" : "+v"(x));
    return __float_as_uint(x + 12582912.0f) - (0x4B400000u - 8u);   // + 1.5 * 2^23
}
// Four low digits held as lo + 8 in the low nibble of each byte -> four int8 (lo in [-8, 7]):
// n ^ 8 is lo in 4-bit two's complement, and its sign bit (bit 3) copied into bits 4..7 of the
// same byte (shifts by 1..4 stay inside the byte) makes the int8.
__device__ __forceinline__ uint32_t low_digit_bytes(uint32_t nib) {
    const uint32_t x = nib ^ 0x08080808u;
    const uint32_t m = x & 0x08080808u;
    return x | (m << 1) | (m << 2) | (m << 3) | (m << 4);
}
// The 16 low digits of one chunk from its nibble form, as the four dwords of int8 the dot
// products take: dword 0 of the pair holds elements 0..3 in its low nibbles and 4..7 in its
// high nibbles, dword 1 elements 8..15 alike.
__device__ __forceinline__ uint4 unpack_low_digits(const uint2 n) {
    return make_uint4(low_digit_bytes(n.x & 0x0F0F0F0Fu), low_digit_bytes((n.x >> 4) & 0x0F0F0F0Fu),
                      low_digit_bytes(n.y & 0x0F0F0F0Fu), low_digit_bytes((n.y >> 4) & 0x0F0F0F0Fu));
}
// v_perm_b32(hi, lo, sel): byte i of the result is byte sel_i of {hi, lo} (lo = 0..3)
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    const uint32_t p01 = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);   // b0.byte0, b1.byte0
    const uint32_t p23 = __builtin_amdgcn_perm(b3, b2, 0x0C0C0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}
// Four elements: their high digits as four int8 in one dword (returned); their low digits as
// four int8 in `lo`, or, offset by 8, as 4-bit values in `nib` (byte i holds element i's).
__device__ __forceinline__ uint32_t pack_codes(const float4 w, float inv, uint32_t& lo, uint32_t& nib) {
    const uint32_t d0 = code_plus8(w.x, inv), d1 = code_plus8(w.y, inv);
    const uint32_t d2 = code_plus8(w.z, inv), d3 = code_plus8(w.w, inv);
    nib = pack_low_bytes(d0, d1, d2, d3) & 0x0F0F0F0Fu;
    lo = low_digit_bytes(nib);
    return pack_low_bytes(d0 >> 4, d1 >> 4, d2 >> 4, d3 >> 4);
}
// maximum of non-negative floats over each 16-lane row of the wave (all 16 lanes get it)
__device__ __forceinline__ float row16_max_nonneg_f32(float x) {
    uint32_t v = __float_as_uint(x);
    v = dpp_max_u32<DPP_SWAP1>(v);
    v = dpp_max_u32<DPP_SWAP2>(v);
    v = dpp_max_u32<DPP_HALF_MIRROR>(v);
    v = dpp_max_u32<DPP_MIRROR>(v);
    return __uint_as_float(v);
}

// 16 int8 x int8 products added into 4 independent int32 chains (v_dot4_i32_i8), and their sum.
__device__ __forceinline__ void dot16x4(const int4 a, const int4 b, int4& acc) {
    acc.x = __builtin_amdgcn_sdot4(a.x, b.x, acc.x, false);
    acc.y = __builtin_amdgcn_sdot4(a.y, b.y, acc.y, false);
    acc.z = __builtin_amdgcn_sdot4(a.z, b.z, acc.z, false);
    acc.w = __builtin_amdgcn_sdot4(a.w, b.w, acc.w, false);
}
__device__ __forceinline__ int hsum(const int4 a) { return (a.x + a.y) + (a.z + a.w); }

// One W1 row coded by one wave (lane l holds elements 4l .. 4l+3): returns lane l's four high
// digits, sets `lo` to its four low digits (int8) and s1 to the row's code step.
__device__ __forceinline__ uint32_t w1_row_quantise(const float4 w, float& s1, uint32_t& lo) {
    float a = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
    a = wave_max_nonneg_f32(a);
    const float inv = w1_code_scale(a);
    s1 = w1_code_step(a);
    uint32_t nib;
    return pack_codes(w, inv, lo, nib);
}

// Where the low digits go: one int8 each (the layout of the high digits), or two per byte.
constexpr int LOW_BYTES = 1;
constexpr int LOW_NIBBLES = 2;

// Per step: W1[prev_b] for every request, coded as above: high digits into w1q, low digits into
// w1l (LOW form), the step into s1[b]. Up to 4 requests (byte form): one per wave, 64 lanes on
// the row. More, or the nibble form: sixteen lanes share a row: lane (quarter q, ql) holds
// elements 16 ql .. 16 ql + 15 of request 4 (iteration * 4 + wave) + q, so one wave instruction
// serves 4 requests; all of a wave's rows are loaded before any is used.
// after_issue() runs once the wave's loads are issued and before their values are used: loads
// it issues complete after the W1 rows (vector memory returns in issue order) without delaying
// them.
// NW: the workgroup's waves (4, or 8 in the nibble form); iterations take 4 NW requests each

template <int W1T, int LOW, int MAX_NIT = 2, int NW = WALK_WAVES, typename AfterIssue>
__device__ __forceinline__ void gather_w1_codes(const WalkParams& p, const int32_t* tok,
                                                uint32_t* w1q, uint32_t* w1l, float* s1, int wave,
                                                int lane, AfterIssue&& after_issue) {
    static_assert(NW == WALK_WAVES || (NW == 8 && LOW == LOW_NIBBLES), "gather waves");
    if (LOW == LOW_BYTES && p.bs <= NW) {
        // at most one request per wave: all 64 lanes on one row (elements 4l .. 4l+3)
        const int b = wave;
        float4 w = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (b < p.bs) w = load4_as_f32<W1T>(p.w1, (int64_t)tok[b] * RANK + lane * 4);
        after_issue();
        if (b < p.bs) {
            float sb;
            uint32_t lo;
            const int d = w1q_chunk_dword(b, lane >> 2) + (lane & 3);
            w1q[d] = w1_row_quantise(w, sb, lo);
            w1l[d] = lo;
            if (lane == 0) s1[b] = sb;
        }
        return;
    }
    // (the per-lane LDS addresses of the codes are computed at every call: hoisted out of the
    // caller's step loop, they were spilled and reloaded before each write)
    asm volatile("" : "+v"(lane));
    // Iterations it0 .. it0 + NIT - 1, NIT a template argument so that the code is
    // straight-line: all their loads are issued before any is used. (With a branch per iteration
    // the compiler moved each iteration's loads next to their use, one memory round trip per
    // iteration.) At most MAX_NIT iterations' rows are held at once, as the caller's register
    // budget allows. Lanes of requests past bs load request 0's row and drop the result.
    auto gather = [&](auto nit_c, int it0, bool issue_hook) {
        constexpr int NIT = decltype(nit_c)::value;
        const int q = lane >> 4, ql = lane & 15;
        uint4 raw[NIT][4];
        // (issued last group first: a pass that shares no leading loads with the one-group
        // pass is not merged with it by the compiler, which put a wait inside the merged code)
#pragma unroll
        for (int ii = 0; ii < NIT; ++ii) {
            const int i = NIT - 1 - ii;
            const int it = it0 + i;
            const int b = (it * NW + wave) * 4 + q;
            const int64_t e = (int64_t)tok[b < p.bs ? b : 0] * RANK + ql * 16;
#pragma unroll
            for (int k = 0; k < 4; ++k) raw[i][k] = load4_raw<W1T>(p.w1, e + 4 * k);
        }
        if (issue_hook) after_issue();
        // without the fence the compiler starts converting the first rows (to free their
        // registers) before the later loads are issued: one round trip per iteration again
        float4 wv[NIT][4];
#pragma unroll
        for (int i = 0; i < NIT; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                fence_raw4<W1T>(raw[i][k]);
                wv[i][k] = raw4_to_f32<W1T>(raw[i][k]);
            }
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const int it = it0 + i;
            const int b = (it * NW + wave) * 4 + q;
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                a = fmaxf(a, fmaxf(fmaxf(fabsf(wv[i][k].x), fabsf(wv[i][k].y)),
                                   fmaxf(fabsf(wv[i][k].z), fabsf(wv[i][k].w))));
            a = row16_max_nonneg_f32(a);
            const float inv = w1_code_scale(a);
            uint4 codes, lo, nib;
            codes.x = pack_codes(wv[i][0], inv, lo.x, nib.x);
            codes.y = pack_codes(wv[i][1], inv, lo.y, nib.y);
            codes.z = pack_codes(wv[i][2], inv, lo.z, nib.z);
            codes.w = pack_codes(wv[i][3], inv, lo.w, nib.w);
            if (b < p.bs) {
                *reinterpret_cast<uint4*>(w1q + w1q_chunk_dword(b, ql)) = codes;
                if constexpr (LOW == LOW_BYTES)
                    *reinterpret_cast<uint4*>(w1l + w1q_chunk_dword(b, ql)) = lo;
                else
                    *reinterpret_cast<uint2*>(w1l + w1n_chunk_dword(b, ql)) =
                        make_uint2(nib.x | (nib.y << 4), nib.z | (nib.w << 4));
                if (ql == 0) s1[b] = w1_code_step(a);
            }
        }
    };
    static_assert(MAX_NIT == 1 || MAX_NIT == 2 || MAX_NIT == 4, "gather passes");
    if constexpr (NW == 8) {
        // 32 requests per iteration: one, or two in one pass
        if (p.bs <= 32 || MAX_NIT == 1) {
            gather(std::integral_constant<int, 1>{}, 0, true);
            if (p.bs > 32) gather(std::integral_constant<int, 1>{}, 1, false);
        } else {
            gather(std::integral_constant<int, 2>{}, 0, true);
        }
        return;
    }
    // iterations with a request for some wave: 16 requests per iteration
    if (p.bs <= 16) {
        gather(std::integral_constant<int, 1>{}, 0, true);
    } else if constexpr (MAX_NIT == 4) {
        gather(std::integral_constant<int, 4>{}, 0, true);   // groups past bs load request 0
    } else if constexpr (MAX_NIT == 2) {
        gather(std::integral_constant<int, 2>{}, 0, true);
        if (p.bs > 32) gather(std::integral_constant<int, 2>{}, 2, false);
    } else {
        // one iteration per pass (kernels with no registers to spare)
        gather(std::integral_constant<int, 1>{}, 0, true);
        gather(std::integral_constant<int, 1>{}, 1, false);
        if (p.bs > 32) {
            gather(std::integral_constant<int, 1>{}, 2, false);
            gather(std::integral_constant<int, 1>{}, 3, false);
        }
    }
}

// Start tokens into LDS, replacing any outside [0, V) by 0 (a documented precondition; this
// keeps every later gather in bounds) and recording DSPARK_ERR_INVALID_ARG.
__device__ __forceinline__ void load_start_tokens(const WalkParams& p, int32_t* tok) {
    const int tid = threadIdx.x;
    if (tid < p.bs) {
        int s = p.start[tid];
        if (s < 0 || s >= p.V) {
            if (blockIdx.x == 0) flag_error(p.err, DSPARK_ERR_INVALID_ARG);
            s = 0;
        }
        tok[tid] = s;
    }
}

// Grid-wide combine of step t, run by wave 0 (all 64 lanes). `key` (lanes < bs) is this
// workgroup's best key for request `lane`. Each workgroup stores its key of request b into slot
// [b][workgroup] of the step (request-major: a reducer's poll round reads whole cache lines);
// the workgroup owning request b (b % num workgroups) waits for all slots of b, takes their
// maximum, writes the token and publishes the winning key in result[t][b] (not for the last
// step) in RESULT_REPLICAS copies on separate cache lines, clears the slots it read and its
// result words of step t-1 (every workgroup read those before filling its slot of step t); then
// every workgroup waits for its copy (workgroup w reads copy w % RESULT_REPLICAS) of the result
// words of step t and writes the new tokens into `tok`. Both waits keep two rounds of loads in
// flight: a store that becomes visible is seen about one load latency later, not one and a half.
// All waits are bounded in time (WaitBound).
__device__ __forceinline__ uint64_t* result_word(const WalkParams& p, int rep, int t, int b) {
    return p.result + ((size_t)rep * MAX_STEPS + t) * MAX_BS + b;
}

// Grid-wide combine for one or two requests (NB = bs). Every step but the last has no reducer:
// every workgroup stores its key and reads all the keys of the step itself, which saves the
// second cross-chip hop of the reducer scheme (reducer -> result word -> every workgroup). The
// keys of a step sit in REPL = 8 replicas, each holding request b's keys of all workgroups side
// by side ([t][replica][b][workgroup] in the step's slot region): a workgroup writes its key into
// every replica and reads replica wg % REPL, so one wave load reads 64 keys from four cache
// lines, and each line is read by at most nwg / REPL workgroups per round instead of all.
// Workgroups are dealt round-robin over the 8 XCDs, so each replica is polled from one XCD; at
// one request this measured 0.1 us per step faster than 16 replicas (V = 151936, T = 16: 60.8
// against 62.3 us) and than 4.
// Having seen all keys of step t, a workgroup knows every workgroup has read all keys of step
// t-1 (each read them before storing its key of step t), so it clears its own keys of step t-1.
// The last step stores its keys into replica 0 only, for one reducer per request (workgroup
// b % nwg), which writes the token and clears the request's keys of steps T-1 and T-2; nothing
// is published. The workspace is all zero when the walk ends. Waits keep two rounds of loads in
// flight and are bounded in time (WaitBound).
__device__ __forceinline__ uint64_t* replica_slot(const WalkParams& p, int t, int rep, int nb,
                                                  int b, int w) {
    return p.slots + (size_t)t * gridDim.x * p.stride + (size_t)(rep * nb + b) * gridDim.x + w;
}

template <int TIMED, int NB>
__device__ __forceinline__ void combine_step_small(const WalkParams& p, int t, uint64_t key,
                                                   int32_t* tok, int lane) {
    constexpr int REPL = 8;
    static_assert(REPL * NB <= 16, "replicas fit the slot region of a step");
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const bool last = t + 1 == p.T;
    // lane l < REPL * NB stores request l % NB's key into replica l / NB
    auto key_of_lane = [&](int src) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((uint32_t)key, src);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((uint32_t)(key >> 32), src);
        return ((uint64_t)hi << 32) | lo;
    };
    uint64_t kb = key_of_lane(0);
    if constexpr (NB == 2) kb = (lane & 1) ? key_of_lane(1) : kb;
    const int my_rep = lane / NB, my_b = lane % NB;
    if (lane < (last ? NB : REPL * NB)) st_dev(replica_slot(p, t, my_rep, NB, my_b, wg), kb);
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 2);

    constexpr int NL = MAX_WORKGROUPS / WAVE;  // key loads per lane and request per round
    bool mine[NB];
    bool any = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        mine[b] = !last || b % nwg == wg;
        any = any || mine[b];
    }
    const int rd_rep = last ? 0 : wg % REPL;
    uint64_t best[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) best[b] = 0;
    if (any) {
        // unconditional loads (lanes past the grid re-read the last key)
        auto issue = [&](uint64_t (&v)[NB][NL]) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int k = 0; k < NL; ++k)
                    v[b][k] = ld_dev(replica_slot(p, t, rd_rep, NB, b, min(lane + k * WAVE, nwg - 1)));
        };
        auto complete = [&](const uint64_t (&v)[NB][NL]) {
            bool all = true;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                uint64_t m = 0;
#pragma unroll
                for (int k = 0; k < NL; ++k) {
                    all = all && (!mine[b] || v[b][k] != 0);
                    m = v[b][k] > m ? v[b][k] : m;
                }
                best[b] = m;
            }
            if (p.wait_unset)
                all = all && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) != 0;
            return __all(all);
        };
        uint64_t va[NB][NL], vb[NB][NL];
        const WaitBound wait;
        issue(va);
        while (true) {
            const uint64_t now = WaitBound::now();
            issue(vb);
            if (complete(va)) break;
            issue(va);
            if (complete(vb)) break;
            if (wait.expired(now, p.spin_ticks)) {
                if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                break;
            }
        }
    }
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 3);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (!mine[b]) continue;
        uint64_t k = wave_max_u64(best[b]);
        if (k == 0) k = 1;  // only after a timeout
        uint32_t token = key_index(k);
        if (token >= (uint32_t)p.V) token = 0;
        if (b % nwg == wg && lane == 0) p.tokens[b * p.T + t] = (int32_t)token;
        if (lane == b) tok[b] = (int32_t)token;
        if (last) {
            // the reducer clears the request's keys: replica 0 of this step, every replica of the
            // step before
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                const int w = lane + k * WAVE;
                if (w < nwg) {
                    st_dev(replica_slot(p, t, 0, NB, b, w), 0);
                    if (t > 0)
                        for (int r = 0; r < REPL; ++r) st_dev(replica_slot(p, t - 1, r, NB, b, w), 0);
                }
            }
        }
    }
    if (!last && t > 0 && lane < REPL * NB) st_dev(replica_slot(p, t - 1, my_rep, NB, my_b, wg), 0);
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 4);
}

template <int TIMED>
__device__ __forceinline__ void combine_step(const WalkParams& p, int t, uint64_t key,
                                             int32_t* tok, int lane) {
    if (p.bs == 1) {
        combine_step_small<TIMED, 1>(p, t, key, tok, lane);
        return;
    }
    if (p.bs == 2) {
        combine_step_small<TIMED, 2>(p, t, key, tok, lane);
        return;
    }
    // the per-lane addresses below are computed here at every step: the compiler would
    // otherwise hoist them out of the caller's step loop and hold (or spill) them for the whole
    // walk
    asm volatile("" : "+v"(lane));
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    uint32_t touch = 0;
    uint64_t* step_slots = p.slots + (size_t)t * nwg * p.stride;
    // request-major: the keys of request b of all workgroups side by side, so its reducer's poll
    // round reads nwg / 16 whole cache lines
    if (lane < p.bs) st_dev(step_slots + (size_t)lane * nwg + wg, key);
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 2);

    constexpr int NL = MAX_WORKGROUPS / WAVE;  // slot loads per lane per round
    for (int b = wg; b < p.bs; b += nwg) {
        const uint64_t* col = step_slots + (size_t)b * nwg;
        // unconditional loads (lanes past the grid re-read the last slot), so that the compiler
        // can count the loads in flight
        auto issue = [&](uint64_t (&v)[NL]) {
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                const int w = min(lane + k * WAVE, nwg - 1);
                v[k] = ld_dev(col + w);
            }
        };
        auto complete = [&](const uint64_t (&v)[NL], uint64_t& best) {
            bool all = true;
            best = 0;
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                all = all && v[k] != 0;
                best = v[k] > best ? v[k] : best;
            }
            if (p.wait_unset)
                all = all && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) != 0;
            return __all(all);
        };
        uint64_t va[NL], vb[NL];
        uint64_t best = 0;
        const WaitBound wait;
        issue(va);
        while (true) {
            const uint64_t now = WaitBound::now();
            issue(vb);
            if (complete(va, best)) break;
            issue(va);
            if (complete(vb, best)) break;
            if (wait.expired(now, p.spin_ticks)) {
                if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                break;
            }
        }
        best = wave_max_u64(best);
        if (best == 0) best = 1;  // only after a timeout: keep the result words non-zero
        uint32_t token = key_index(best);
        if (token >= (uint32_t)p.V) token = 0;
        if (lane == 0) p.tokens[b * p.T + t] = (int32_t)token;
        if (lane < RESULT_REPLICAS) {
            if (t + 1 < p.T) st_dev(result_word(p, lane, t, b), best);
            if (t > 0) st_dev(result_word(p, lane, t - 1, b), 0);
        }
        // Every workgroup gathers W1 row `token` at the next step, about one exchange from now:
        // one word of each 64 bytes of it is read here, which brings the row into the
        // memory-side cache first. (The value is consumed at the end of the combine, after the
        // polls, which complete behind it anyway.) Above 16 requests only: there it measured
        // 3-4 us faster per walk at 64 requests, while at 16 the sampling walk was 1 us slower.
        if (p.bs > 16 && t + 1 < p.T && lane * 64 < p.w1_row_bytes)
            touch ^= *reinterpret_cast<const uint32_t*>(static_cast<const char*>(p.w1) +
                                                         (int64_t)token * p.w1_row_bytes + lane * 64);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int w = lane + k * WAVE;
            if (w < nwg) st_dev(step_slots + (size_t)b * nwg + w, 0);
        }
    }
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 3);

    if (t + 1 < p.T) {
        const uint64_t* mine = result_word(p, wg % RESULT_REPLICAS, t, lane < p.bs ? lane : 0);
        uint64_t ka, kb;
        const WaitBound wait;
        auto seen = [&](uint64_t k) {
            bool ok = lane >= p.bs || k != 0;
            if (p.wait_unset)
                ok = ok && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) != 0;
            return __all(ok);
        };
        uint64_t k = 0;
        ka = ld_dev(mine);
        while (true) {
            const uint64_t now = WaitBound::now();
            kb = ld_dev(mine);
            if (seen(ka)) {
                k = ka;
                break;
            }
            ka = ld_dev(mine);
            if (seen(kb)) {
                k = kb;
                break;
            }
            if (wait.expired(now, p.spin_ticks)) {
                if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                k = kb;
                break;
            }
        }
        if (lane < p.bs) {
            uint32_t token = key_index(k);
            if (token >= (uint32_t)p.V) token = 0;
            tok[lane] = (int32_t)token;
        }
    }
    asm volatile("" ::"v"(touch));
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 4);
}

// ---- inverse-CDF combine (sample == 2) ---------------------------------------------------------
// Each workgroup holds, per request, the pair (m, s) of its slice: the maximum m of z =
// lb * log2(e) / temp over its rows and s = sum 2^(z - m). The token is the first row whose
// running mass passes u * (total mass), which takes three hops per step (wave 0, lanes =
// requests, all waits bounded in time):
//  1. every workgroup stores its pair of request b in the step's slots ([b][workgroup], as the
//     argmax keys); the reducer of b (workgroup b % num workgroups) reads them all, merges them in
//     workgroup order (the vocabulary order of the slices), finds the workgroup w* whose slice
//     holds the point u * S and the remaining mass lt inside it (in units of 2^(z - m_w*)),
//     clears the slots, and publishes (w* + 1, lt) in ICDF_REPL copies of the step's selection
//     word; having seen every pair of step t it also clears request b's selection and token
//     words of step t - 1 (every workgroup read them before storing a pair of step t);
//  2. every workgroup reads the selection words; for each request that selects it, it scans its
//     own slice of the stored bf16 row (its own stores, visible after the workgroup barrier that
//     precedes the combine) in vocabulary order for the first row whose running mass passes lt
//     (the slice's last row with mass if rounding leaves none), writes the token and, unless the
//     step is the last, publishes it (+1) in ICDF_REPL copies of the step's token word;
//  3. every workgroup reads the token words (not after the last step).
// After the last step every workgroup raises its done flag, and workgroup 0 waits for all of
// them and clears the last step's selection words and the flags: the workspace is zero again.
constexpr int ICDF_REPL = RESULT_REPLICAS / 2;   // copies of each selection / token word
constexpr int ICDF_SCAN_ROWS = 8;                // rows per lane per pass of the slice scan

__device__ __forceinline__ uint64_t* icdf_sel_word(const WalkParams& p, int rep, int t, int b) {
    return result_word(p, rep, t, b);
}
__device__ __forceinline__ uint64_t* icdf_tok_word(const WalkParams& p, int rep, int t, int b) {
    return result_word(p, ICDF_REPL + rep, t, b);
}

// Run by one whole wave: the first row of this workgroup's slice whose running mass
// sum 2^(z - m) passes lt, z = lb * kz over the stored row of request b at step t.
__device__ __forceinline__ uint32_t icdf_scan_slice(const WalkParams& p, int b, int t, float m,
                                                    float kz, float lt, int lane) {
    const int row0 = blockIdx.x * p.rows_per_wg;
    const int nrows = min(p.rows_per_wg, p.V - row0);
    const uint16_t* lb = p.draft_logits + ((int64_t)b * p.T + t) * p.V + row0;
    float run = 0.0f;       // mass of the passes before
    int last = -1;          // last row with mass (the rounding fallback)
    for (int r0 = 0; r0 < nrows; r0 += WAVE * ICDF_SCAN_ROWS) {
        const int rb = r0 + lane * ICDF_SCAN_ROWS;
        float e[ICDF_SCAN_ROWS];
        float mine = 0.0f;
#pragma unroll
        for (int i = 0; i < ICDF_SCAN_ROWS; ++i) {
            const int r = rb + i;
            const float x = r < nrows ? bf16_value(lb[r]) : -INFINITY;
            e[i] = x == -INFINITY ? 0.0f : exp2f(x * kz - m);
            mine += e[i];
            if (e[i] > 0.0f) last = max(last, r);
        }
        float incl = mine;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const float v = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += v;
        }
        const float before = run + (incl - mine);
        const uint64_t cross = __ballot(mine > 0.0f && before + mine > lt);
        if (cross) {
            const int L = __builtin_ctzll(cross);
            int tok = -1;
            if (lane == L) {
                float c = before;
#pragma unroll
                for (int i = 0; i < ICDF_SCAN_ROWS; ++i) {
                    c += e[i];
                    if (tok < 0 && e[i] > 0.0f && c > lt) tok = rb + i;
                }
                if (tok < 0) {       // rounding inside the lane: its last row with mass
#pragma unroll
                    for (int i = 0; i < ICDF_SCAN_ROWS; ++i)
                        if (e[i] > 0.0f) tok = rb + i;
                }
            }
            return (uint32_t)(row0 + __shfl(tok, L, WAVE));
        }
        run += __shfl(incl, WAVE - 1, WAVE);
    }
    // the running mass never passed lt (rounding): the slice's last row with mass
    int l = last;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l = max(l, __shfl_xor(l, o, WAVE));
    return (uint32_t)(row0 + max(l, 0));
}

template <int TIMED>
__device__ __forceinline__ void combine_icdf_step(const WalkParams& p, int t, uint64_t pair,
                                                  int32_t* tok, int lane) {
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const bool last_step = t + 1 == p.T;
    uint32_t touch = 0;
    uint64_t* step_slots = p.slots + (size_t)t * nwg * p.stride;
    if (lane < p.bs) st_dev(step_slots + (size_t)lane * nwg + wg, pair);
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 2);

    // ---- 1. reducers: merge the pairs, select the slice ----------------------------------------
    constexpr int NL = MAX_WORKGROUPS / WAVE;
    for (int b = wg; b < p.bs; b += nwg) {
        const uint64_t* col = step_slots + (size_t)b * nwg;
        auto issue = [&](uint64_t (&v)[NL]) {
#pragma unroll
            for (int k = 0; k < NL; ++k) v[k] = ld_dev(col + min(lane + k * WAVE, nwg - 1));
        };
        auto complete = [&](const uint64_t (&v)[NL]) {
            bool all = true;
#pragma unroll
            for (int k = 0; k < NL; ++k) all = all && v[k] != 0;
            if (p.wait_unset)
                all = all && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) != 0;
            return __all(all);
        };
        uint64_t va[NL], vb[NL];
        const WaitBound wait;
        bool ok = true;
        issue(va);
        while (true) {
            const uint64_t now = WaitBound::now();
            issue(vb);
            if (complete(va)) break;
            issue(va);
            if (complete(vb)) {
#pragma unroll
                for (int k = 0; k < NL; ++k) va[k] = vb[k];
                break;
            }
            if (wait.expired(now, p.spin_ticks)) {
                if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                ok = false;
                break;
            }
        }
        // the slice pairs in workgroup order: k-major (workgroup k * 64 + lane)
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NL; ++k)
            if (lane + k * WAVE < nwg && va[k] != 0) M = fmaxf(M, packed_m(va[k]));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, WAVE));
        float mass[NL];
        float S = 0.0f;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const bool in = lane + k * WAVE < nwg && va[k] != 0;
            const float m = packed_m(va[k]);
            mass[k] = (in && m != -INFINITY) ? packed_s(va[k]) * exp2f(m - M) : 0.0f;
        }
        // running mass in workgroup order, and the first workgroup whose interval passes u * S
        float tot[NL], before[NL];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            float incl = mass[k];
#pragma unroll
            for (int o = 1; o < WAVE; o <<= 1) {
                const float v = __shfl_up(incl, o, WAVE);
                if (lane >= o) incl += v;
            }
            tot[k] = __shfl(incl, WAVE - 1, WAVE);
            before[k] = incl - mass[k];
        }
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            before[k] += S;
            S += tot[k];
        }
        const uint64_t seed = p.seeds[b];
        const uint64_t P = (uint64_t)(p.positions ? p.positions[b] : 0) + (uint64_t)t;
        const float target = icdf_uniform(seed, P) * S;
        int wsel = -1;
        float lt = INFINITY;
        int lastw = 0;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const uint64_t has = __ballot(mass[k] > 0.0f);
            if (has) lastw = k * WAVE + 63 - __builtin_clzll(has);
            const uint64_t cross = __ballot(mass[k] > 0.0f && before[k] + mass[k] > target);
            if (wsel < 0 && cross) {
                const int L = __builtin_ctzll(cross);
                wsel = k * WAVE + L;
                // remaining mass inside the selected slice, in units of its own 2^(z - m_w*)
                const float rem = target - __shfl(before[k], L, WAVE);
                const float mw = __shfl(packed_m(va[k]), L, WAVE);
                lt = rem * exp2f(M - mw);
            }
        }
        if (wsel < 0) wsel = lastw;        // rounding: the last slice with mass, its last row
        if (!ok) wsel = 0;
        // clear the pairs read, and request b's words of step t - 1
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int w = lane + k * WAVE;
            if (w < nwg) st_dev(step_slots + (size_t)b * nwg + w, 0);
        }
        if (lane < ICDF_REPL) {
            if (t > 0) {
                st_dev(icdf_sel_word(p, lane, t - 1, b), 0);
                st_dev(icdf_tok_word(p, lane, t - 1, b), 0);
            }
            st_dev(icdf_sel_word(p, lane, t, b),
                   ((uint64_t)(uint32_t)(wsel + 1) << 32) | __float_as_uint(lt));
        }
    }
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 3);

    // ---- 2. every workgroup: the selection words; scan own slice for the requests it holds ----
    {
        const uint64_t* mine = icdf_sel_word(p, wg % ICDF_REPL, t, lane < p.bs ? lane : 0);
        auto seen = [&](uint64_t k) {
            bool okk = lane >= p.bs || k != 0;
            if (p.wait_unset)
                okk = okk && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) != 0;
            return __all(okk);
        };
        uint64_t ka = ld_dev(mine), kb, sel = 0;
        const WaitBound wait;
        while (true) {
            const uint64_t now = WaitBound::now();
            kb = ld_dev(mine);
            if (seen(ka)) { sel = ka; break; }
            ka = ld_dev(mine);
            if (seen(kb)) { sel = kb; break; }
            if (wait.expired(now, p.spin_ticks)) {
                if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                sel = kb;
                break;
            }
        }
        uint64_t todo = __ballot(lane < p.bs && sel != 0 && (int)(sel >> 32) - 1 == wg);
        while (todo) {
            const int b = __builtin_ctzll(todo);
            todo &= todo - 1;
            const uint64_t sb = __shfl(sel, b, WAVE);
            const float lt = __uint_as_float((uint32_t)sb);
            const float kz = LOG2E_F * inv_temperature(p.temps[b]);
            // this slice's own pair of request b: the one it stored (lane b holds it)
            const float m_own = packed_m(__shfl(pair, b, WAVE));
            uint32_t token = icdf_scan_slice(p, b, t, m_own, kz, lt, lane);
            if (token >= (uint32_t)p.V) token = 0;
            if (lane == 0) p.tokens[b * p.T + t] = (int32_t)token;
            if (!last_step && lane < ICDF_REPL)
                st_dev(icdf_tok_word(p, lane, t, b), (uint64_t)token + 1);
            // as in combine_step: the token's W1 row is read here, one hop before every
            // workgroup gathers it, so that it is in the memory-side cache by then
            if (!last_step && p.bs > 16 && lane * 64 < p.w1_row_bytes)
                touch ^= *reinterpret_cast<const uint32_t*>(static_cast<const char*>(p.w1) +
                                                             (int64_t)token * p.w1_row_bytes + lane * 64);
        }
    }
    stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 4);

    if (!last_step) {
        // ---- 3. the tokens ----------------------------------------------------------------------
        const uint64_t* mine = icdf_tok_word(p, wg % ICDF_REPL, t, lane < p.bs ? lane : 0);
        auto seen = [&](uint64_t k) {
            bool okk = lane >= p.bs || k != 0;
            if (p.wait_unset)
                okk = okk && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) != 0;
            return __all(okk);
        };
        uint64_t ka = ld_dev(mine), kb, k = 0;
        const WaitBound wait;
        while (true) {
            const uint64_t now = WaitBound::now();
            kb = ld_dev(mine);
            if (seen(ka)) { k = ka; break; }
            ka = ld_dev(mine);
            if (seen(kb)) { k = kb; break; }
            if (wait.expired(now, p.spin_ticks)) {
                if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                k = kb;
                break;
            }
        }
        if (lane < p.bs) {
            uint32_t token = k == 0 ? 0u : (uint32_t)(k - 1);
            if (token >= (uint32_t)p.V) token = 0;
            tok[lane] = (int32_t)token;
        }
    } else {
        // ---- end of walk: done flags; workgroup 0 clears the last step's selection words ----
        if (lane == 0) st_dev(p.done + wg, 1);
        if (wg == 0) {
            auto all_done = [&]() {
                bool a = true;
#pragma unroll
                for (int k = 0; k < NL; ++k) {
                    const int w = lane + k * WAVE;
                    if (w < nwg) a = a && ld_dev(p.done + w) != 0;
                }
                return __all(a);
            };
            const WaitBound wait;
            while (true) {
                const uint64_t now = WaitBound::now();
                if (all_done()) break;
                if (wait.expired(now, p.spin_ticks)) {
                    if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                    break;
                }
            }
#pragma unroll
            for (int k = 0; k < NL; ++k) {
                const int w = lane + k * WAVE;
                if (w < nwg) st_dev(p.done + w, 0);
            }
            for (int i = lane; i < ICDF_REPL * p.bs; i += WAVE)
                st_dev(icdf_sel_word(p, i / p.bs, t, i % p.bs), 0);
        }
    }
    asm volatile("" ::"v"(touch));
}

// Kernel entry points, as host-side stubs for hipLaunchKernel (sample: 0 greedy, 1 Gumbel,
// 2 inverse CDF; w1t: DT_*).
const void* dot4_walk_kernel(int sample, int w1t, bool timed);
const void* mfma1_walk_kernel(int sample, int w1t, bool timed, bool lds_tiles, int reg_slots);
const void* mfma_walk_kernel(int sample, int w1t, bool timed, bool static_stage, bool out_logits,
                             int slots, int waves);
int mfma_fixed_lds_bytes(int rows_per_wg);

}  // namespace dspark
