// Device helpers of the gfx950 Markov-walk kernels: argmax keys, bf16 rounding, Philox4x32-10,
// Gumbel noise and wave-wide reductions. GPU code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int RANK = 256;
constexpr int MAX_STEPS = 16;
constexpr int MAX_BS = 64;
constexpr int WAVE = 64;

// ---------------------------------------------------------------------------------------------
// torch.argmax order as one unsigned 64-bit key (vLLM PR #64476, Claims: the first NaN wins,
// otherwise the first maximum): the high word maps the float to an order-preserving u32 (every
// NaN to the top, -0 onto +0), the low word is ~index so that at equal values the lower index
// is the larger key. An atomic or wave-wide unsigned max then yields the torch.argmax winner.
// Every real key is >= 0x007FFFFF00000000 (the key of -inf), so a zeroed slot is below all.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key32(float x) {
    uint32_t u = __float_as_uint(x);
    if (x != x) return 0xFFFFFFFFu;
    if (x == 0.0f) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t ORDER_KEY_NEG_INF = 0x007FFFFFu;  // order_key32(-inf), the smallest real key

__device__ __forceinline__ uint64_t argmax_key(float x, uint32_t idx) {
    return ((uint64_t)order_key32(x) << 32) | (uint64_t)(~idx);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

// Running torch.argmax of one lane's values, offered in increasing index order: a value
// replaces the best so far if it is larger (so the first of equal values stays, and -0 and +0
// are equal), if it is a NaN and the best is not (the first NaN stays), or if there is no best
// yet. Three compares and two selects per value, instead of building and comparing a 64-bit
// key for each; key() gives the argmax_key of the element it holds (0 if none).
struct RunningArgmax {
    float v = 0.0f;
    uint32_t i = 0xFFFFFFFFu;
    __device__ __forceinline__ void offer(float x, uint32_t idx, bool ok) {
        // bitwise, not short-circuit, operators: selects rather than branches
        const bool better = (x > v) | (i == 0xFFFFFFFFu) | ((x != x) & (v == v));
        const bool take = ok & better;
        v = take ? x : v;
        i = take ? idx : i;
    }
    __device__ __forceinline__ uint64_t key() const {
        return i == 0xFFFFFFFFu ? 0ull : argmax_key(v, i);
    }
};

// The drafted logit of one vocabulary row: base + (s[v] * s1) * acc, where acc is the exact
// int32 dot product of the row's int8 codes with the request's integer W1 codes and s1 the W1
// row's code step. Written as one explicit fused multiply-add so that every kernel (dense dot4,
// MFMA, top-k) rounds it identically.
__device__ __forceinline__ float walk_logit(float base, float s_row, float s1, int32_t acc) {
    return __builtin_fmaf(s_row * s1, (float)acc, base);
}
// The dot product with the W1 codes C = 16 hi + lo from its two int8 parts (exact in int32).
__device__ __forceinline__ int32_t join_digits(int32_t dot_hi, int32_t dot_lo) {
    return (int32_t)((uint32_t)dot_hi << 4) + dot_lo;
}

// ---------------------------------------------------------------------------------------------
// bf16, round to nearest even; a NaN keeps its sign and top payload bits and becomes quiet:
// (bits >> 16) | 0x40 (vLLM PR #62958, Details: draft_logits are the bf16 logits the sample was
// drawn from). gfx950's packed conversion v_cvt_pk_bf16_f32 gives exactly these bits (checked
// on the device against the integer rule over 67.5M patterns: every high half with the tie and
// boundary low halves, NaN payloads and denormals included), two values per instruction and
// without the NaN branch the integer rule needs.
// ---------------------------------------------------------------------------------------------
typedef float float2_vt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_vt __attribute__((ext_vector_type(2)));
// bf16(lo) in bits 0..15, bf16(hi) in bits 16..31
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    const float2_vt v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_vt));
}
__device__ __forceinline__ uint32_t bf16_bits(float x) { return bf16x2_bits(x, 0.0f) & 0xFFFFu; }

__device__ __forceinline__ float bf16_value(uint32_t h) { return __uint_as_float(h << 16); }
// the two values of a bf16x2_bits pair
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; a round takes the 64-bit
// products of M0 * c0 and M1 * c2 and yields (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key
// advances by the Weyl constants between rounds.
// ---------------------------------------------------------------------------------------------
// a ^ b ^ c in one v_bitop3_b32 (truth table 0x96), where the compiler emits two XORs
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return make_uint4(c0, c1, c2, c3);
}

// The same generator for a run of counters (c0, lo32 P, hi32 P, 0) that differ only in c0 (one
// request at one draft position, every vocabulary group): round 0's product of M1 and hi32 P
// does not depend on c0 and is taken once per run.
struct PhiloxRun {
    uint32_t n0;   // round 0's new c0: hi(M1 * hi32 P) ^ lo32 P ^ k0
    uint32_t c1;   // round 0's new c1: lo(M1 * hi32 P)
    uint32_t k0, k1;
};
__device__ __forceinline__ PhiloxRun philox_run(uint64_t seed, uint64_t P) {
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint32_t)(P >> 32);
    PhiloxRun r;
    r.k0 = (uint32_t)seed;
    r.k1 = (uint32_t)(seed >> 32);
    r.n0 = (uint32_t)(p1 >> 32) ^ (uint32_t)P ^ r.k0;
    r.c1 = (uint32_t)p1;
    return r;
}
__device__ __forceinline__ uint4 philox_run_words(const PhiloxRun& run, uint32_t c0) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint32_t x0 = run.n0, x1 = run.c1, x2 = (uint32_t)(p0 >> 32) ^ run.k1, x3 = (uint32_t)p0;
    uint32_t k0 = run.k0, k1 = run.k1;
#pragma unroll
    for (int r = 1; r < 10; ++r) {
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
        const uint64_t q0 = (uint64_t)0xD2511F53u * x0;
        const uint64_t q1 = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t n0 = xor3((uint32_t)(q1 >> 32), x1, k0);
        const uint32_t n2 = xor3((uint32_t)(q0 >> 32), x3, k1);
        x1 = (uint32_t)q1;
        x3 = (uint32_t)q0;
        x0 = n0;
        x2 = n2;
    }
    return make_uint4(x0, x1, x2, x3);
}

// Noise word of vocabulary entry v at draft position P for a request keyed by `seed`
// (vLLM PR #62958, Details: the noise comes from Philox, with the request's seed and the draft position as inputs):
// counter (v >> 2, lo32 P, hi32 P, 0), key (lo32 seed, hi32 seed), word v & 3.
__device__ __forceinline__ uint32_t noise_word(uint64_t seed, uint64_t P, uint32_t v) {
    const uint4 r = philox4x32_10(v >> 2, (uint32_t)P, (uint32_t)(P >> 32), 0u, (uint32_t)seed,
                                  (uint32_t)(seed >> 32));
    const uint32_t w = v & 3u;
    return w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
}

// Temperature scaling of a bf16 logit: x * (1 / temp) with the reciprocal rounded once per
// request, instead of a correctly rounded x / temp (about ten instructions per element). The
// product is within one unit in the last place of the quotient, and exact at temp = 1, so no
// branch is needed for that common case.
__device__ __forceinline__ float inv_temperature(float temp) { return 1.0f / temp; }

// u = (2 (x >> 9) + 1) 2^-24 is exact in fp32 and lies strictly inside (0, 1); the standard
// Gumbel variate is g = -log(-log u). Both logarithms use the hardware log2 (v_log_f32) scaled
// by ln 2: every argument here is a normal float (u >= 2^-24, -log u >= 6e-8), so the libm
// path's denormal scaling and extra-precision steps (~13 instructions per call) buy nothing;
// over all 2^23 possible u the result is within 1.7e-6 of the exact g, the same bound as logf.
__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
    constexpr float LN2 = 0.6931471805599453f;
    const float u = (float)(2u * (x >> 9) + 1u) * 0x1p-24f;
    const float neg_ln_u = -__builtin_amdgcn_logf(u) * LN2;
    return -(__builtin_amdgcn_logf(neg_ln_u) * LN2);
}

// ---------------------------------------------------------------------------------------------
// Inverse-CDF sampling (the walk's second sampler). The uniform of a request at draft position P
// is word 0 of Philox4x32-10 at counter (0, lo32 P, hi32 P, 1) under the request's seed, a
// counter space disjoint from the Gumbel noise's (whose last counter word is 0), mapped to
// (2 (x >> 9) + 1) 2^-24 like the noise. The step's distribution is softmax(lb / temp), handled
// in the base-2 domain: z = lb * (log2(e) / temp), probabilities 2^(z - m) / s.
// ---------------------------------------------------------------------------------------------
constexpr float LOG2E_F = 1.4426950408889634f;

__device__ __forceinline__ float icdf_uniform(uint64_t seed, uint64_t P) {
    const uint4 r = philox4x32_10(0u, (uint32_t)P, (uint32_t)(P >> 32), 1u, (uint32_t)seed,
                                  (uint32_t)(seed >> 32));
    return (float)(2u * (r.x >> 9) + 1u) * 0x1p-24f;
}

// Running maximum m and sum s of 2^(z - m) over the values offered (m = -inf, s = 0: none, or
// only -inf values). merge() combines two such pairs.
struct RunningSoftmax {
    float m = -INFINITY, s = 0.0f;
    __device__ __forceinline__ void merge(float m2, float s2) {
        const float M = fmaxf(m, m2);
        const float a = m == -INFINITY ? 0.0f : s * exp2f(m - M);
        const float b = m2 == -INFINITY ? 0.0f : s2 * exp2f(m2 - M);
        m = M;
        s = a + b;
    }
    __device__ __forceinline__ void offer(float z, bool ok) {
        if (ok) merge(z, 1.0f);
    }
};
// A pair as one 64-bit word (m's bits high, s's low). A real pair is never 0: s >= 1 when m is
// finite, and m = -inf has non-zero bits.
__device__ __forceinline__ uint64_t pack_softmax(float m, float s) {
    return ((uint64_t)__float_as_uint(m) << 32) | __float_as_uint(s);
}
__device__ __forceinline__ float packed_m(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }
__device__ __forceinline__ float packed_s(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Wave-wide merge of (m, s) pairs; every lane ends with the whole wave's pair.
__device__ __forceinline__ void wave_softmax(float& m, float& s) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        RunningSoftmax r;
        r.m = m;
        r.s = s;
        r.merge(__shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
        m = r.m;
        s = r.s;
    }
}

// ---------------------------------------------------------------------------------------------
// Wave-wide maxima over the 64 lanes with DPP lane moves (a few cycles each, against ~100 for
// an LDS-routed shuffle): swap within pairs and quads, mirror within 8 and 16 lanes, then
// broadcast lane 15 of each 16-lane row into the next row and lane 31 into the upper half;
// lane 63 ends with the maximum of all 64 lanes and is read back as a wave-uniform value.
// Callers run them with all 64 lanes active.
// ---------------------------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    const uint32_t o = dpp_u32<CTRL, ROW_MASK>(v);
    return o > v ? o : v;
}

constexpr int DPP_SWAP1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_SWAP2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // row_half_mirror
constexpr int DPP_MIRROR = 0x140;      // row_mirror
constexpr int DPP_BCAST15 = 0x142;     // row_bcast:15
constexpr int DPP_BCAST31 = 0x143;     // row_bcast:31
constexpr int DPP_ROW_ROR8 = 0x128;    // row_ror:8 (lane l reads lane l ^ 8 of its 16-lane row)

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_u32<DPP_SWAP1>(v);
    v = dpp_max_u32<DPP_SWAP2>(v);
    v = dpp_max_u32<DPP_HALF_MIRROR>(v);
    v = dpp_max_u32<DPP_MIRROR>(v);
    v = dpp_max_u32<DPP_BCAST15, 0xA>(v);
    v = dpp_max_u32<DPP_BCAST31, 0xC>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

// The lexicographic maximum in two 32-bit passes: the largest high word, then the largest low
// word among the lanes that hold it (a 64-bit pass needs a 64-bit compare and two selects per
// step).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t mh = wave_max_u32(hi);
    const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)v : 0u);
    return ((uint64_t)mh << 32) | ml;
}

// maximum of non-negative floats (ordered like their bit patterns)
__device__ __forceinline__ float wave_max_nonneg_f32(float x) {
    return __uint_as_float(wave_max_u32(__float_as_uint(x)));
}

// ---------------------------------------------------------------------------------------------
// Loads of 4 consecutive W1 / W2 elements as fp32 (exact upcasts).
// ---------------------------------------------------------------------------------------------
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// The same four elements in two steps: the raw words (f32: four; bf16 / f16: two, in x and y),
// then their values. fence_raw4 between them makes every load before it issue first and every
// use of the words come after it (the words are in-out operands of an empty asm, so the compiler
// waits for their loads there, once, and cannot move a conversion above it).
template <int DT>
__device__ __forceinline__ uint4 load4_raw(const void* base, int64_t elem) {
    if constexpr (DT == DT_F32) {
        return *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + elem);
    } else {
        const uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + elem);
        return make_uint4(r.x, r.y, 0u, 0u);
    }
}
template <int DT>
__device__ __forceinline__ void fence_raw4(uint4& r) {
    if constexpr (DT == DT_F32)
        asm volatile("" : "+v"(r.x), "+v"(r.y), "+v"(r.z), "+v"(r.w)::"memory");
    else
        asm volatile("" : "+v"(r.x), "+v"(r.y)::"memory");
}
template <int DT>
__device__ __forceinline__ float4 raw4_to_f32(const uint4 r) {
    if constexpr (DT == DT_F32) {
        return make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                           __uint_as_float(r.w));
    } else if constexpr (DT == DT_BF16) {
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
    } else {
        const _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(r.x & 0xFFFFu));
        const _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(r.x >> 16));
        const _Float16 h2 = __builtin_bit_cast(_Float16, (uint16_t)(r.y & 0xFFFFu));
        const _Float16 h3 = __builtin_bit_cast(_Float16, (uint16_t)(r.y >> 16));
        return make_float4((float)h0, (float)h1, (float)h2, (float)h3);
    }
}

template <int DT>
__device__ __forceinline__ float4 load4_as_f32(const void* base, int64_t elem) {
    if constexpr (DT == DT_F32) {
        return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + elem);
        if constexpr (DT == DT_BF16) {
            return make_float4(__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                               __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u));
        } else {
            const _Float16 h0 = __builtin_bit_cast(_Float16, (uint16_t)(raw.x & 0xFFFFu));
            const _Float16 h1 = __builtin_bit_cast(_Float16, (uint16_t)(raw.x >> 16));
            const _Float16 h2 = __builtin_bit_cast(_Float16, (uint16_t)(raw.y & 0xFFFFu));
            const _Float16 h3 = __builtin_bit_cast(_Float16, (uint16_t)(raw.y >> 16));
            return make_float4((float)h0, (float)h1, (float)h2, (float)h3);
        }
    }
}

}  // namespace dspark
