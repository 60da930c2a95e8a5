// The top-k Markov walk (vLLM PR #49969, Purpose: the drafter's logits restricted to the k
// best candidates of the target's base logits and scattered into a dense -inf row; vLLM PR
// #62958, Details: the unchanged sampler over that row), on the caller's stream.
//
// The select (select_row), one workgroup per (request, step) row of base logits: the k largest
// base logits, ties toward the lower vocabulary index. Every element gets a unique 51-bit key
// (the 32-bit order key of its value above 19 bits of reversed index), so "the k largest keys"
// is exactly the wanted set, and an MSB-first radix select finds the k-th key. The row is read
// from HBM once: its first 18432 elements stay in registers while their top-12-bit histogram
// gives a bound, the bin L of the chunk's ceil(2 k chunk / V)-th largest key (k itself when the
// chunk is the whole row). One pass over the rest of the row then appends every element of a
// bin >= L to an LDS buffer, where 12- and 10-bit radix levels find the k-th key and the winners
// are emitted. If fewer than k keys reach L, or the buffer overflows (rows sorted ascending,
// long plateaus, a chunk holding much of the top), an exact fallback takes two more passes: the
// histogram of the whole row, then the elements above the k-th key's bin out directly and that
// bin to LDS (or, if that bin is itself too large, its levels over the row in global memory).
// The first pass also writes -inf over the dense output row when there is one.
//
// The walk, one workgroup per request, its steps in sequence (requests never wait for each
// other): per step the wave-level int8 quantisation of W1[prev] used by the dense walk, the
// v_dot4 logits of the step's k candidates with the dense walk's rounding, their values in the
// dense output row, the sampler's noise keyed by vocabulary index, and the argmax over the
// candidates, which equals the argmax of the dense row with -inf elsewhere.
//
// Two forms. topk_fused_kernel (k <= 512, float4 rows, more rows than compute units): one launch
// in which the workgroups of step 0 walk their request once their own row is selected, reading
// each later step's candidates as they are written. Otherwise topk_select_kernel, then
// topk_walk_kernel, whose candidate rows for the next step load while the current step runs.
#include "walk_common.hpp"

namespace dspark {

constexpr int SEL_THREADS = 512;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;
constexpr int STASH_GROUPS = 9;                       // 4-element groups per thread in registers
constexpr int STASH_ELEMS = SEL_THREADS * STASH_GROUPS * 4;   // 18432
constexpr int MAIN_UNROLL = 8;                        // groups per thread per batch (2 in flight)
constexpr int IDX_BITS = 19;                          // a vocabulary index fits in 19 bits
constexpr uint64_t IDX_MASK = (1ull << IDX_BITS) - 1;
constexpr int CK_BITS = 32 + IDX_BITS;                // 51-bit composite keys
constexpr int L1_BITS = 12;                           // first level: the top 12 bits
constexpr int L1_BINS = 1 << L1_BITS;
constexpr int L1_SHIFT = CK_BITS - L1_BITS;           // 39
constexpr int REGION_CAP = 992;                       // LDS keys per wave (8 waves: 7936 keys)
constexpr int BUF_CAP = SEL_WAVES * REGION_CAP;       // fits two workgroups per CU
constexpr int LDS_LEVEL_BITS = 10;                    // later levels over the LDS buffer
constexpr int GLOBAL_LEVEL_BITS = 12;                 // later levels over the row (fallback)
constexpr int SEL_LDS_BYTES = BUF_CAP * 8 + L1_BINS * 4 + 128;
constexpr int TKW_THREADS = 512;
constexpr int TKW_WAVES = TKW_THREADS / WAVE;
static_assert(DSPARK_MAX_V <= (1 << IDX_BITS), "vocabulary index must fit the composite key");
static_assert(DSPARK_MAX_TOPK <= STASH_ELEMS, "the register chunk must hold k keys");

__device__ __forceinline__ uint64_t composite_key(float x, uint32_t idx) {
    return ((uint64_t)order_key32(x) << IDX_BITS) | (IDX_MASK - idx);
}
__device__ __forceinline__ uint32_t composite_index(uint64_t ck) {
    return (uint32_t)(IDX_MASK - (ck & IDX_MASK));
}
__device__ __forceinline__ uint32_t top_bin(float x) { return order_key32(x) >> (32 - L1_BITS); }

// Instrumented builds: thread 0 records the 100 MHz device clock. Select rows use words
// row * 8 + (0 start, 1 first bound known, 2 row scanned, 3 k-th key known, 4 done, 5 bin of
// the k-th key known, 6 bins above it emitted); walk
// requests use TK_WALK_STAMPS0 + request * 40 + (0 start, then per step t: 1 + 2t W1 codes
// ready, 2 + 2t token known).
constexpr int TK_WALK_STAMPS0 = 8192;
template <bool TIMED>
__device__ __forceinline__ void tk_stamp(uint64_t* st, int64_t idx) {
    if constexpr (TIMED) {
        if (threadIdx.x == 0) st[idx] = __builtin_amdgcn_s_memrealtime();
    }
}

// Lanes of this wave below the calling lane whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Positions for the lanes of a wave whose `pred` is set, reserved with one LDS atomic for the
// whole wave (lanes in ascending order). Every write into a candidate row or into the LDS
// buffer below is also checked against its capacity.
__device__ __forceinline__ uint32_t wave_append(uint32_t* counter, bool pred, int lane) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return 0;
    const int leader = __ffsll((unsigned long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = (uint32_t)__shfl((int)base, leader);
    return base + lanes_below(m);
}

// Inclusive suffix sum over the 64 lanes (lane l gets the sum of lanes l .. 63).
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < WAVE; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_down((int)v, off);
        if (lane + off < WAVE) v += o;
    }
    return v;
}

// Run by one whole wave: the bin d such that fewer than `need` counted keys lie in bins above d
// and at least `need` in bins >= d (1 <= need <= total); `above` = the count above d. Lane l
// sums bins [l * PER, l * PER + PER) in a lane-rotated order (no LDS bank conflicts); a suffix
// scan over lanes finds the lane range holding d, and a second scan over that range's bins
// (one per lane) finds d.
template <int NBINS>
__device__ __forceinline__ void select_digit(const uint32_t* hist, uint32_t need, int lane,
                                             uint32_t& d, uint32_t& above) {
    constexpr int PER = NBINS / WAVE;
    static_assert(PER >= 1 && PER <= WAVE && (PER & (PER - 1)) == 0, "bins per lane");
    uint32_t s = 0;
#pragma unroll 8
    for (int j = 0; j < PER; ++j) s += hist[lane * PER + ((j + lane) & (PER - 1))];
    const uint32_t suf = wave_suffix_sum(s, lane);
    const uint64_t m1 = __ballot(suf - s < need && need <= suf);
    const int src = m1 ? __ffsll((unsigned long long)m1) - 1 : 0;
    const uint32_t above_src = (uint32_t)__shfl((int)(suf - s), src);
    const uint32_t c = lane < PER ? hist[src * PER + lane] : 0u;
    const uint32_t suf2 = wave_suffix_sum(c, lane) + above_src;
    const uint64_t m2 = __ballot(lane < PER && suf2 - c < need && need <= suf2);
    const int j = m2 ? __ffsll((unsigned long long)m2) - 1 : 0;
    d = (uint32_t)(src * PER + j);
    above = (uint32_t)__shfl((int)(suf2 - c), j);
}

struct SelectParams {
    const float* base;    // [rows][V]
    int32_t* cand;        // [rows][k] (workspace)
    uint16_t* fill_bf16;  // [rows][V] dense bf16 output to set to -inf, or null
    float* fill_f32;      // [rows][V] dense fp32 output to set to -inf, or null
    uint64_t* stamps;     // instrumented builds
    int V, k;
};

// Group g of a row: elements 4g .. 4g+3 (those < V); absent elements read as -inf and are
// excluded by the callers through the element count. VEC: the row allows float4 loads.
template <bool VEC>
__device__ __forceinline__ float4 load_group(const SelectParams& p, const float* x, int g) {
    const int i = 4 * g;
    if constexpr (VEC) {
        return reinterpret_cast<const float4*>(x)[g];
    } else {
        float4 a;
        a.x = i < p.V ? x[i] : -INFINITY;
        a.y = i + 1 < p.V ? x[i + 1] : -INFINITY;
        a.z = i + 2 < p.V ? x[i + 2] : -INFINITY;
        a.w = i + 3 < p.V ? x[i + 3] : -INFINITY;
        return a;
    }
}

// The same, never branching around the load (so that the compiler can count loads in
// flight): a group index past the end reads the last group, whose values the caller ignores.
template <bool VEC>
__device__ __forceinline__ float4 load_group_clamped(const SelectParams& p, const float* x, int g,
                                                     int ngroups) {
    const int gc = g < ngroups ? g : ngroups - 1;
    if constexpr (VEC) {
        return reinterpret_cast<const float4*>(x)[gc];
    } else {
        const int i = 4 * gc, last = p.V - 1;
        return make_float4(x[min(i, last)], x[min(i + 1, last)], x[min(i + 2, last)],
                           x[min(i + 3, last)]);
    }
}

// A candidate list entry holds its vocabulary index + 1: the lists are zero between calls, so a
// non-zero entry is a written one. Entries are written once per call with device-scope stores
// (write-through, seen by device-scope loads from any XCD), so the walk of the same launch can
// read each entry as soon as it is non-zero.
__device__ __forceinline__ void put_cand(int32_t* out, uint32_t pos, uint32_t v) {
    __hip_atomic_store(out + pos, (int32_t)(v + 1u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// -inf over group g of the dense output row. COH: device-scope 8-byte stores, complete at the
// device's coherence point when they are acknowledged, so that a walk of the same launch on
// another XCD can then overwrite the candidates' entries without a cache write-back between.
template <bool VEC, bool COH = false>
__device__ __forceinline__ void fill_group(const SelectParams& p, int64_t row, int g) {
    const int i = 4 * g;
    constexpr uint64_t NEG_INF_BF16X4 = 0xFF80FF80FF80FF80ull;
    constexpr uint64_t NEG_INF_F32X2 = 0xFF800000FF800000ull;
    if (p.fill_bf16) {
        uint16_t* o = p.fill_bf16 + row * p.V + i;
        if constexpr (VEC && COH) {
            __hip_atomic_store(reinterpret_cast<uint64_t*>(o), NEG_INF_BF16X4, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        } else if constexpr (VEC) {
            *reinterpret_cast<uint2*>(o) = make_uint2(0xFF80FF80u, 0xFF80FF80u);
        } else {
            for (int u = 0; u < 4; ++u)
                if (i + u < p.V) o[u] = 0xFF80u;
        }
    }
    if (p.fill_f32) {
        float* o = p.fill_f32 + row * p.V + i;
        if constexpr (VEC && COH) {
            uint64_t* o2 = reinterpret_cast<uint64_t*>(o);
            __hip_atomic_store(o2, NEG_INF_F32X2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(o2 + 1, NEG_INF_F32X2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if constexpr (VEC) {
            *reinterpret_cast<float4*>(o) = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        } else {
            for (int u = 0; u < 4; ++u)
                if (i + u < p.V) o[u] = -INFINITY;
        }
    }
}

// The LDS buffer is SEL_WAVES regions of REGION_CAP keys; region r holds cnt[r] keys.
__device__ __forceinline__ bool buf_slot(const uint32_t* cnt, uint32_t e) {
    return e % REGION_CAP < cnt[e / REGION_CAP];
}

// Radix levels over the keys in LDS (all threads): from bit `lo` down, among keys whose bits
// above `lo` equal `prefix`, the need-th largest. The first level below bit 51 takes 12 bits,
// later ones 10 (NBINS = 1024 takes only 10-bit levels). Returns the full 51-bit key, or the
// lowest key of a bin all of whose keys are needed (the same threshold for `>=`). The keys
// are buf[e] for e < n_linear, or, with n_linear < 0, the wave regions of counts cnt.
template <int NBINS = L1_BINS>
__device__ __forceinline__ uint64_t lds_select(const uint64_t* buf, const uint32_t* cnt,
                                               int n_linear, uint32_t need, uint64_t prefix,
                                               int lo, uint32_t* hist, uint32_t* sh, int tid,
                                               int lane) {
    const uint32_t n_slots = n_linear < 0 ? (uint32_t)BUF_CAP : (uint32_t)n_linear;
    while (lo > 0) {
        const int w = lo == CK_BITS ? L1_BITS : (lo < LDS_LEVEL_BITS ? lo : LDS_LEVEL_BITS);
        lo -= w;
        for (int i = tid; i < NBINS; i += SEL_THREADS) hist[i] = 0;
        __syncthreads();
        for (uint32_t e = tid; e < n_slots; e += SEL_THREADS) {
            if (n_linear < 0 && !buf_slot(cnt, e)) continue;
            const uint64_t ck = buf[e];
            if ((ck >> (lo + w)) == prefix) atomicAdd(&hist[(ck >> lo) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        if (tid < WAVE) {
            uint32_t d, above;
            select_digit<NBINS>(hist, need, lane, d, above);
            if (lane == 0) {
                sh[0] = d;
                sh[1] = above;
                sh[5] = hist[d];
            }
        }
        __syncthreads();
        prefix = (prefix << w) | sh[0];
        need -= sh[1];
        // Every key of the chosen bin is needed: the keys >= the bin's lowest possible key are
        // exactly the `need` wanted ones (those of higher bins at every level, and this bin's),
        // so that key serves as the threshold without resolving the lower bits.
        if (sh[5] == need) return prefix << lo;
    }
    return prefix;
}

// Appends the keys >= kth of the buffer whose top 12 bits are `bin` to the candidate row (all
// threads).
__device__ __forceinline__ void emit_from_buffer(const uint64_t* buf, const uint32_t* cnt,
                                                 uint64_t kth, uint32_t bin, int32_t* out,
                                                 uint32_t* n_out, int k, int tid, int lane) {
    for (uint32_t e0 = 0; e0 < (uint32_t)BUF_CAP; e0 += SEL_THREADS) {
        const uint32_t e = e0 + tid;
        const bool in = e < (uint32_t)BUF_CAP && buf_slot(cnt, e) && buf[e] >= kth &&
                        (buf[e] >> L1_SHIFT) == bin;
        const uint32_t po = wave_append(n_out, in, lane);
        if (in && po < (uint32_t)k) put_cand(out, po, composite_index(buf[e]));
    }
}

// The exact path for rows whose first bound lets too many keys through: see the file header.
// Uses region 0's count for the whole buffer (one region of BUF_CAP keys).
template <bool VEC>
__device__ __forceinline__ void select_fallback(const SelectParams& p, const float* x, int32_t* out,
                                                uint64_t* buf, uint32_t* hist, uint32_t* sh,
                                                uint32_t* cnt, int tid, int lane) {
    const int ngroups = (p.V + 3) / 4;
    uint32_t* n_out = sh + 2;
    uint32_t* n_buf = sh + 3;
    for (int i = tid; i < L1_BINS; i += SEL_THREADS) hist[i] = 0;
    if (tid == 0) {
        *n_out = 0;
        *n_buf = 0;
    }
    __syncthreads();
    for (int g = tid; g < ngroups; g += SEL_THREADS) {
        const float4 a = load_group<VEC>(p, x, g);
        const float e[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (4 * g + u < p.V) atomicAdd(&hist[top_bin(e[u])], 1u);
    }
    __syncthreads();
    if (tid < WAVE) {
        uint32_t d, above;
        select_digit<L1_BINS>(hist, (uint32_t)p.k, lane, d, above);
        if (lane == 0) {
            sh[0] = d;
            sh[1] = above;
        }
    }
    __syncthreads();
    const uint32_t d1 = sh[0];
    const uint32_t need = (uint32_t)p.k - sh[1];
    const uint32_t bin_count = hist[d1];
    for (int g0 = 0; g0 < ngroups; g0 += SEL_THREADS) {
        const int g = g0 + tid;
        const float4 a = g < ngroups ? load_group<VEC>(p, x, g) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float e[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = 4 * g + u;
            const bool valid = g < ngroups && i < p.V;
            const uint32_t bin = top_bin(e[u]);
            const bool hi = valid && bin > d1, eq = valid && bin == d1;
            const uint32_t po = wave_append(n_out, hi, lane);
            if (hi && po < (uint32_t)p.k) put_cand(out, po, (uint32_t)i);
            const uint32_t pb = wave_append(n_buf, eq, lane);
            if (eq && pb < (uint32_t)BUF_CAP) buf[pb] = composite_key(e[u], (uint32_t)i);
        }
    }
    __syncthreads();
    if (bin_count <= (uint32_t)BUF_CAP) {
        // the whole buffer as consecutive regions: full ones, then the remainder
        if (tid < SEL_WAVES) {
            const int r = tid;
            const int n = (int)bin_count - r * REGION_CAP;
            cnt[r] = n <= 0 ? 0u : (n >= REGION_CAP ? (uint32_t)REGION_CAP : (uint32_t)n);
        }
        __syncthreads();
        const uint64_t kth = lds_select(buf, cnt, -1, need, d1, L1_SHIFT, hist, sh, tid, lane);
        emit_from_buffer(buf, cnt, kth, d1, out, n_out, p.k, tid, lane);
        return;
    }
    uint64_t prefix = d1;
    uint32_t nd = need;
    int lo = L1_SHIFT;
    while (lo > 0) {
        const int w = lo < GLOBAL_LEVEL_BITS ? lo : GLOBAL_LEVEL_BITS;
        lo -= w;
        for (int i = tid; i < L1_BINS; i += SEL_THREADS) hist[i] = 0;
        __syncthreads();
        for (int g = tid; g < ngroups; g += SEL_THREADS) {
            const float4 a = load_group<VEC>(p, x, g);
            const float e[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = 4 * g + u;
                if (i >= p.V) continue;
                const uint64_t ck = composite_key(e[u], (uint32_t)i);
                if ((ck >> (lo + w)) == prefix) atomicAdd(&hist[(ck >> lo) & ((1u << w) - 1u)], 1u);
            }
        }
        __syncthreads();
        if (tid < WAVE) {
            uint32_t d, above;
            select_digit<L1_BINS>(hist, nd, lane, d, above);
            if (lane == 0) {
                sh[0] = d;
                sh[1] = above;
            }
        }
        __syncthreads();
        prefix = (prefix << w) | sh[0];
        nd -= sh[1];
    }
    const uint64_t kth = prefix;
    for (int g0 = 0; g0 < ngroups; g0 += SEL_THREADS) {
        const int g = g0 + tid;
        const float4 a = g < ngroups ? load_group<VEC>(p, x, g) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float e[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = 4 * g + u;
            const uint64_t ck = composite_key(e[u], (uint32_t)i);
            const bool in = g < ngroups && i < p.V && (ck >> L1_SHIFT) == d1 && ck >= kth;
            const uint32_t po = wave_append(n_out, in, lane);
            if (in && po < (uint32_t)p.k) put_cand(out, po, (uint32_t)i);
        }
    }
}

// (2 workgroups per CU: at most 128 VGPRs, i.e. 4 waves per SIMD)
// The k best keys of one base row (all threads of a workgroup of SEL_THREADS), with the row's
// -inf fill when asked for; smem holds SEL_LDS_BYTES.
template <bool VEC, bool TIMED, bool COH = false>
__device__ __forceinline__ void select_row(const SelectParams& p, const int64_t row,
                                           unsigned char* smem) {
    uint64_t* buf = reinterpret_cast<uint64_t*>(smem);
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + BUF_CAP * 8);
    uint32_t* sh = hist + L1_BINS;  // [0] digit, [1] count above, [2] n_out, [3] n_buf,
                                    // [4] keys of the k-th key's bin, [16 .. 31] per-wave
                                    // counts of the compaction
    uint32_t* cnt = sh + 8;         // [8 .. 15] keys per wave region
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    const float* x = p.base + row * p.V;
    int32_t* out = p.cand + row * p.k;
    const int ngroups = (p.V + 3) / 4;
    tk_stamp<TIMED>(p.stamps, row * 8 + 0);

    for (int i = tid; i < L1_BINS; i += SEL_THREADS) hist[i] = 0;
    if (tid == 0) {
        sh[2] = 0;
        sh[3] = 0;
    }
    // the first chunk into registers
    float4 stash[STASH_GROUPS];
#pragma unroll
    for (int s = 0; s < STASH_GROUPS; ++s) {
        const int g = s * SEL_THREADS + tid;
        stash[s] = load_group_clamped<VEC>(p, x, g, ngroups);
    }
    // and the first batch of the main pass, so that it is in flight while the chunk's histogram
    // and bound are computed (every workgroup starts at once, so HBM would idle meanwhile)
    // (rows without float4 loads take half batches: their scalar loads need more address
    // registers)
    constexpr int MU = VEC ? MAIN_UNROLL : MAIN_UNROLL / 2;
    constexpr int BATCH = MU * SEL_THREADS;
    int g0 = STASH_GROUPS * SEL_THREADS;
    float4 cur[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
        const int g = g0 + u * SEL_THREADS + tid;
        cur[u] = load_group_clamped<VEC>(p, x, g, ngroups);
    }
    __syncthreads();
    // its top-12-bit histogram; -inf over the output
#pragma unroll
    for (int s = 0; s < STASH_GROUPS; ++s) {
        const int g = s * SEL_THREADS + tid;
        if (g < ngroups) {
            const float e[4] = {stash[s].x, stash[s].y, stash[s].z, stash[s].w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (VEC || 4 * g + u < p.V) atomicAdd(&hist[top_bin(e[u])], 1u);
            fill_group<VEC, COH>(p, row, g);
        }
    }
    __syncthreads();
    // The bound: the bin of the chunk's kb-th largest key. When the chunk is the whole row, kb
    // = k. Otherwise kb = ceil(2 k chunk / V), twice the chunk's expected share of the row's top
    // k (at most k): on a row without order about 2k keys then reach the bound, not k V / chunk,
    // and fewer of the scan's groups hold a key that does. A row where fewer than k keys reach
    // it (the chunk holding more than its share of the top) takes the exact fallback.
    uint32_t kb = (uint32_t)p.k;
    if (p.V > STASH_ELEMS) {
        const int64_t e = (2 * (int64_t)p.k * STASH_ELEMS + p.V - 1) / p.V;
        kb = (uint32_t)(e < 1 ? 1 : e < p.k ? e : p.k);
    }
    if (tid < WAVE) {
        uint32_t d, above;
        select_digit<L1_BINS>(hist, kb, lane, d, above);
        if (lane == 0) sh[0] = d;
    }
    __syncthreads();
    const uint32_t bin_lo = sh[0];
    tk_stamp<TIMED>(p.stamps, row * 8 + 1);
    for (int i = tid; i < L1_BINS; i += SEL_THREADS) hist[i] = 0;  // now: the offered keys
    __syncthreads();

    // Every key in a bin >= bin_lo goes into this wave's LDS region (wave-uniform count, no
    // atomics for the position). Membership is one float compare per
    // element: the keys order values as IEEE comparison does (-0 with +0), with NaN above +inf,
    // so "key >= the bin's lowest key B" is "not (x < t)" for t the value whose key is B (NaN
    // passes, as it should). The bins below -inf's key hold no value (t = -inf admits all).
    // Those above +inf's hold only NaN: t = +inf then also admits +inf, a key below the bound.
    // Extra keys below the bound are harmless: at least k keys reach it, so the k-th largest
    // offered key, and every key the select emits, is one of those.
    const uint32_t kB = bin_lo << (32 - L1_BITS);
    const float t_lo = kB <= ORDER_KEY_NEG_INF ? -INFINITY
                       : kB > 0xFF800000u      ? INFINITY
                       : kB >= 0x80000000u     ? __uint_as_float(kB & 0x7FFFFFFFu)
                                               : __uint_as_float(~kB);
    uint64_t* region = buf + wave * REGION_CAP;
    uint32_t n_region = 0;
    // The scan stores each member as its raw (index, value bits) pair: element u of the group
    // goes to the position given by the members of element u in the lanes below (one ballot per
    // element). Order keys and the histogram are made after the scan, over the region only, so
    // that the streaming loop does the least work per element.
    auto offer = [&](const float4 a, int g, bool present) {
        const float e[4] = {a.x, a.y, a.z, a.w};
        bool in[4];
        uint64_t m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            in[u] = present && (VEC || 4 * g + u < p.V) && !(e[u] < t_lo);
            m[u] = __ballot(in[u]);
        }
        if ((m[0] | m[1] | m[2] | m[3]) == 0) return;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (m[u] == 0) continue;
            const uint32_t pos = n_region + lanes_below(m[u]);
            if (in[u] && pos < (uint32_t)REGION_CAP)
                region[pos] = ((uint64_t)(uint32_t)(4 * g + u) << 32) | __float_as_uint(e[u]);
            n_region += (uint32_t)__popcll(m[u]);
        }
    };
#pragma unroll
    for (int s = 0; s < STASH_GROUPS; ++s) {
        const int g = s * SEL_THREADS + tid;
        offer(stash[s], g, g < ngroups);
    }
    // The rest of the row in two register sets used in turn, so that one batch is in flight
    // while the other is examined and no loaded value is ever copied between registers (a copy
    // would wait for its load).
    for (; g0 < ngroups; g0 += 2 * BATCH) {
        float4 nxt[MU];
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            const int g = g0 + BATCH + u * SEL_THREADS + tid;
            nxt[u] = load_group_clamped<VEC>(p, x, g, ngroups);
        }
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            const int g = g0 + u * SEL_THREADS + tid;
            offer(cur[u], g, g < ngroups);
            if (g < ngroups) fill_group<VEC, COH>(p, row, g);
        }
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            const int g = g0 + 2 * BATCH + u * SEL_THREADS + tid;
            cur[u] = load_group_clamped<VEC>(p, x, g, ngroups);
        }
#pragma unroll
        for (int u = 0; u < MU; ++u) {
            const int g = g0 + BATCH + u * SEL_THREADS + tid;
            offer(nxt[u], g, g < ngroups);
            if (g < ngroups) fill_group<VEC, COH>(p, row, g);
        }
    }
    // the region's pairs to order keys, counted in the histogram of the offered keys
    {
        const uint32_t n = n_region < (uint32_t)REGION_CAP ? n_region : (uint32_t)REGION_CAP;
        for (uint32_t e = lane; e < n; e += WAVE) {
            const uint64_t r = region[e];
            const float v = __uint_as_float((uint32_t)r);
            atomicAdd(&hist[top_bin(v)], 1u);
            region[e] = composite_key(v, (uint32_t)(r >> 32));
        }
    }
    // COH: every -inf fill store of the row is acknowledged before any candidate entry is
    // written (those come after this barrier), so a reader that sees an entry also sees the fill
    if constexpr (COH) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) cnt[wave] = n_region;
    __syncthreads();
    tk_stamp<TIMED>(p.stamps, row * 8 + 2);
    bool overflow = false;
    uint32_t offered = 0;
#pragma unroll
    for (int r = 0; r < SEL_WAVES; ++r) {
        overflow = overflow || cnt[r] > (uint32_t)REGION_CAP;
        offered += cnt[r];
    }
    // too many keys for the buffer, or too few reached the bound to hold the row's top k
    if (overflow || offered < (uint32_t)p.k) {
        select_fallback<VEC>(p, x, out, buf, hist, sh, cnt, tid, lane);
        tk_stamp<TIMED>(p.stamps, row * 8 + 4);
        return;
    }
    // the bin d1 of the k-th key, from the histogram of the offered keys
    if (tid < WAVE) {
        uint32_t d, above;
        select_digit<L1_BINS>(hist, (uint32_t)p.k, lane, d, above);
        if (lane == 0) {
            sh[0] = d;
            sh[1] = above;
            sh[4] = 0;  // keys of bin d1 collected below
        }
    }
    __syncthreads();
    tk_stamp<TIMED>(p.stamps, row * 8 + 5);
    const uint32_t d1 = sh[0];
    const uint32_t need = (uint32_t)p.k - sh[1];
    // Keys above bin d1 are in; those of bin d1 go to a small list in the first half of the
    // histogram's memory (no longer needed). Each wave counts its own region's keys of both
    // kinds, the waves take consecutive ranges of the outputs, then each writes its keys: no
    // atomics. (A bin too large for the list takes radix levels over the whole buffer.)
    constexpr uint32_t SMALL_CAP = 1024;
    uint64_t* small = reinterpret_cast<uint64_t*>(hist);
    uint32_t* hist2 = hist + 2 * SMALL_CAP;          // 1024 bins after the small list
    // This wave's region (n_mine <= REGION_CAP here: no overflow) is read into registers once,
    // all reads issued together, for both passes below.
    constexpr int MINE_REGS = (REGION_CAP + WAVE - 1) / WAVE;
    const uint64_t* mine = buf + wave * REGION_CAP;
    const uint32_t n_mine = cnt[wave];
    uint64_t mk[MINE_REGS];
#pragma unroll
    for (int i = 0; i < MINE_REGS; ++i) {
        const uint32_t e = (uint32_t)(i * WAVE + lane);
        mk[i] = e < n_mine ? mine[e] : 0ull;
    }
    uint32_t n_hi = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < MINE_REGS; ++i) {
        const uint32_t e = (uint32_t)(i * WAVE + lane);
        const uint32_t bin = (uint32_t)(mk[i] >> L1_SHIFT);
        n_hi += (uint32_t)__popcll(__ballot(e < n_mine && bin > d1));
        n_eq += (uint32_t)__popcll(__ballot(e < n_mine && bin == d1));
    }
    __syncthreads();  // every wave is past select_digit's reads of the histogram
    uint32_t* wc = sh + 16;  // [16 + w] keys above d1, [24 + w] keys of d1, per wave
    if (lane == 0) {
        wc[wave] = n_hi;
        wc[SEL_WAVES + wave] = n_eq;
    }
    __syncthreads();
    uint32_t off_hi = 0, off_eq = 0, m = 0;
#pragma unroll
    for (int w = 0; w < SEL_WAVES; ++w) {
        off_hi += w < wave ? wc[w] : 0u;
        off_eq += w < wave ? wc[SEL_WAVES + w] : 0u;
        m += wc[SEL_WAVES + w];
    }
#pragma unroll
    for (int i = 0; i < MINE_REGS; ++i) {
        const uint32_t e = (uint32_t)(i * WAVE + lane);
        const uint64_t ck = mk[i];
        const uint32_t bin = (uint32_t)(ck >> L1_SHIFT);
        const bool hi = e < n_mine && bin > d1, eq = e < n_mine && bin == d1;
        const uint64_t mh = __ballot(hi), me = __ballot(eq);
        const uint32_t ph = off_hi + lanes_below(mh), pe = off_eq + lanes_below(me);
        if (hi && ph < (uint32_t)p.k) put_cand(out, ph, composite_index(ck));
        if (eq && pe < SMALL_CAP) small[pe] = ck;
        off_hi += (uint32_t)__popcll(mh);
        off_eq += (uint32_t)__popcll(me);
    }
    if (tid == 0) sh[2] = (uint32_t)p.k - need;  // keys emitted so far (all above bin d1)
    __syncthreads();
    tk_stamp<TIMED>(p.stamps, row * 8 + 6);
    if (m <= SMALL_CAP) {
        const uint64_t kth = lds_select<1024>(small, cnt, (int)m, need, d1, L1_SHIFT, hist2, sh,
                                              tid, lane);
        tk_stamp<TIMED>(p.stamps, row * 8 + 3);
        for (uint32_t e0 = 0; e0 < m; e0 += SEL_THREADS) {
            const uint32_t e = e0 + tid;
            const bool in = e < m && small[e] >= kth;
            const uint32_t po = wave_append(sh + 2, in, lane);
            if (in && po < (uint32_t)p.k) put_cand(out, po, composite_index(small[e]));
        }
    } else {
        // radix levels over the whole buffer (still intact)
        const uint64_t kth = lds_select(buf, cnt, -1, need, d1, L1_SHIFT, hist, sh, tid, lane);
        tk_stamp<TIMED>(p.stamps, row * 8 + 3);
        emit_from_buffer(buf, cnt, kth, d1, out, sh + 2, p.k, tid, lane);
    }
    tk_stamp<TIMED>(p.stamps, row * 8 + 4);
}

template <bool VEC, bool TIMED>
__global__ __launch_bounds__(SEL_THREADS, 4) void topk_select_kernel(const SelectParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    select_row<VEC, TIMED>(p, blockIdx.x, smem);
}

struct TopkWalkParams {
    const int8_t* q;
    const float* scale;
    const void* w1;
    const float* base;
    const int32_t* start;
    int32_t* tokens;
    float* out_f32;        // greedy: dense fp32 logits row, or null
    uint16_t* out_bf16;    // sample: dense bf16 logits row
    const uint64_t* seeds;
    const int64_t* positions;
    const float* temps;
    int32_t* cand;         // [bs][T][k] from topk_select_kernel; cleared at the end
    uint32_t* err;
    uint64_t* stamps;      // instrumented builds
    const float* w2_bound; // pruned greedy walk: the load-time bound B (see dspark_w2_prune_bound)
    int32_t* dense_steps;  // pruned greedy walk: per request, steps computed over the whole row
    int bs, T, V, k;
};

// Value of the float whose order key is the high word of `key` (order_key32 inverted; every
// NaN maps back to a NaN, the canonical zero to +0).
__device__ __forceinline__ float key_value(uint64_t key) {
    const uint32_t k32 = (uint32_t)(key >> 32);
    return __uint_as_float((k32 & 0x80000000u) ? (k32 & 0x7FFFFFFFu) : ~k32);
}

// The 64 candidates of one wave for one step. Rows are read cooperatively so that every load
// instruction fetches whole cache lines: in load i (0..15) the 16 lanes of lane group r (lanes
// 16r .. 16r+15) read the 16-byte chunks of the row of candidate 4i + r, lane 16r + c taking
// chunk c. Lane 16r + i owns candidate 4i + r: its scale, base logit and vocabulary index.
struct CandBlock {
    int4 q[RANK / 16];  // q[i]: chunk (lane & 15) of the row of candidate 4i + (lane >> 4)
    float s, base;
    uint32_t v;
};

// Sum over each 16-lane row of the wave (every lane of the row gets it).
__device__ __forceinline__ int row16_sum_i32(int x) {
    x += (int)dpp_u32<DPP_SWAP1>((uint32_t)x);
    x += (int)dpp_u32<DPP_SWAP2>((uint32_t)x);
    x += (int)dpp_u32<DPP_HALF_MIRROR>((uint32_t)x);
    x += (int)dpp_u32<DPP_MIRROR>((uint32_t)x);
    return x;
}

// The exact int32 dot of W1 codes with the W2 row of this lane's candidate: lane group r's 16
// lanes hold the rows of candidates 4i + r in load i, each lane one 16-byte chunk; lane 16r + i
// ends with candidate 4i + r's sum, 16 * (high digits' products) + (low digits' products).
__device__ __forceinline__ int cand_dot(const CandBlock& blk, const int4 wc, const int4 wl,
                                        int lane) {
    int acc = 0;
#pragma unroll
    for (int i = 0; i < RANK / 16; ++i) {
        int d = __builtin_amdgcn_sdot4(blk.q[i].x, wc.x, 0, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].y, wc.y, d, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].z, wc.z, d, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].w, wc.w, d, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].x, wl.x, d << 4, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].y, wl.y, d, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].z, wl.z, d, false);
        d = __builtin_amdgcn_sdot4(blk.q[i].w, wl.w, d, false);
        d = row16_sum_i32(d);
        acc = (lane & 15) == i ? d : acc;
    }
    return acc;
}

// MULTI: k > TKW_THREADS, candidates in several chunks per step, loaded as they are scored;
// otherwise one candidate per thread, the next step's loaded while this step is scored.
// PRUNE (greedy only): the lossless top-k pruned walk. Its result is the dense greedy walk's:
// a step keeps its candidates' argmax only when no other row can reach it. Every non-candidate
// v has base[v] <= kth (the smallest candidate base logit) and |bias(v)| <= B * a, with B the
// load-time bound max_v s[v] * sum_k |q[v,k]| and a = max_k |W1[prev,k]| (the codes times their
// scale never exceed a), so its logit is at most kth + B * a up to rounding. The step is
// certified when the best candidate logit exceeds that by a relative margin of 2^-16 (far above
// the few ulps of rounding in either logit); otherwise, and whenever a value is not finite, the
// step is computed over every row, as the dense walk does, with the same rounding.
template <int SAMPLE, int W1T, bool MULTI, bool TIMED, bool PRUNE = false>
__global__ __launch_bounds__(TKW_THREADS) void topk_walk_kernel(const TopkWalkParams p) {
    __shared__ __align__(16) uint32_t w1q[TKW_WAVES][RANK / 4];  // one copy per wave: high
    __shared__ __align__(16) uint32_t w1l[TKW_WAVES][RANK / 4];  // and low W1 digits
    __shared__ uint64_t wkeys[2][TKW_WAVES];                      // by step parity
    __shared__ float wmin[2][TKW_WAVES];                          // PRUNE: smallest candidate base
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    const int b = blockIdx.x;
    const int64_t st0 = TK_WALK_STAMPS0 + (int64_t)b * 40;
    tk_stamp<TIMED>(p.stamps, st0);

    int prev = p.start[b];
    if (prev < 0 || prev >= p.V) {
        if (tid == 0) flag_error(p.err, DSPARK_ERR_INVALID_ARG);
        prev = 0;
    }
    uint64_t seed = 0, P0 = 0;
    float rtemp = 1.0f;
    if constexpr (SAMPLE) {
        seed = p.seeds[b];
        P0 = p.positions ? (uint64_t)p.positions[b] : 0;
        rtemp = inv_temperature(p.temps[b]);
    }
    const int32_t* req_cand = p.cand + (int64_t)b * p.T * p.k;
    const float w2_bound = PRUNE ? p.w2_bound[0] : 0.0f;
    int dense_count = 0;
    const int own = (lane & 15) * 4 + (lane >> 4);  // this lane's candidate within the wave's 64
    // raw index of candidate j of step t (j clamped into the list; load_block bounds the value)
    auto cand_index = [&](int t, int j) -> uint32_t {
        return (uint32_t)req_cand[(int64_t)t * p.k + min(j, p.k - 1)] - 1u;
    };
    auto load_block = [&](int t, uint32_t own_idx, CandBlock& blk) {
        const uint32_t v = own_idx < (uint32_t)p.V ? own_idx : 0u;  // always: select emits rows
        blk.v = v;
        blk.s = p.scale[v];
        blk.base = p.base[((int64_t)b * p.T + t) * p.V + v];
        const int c = lane & 15;
#pragma unroll
        for (int i = 0; i < RANK / 16; ++i) {
            const uint32_t vi = (uint32_t)__shfl((int)v, (lane & 48) | i);
            blk.q[i] = reinterpret_cast<const int4*>(p.q + (int64_t)vi * RANK)[c];
        }
    };

    // One step: this wave's copy of the W1 codes of the previous token (no workgroup barrier
    // for it), the candidates' logits and keys, then one barrier for the step's argmax. The
    // next step's rows load into `fill` (from `fill_idx`, loaded a step earlier) while the W1
    // row is in flight, and the index two steps ahead into `next_idx`.
    // When sampling, the candidates' bf16 logits go to the dense output one step late. Stores
    // share the in-order count of vector memory operations with loads, so a store issued at the
    // end of a step would hold the next step's wait for its W1 row until the store completed.
    // Issued after that W1 load instead, it has the whole next step to complete. (One candidate
    // per lane; a lane with none holds pend_off < 0.) The greedy walk stores only when its fp32
    // logits are asked for, and stores at once: the pending state cost its timed configuration,
    // which stores nothing, more than it saved.
    constexpr bool DEFER = SAMPLE && !MULTI;
    int64_t pend_off = -1;
    uint32_t pend_val = 0;
    auto flush_pending = [&]() {
        if constexpr (DEFER)
            if (pend_off >= 0) p.out_bf16[pend_off] = (uint16_t)pend_val;
    };
    auto step = [&](int t, CandBlock& use, CandBlock& fill, uint32_t fill_idx, uint32_t& next_idx) {
        const int64_t row = (int64_t)b * p.T + t;
        const float4 w = load4_as_f32<W1T>(p.w1, (int64_t)prev * RANK + lane * 4);
        if constexpr (!MULTI) {
            // Vector loads complete in issue order, so the order of issue is chosen: the W1 row
            // first (its wait then covers nothing else), the index two steps ahead next (the
            // next step waits for it before its rows, and then waits for nothing issued after
            // it), the next step's rows last. The scheduling barrier keeps the rows there; left to
            // itself the scheduler sank the rows below the wait for the W1 row.
            next_idx = cand_index(min(t + 2, p.T - 1), wave * WAVE + own);
            // unconditional (past the last step they re-read the last step's rows), so that
            // no branch keeps the compiler from counting the loads in flight
            load_block(min(t + 1, p.T - 1), fill_idx, fill);
            __builtin_amdgcn_sched_barrier(0);
            flush_pending();   // the previous step's logit, behind this step's loads
        }
        float a = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
        a = wave_max_nonneg_f32(a);
        const float inv = w1_code_scale(a);
        const float sb = w1_code_step(a);
        uint32_t lo, nib;
        w1q[wave][lane] = pack_codes(w, inv, lo, nib);
        w1l[wave][lane] = lo;
        tk_stamp<TIMED>(p.stamps, st0 + 1 + 2 * t);
        const int4 wc = reinterpret_cast<const int4*>(w1q[wave])[lane & 15];
        const int4 wl = reinterpret_cast<const int4*>(w1l[wave])[lane & 15];
        uint64_t best = 0;
        float min_base = INFINITY;
        auto score = [&](const CandBlock& blk, bool has) {
            const int acc = cand_dot(blk, wc, wl, lane);
            const float l = walk_logit(blk.base, blk.s, sb, acc);
            uint64_t key;
            const int64_t off = row * p.V + blk.v;
            if constexpr (!SAMPLE) {
                if (has && p.out_f32) p.out_f32[off] = l;
                key = argmax_key(l, blk.v);
            } else {
                const uint32_t h = bf16_bits(l);
                if constexpr (DEFER) {
                    pend_off = has ? off : -1;
                    pend_val = h;
                } else {
                    if (has) p.out_bf16[off] = (uint16_t)h;
                }
                const float xs = bf16_value(h) * rtemp;
                const float g = gumbel_from_word(noise_word(seed, P0 + (uint64_t)t, blk.v));
                key = argmax_key(xs + g, blk.v);
            }
            if (has) best = key > best ? key : best;
            if constexpr (PRUNE)
                if (has) min_base = fminf(min_base, blk.base);
        };
        if constexpr (MULTI) {
            for (int c0 = 0; c0 < p.k; c0 += TKW_THREADS) {
                const int j = c0 + wave * WAVE + own;
                load_block(t, cand_index(t, j), use);
                score(use, j < p.k);
            }
        } else {
            score(use, wave * WAVE + own < p.k);
        }
        best = wave_max_u64(best);
        if constexpr (PRUNE) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) min_base = fminf(min_base, __shfl_xor(min_base, o, WAVE));
            if (lane == 0) wmin[t & 1][wave] = min_base;
        }
        if (lane == 0) wkeys[t & 1][wave] = best;
        __syncthreads();
        uint64_t m = wkeys[t & 1][0];
#pragma unroll
        for (int w2 = 1; w2 < TKW_WAVES; ++w2) m = wkeys[t & 1][w2] > m ? wkeys[t & 1][w2] : m;
        if constexpr (PRUNE) {
            float kth = wmin[t & 1][0];
#pragma unroll
            for (int w2 = 1; w2 < TKW_WAVES; ++w2) kth = fminf(kth, wmin[t & 1][w2]);
            const float lstar = key_value(m);
            const float reach = w2_bound * a;        // bound on any row's |bias| this step
            const float margin = (fabsf(lstar) + fabsf(kth) + reach) * 0x1p-16f;
            // false for any NaN or infinity (then the difference or the margin is not finite)
            const bool certified = lstar - kth > reach + margin;
            if (!certified) {
                // the whole row, every row scored as the dense walk scores it
                best = 0;
                for (int r0 = 0; r0 < p.V; r0 += TKW_THREADS) {
                    const int j = r0 + wave * WAVE + own;
                    load_block(t, (uint32_t)min(j, p.V - 1), use);
                    score(use, j < p.V);
                }
                best = wave_max_u64(best);
                __syncthreads();                     // every wave has read this step's keys
                if (lane == 0) wkeys[t & 1][wave] = best;
                __syncthreads();
                m = wkeys[t & 1][0];
#pragma unroll
                for (int w2 = 1; w2 < TKW_WAVES; ++w2)
                    m = wkeys[t & 1][w2] > m ? wkeys[t & 1][w2] : m;
                ++dense_count;
            }
        }
        // every candidate at -inf: the dense row is -inf throughout, whose first max is 0
        uint32_t token = (uint32_t)(m >> 32) <= ORDER_KEY_NEG_INF ? 0u : key_index(m);
        if (token >= (uint32_t)p.V) token = 0;
        if (tid == 0) p.tokens[b * p.T + t] = (int32_t)token;
        prev = (int)token;
        tk_stamp<TIMED>(p.stamps, st0 + 2 + 2 * t);
    };

    CandBlock ra, rb;  // alternate between steps: one is scored while the other fills
    uint32_t ia = 0, ib = 0;
    if (!MULTI) {
        load_block(0, cand_index(0, wave * WAVE + own), ra);
        ib = cand_index(min(1, p.T - 1), wave * WAVE + own);
    }
    for (int t = 0; t < p.T; t += 2) {
        step(t, ra, rb, ib, ia);
        if (t + 1 < p.T) step(t + 1, rb, ra, ia, ib);
    }
    flush_pending();   // the last step's logit (sampling)
    if constexpr (PRUNE)
        if (tid == 0 && p.dense_steps) p.dense_steps[b] = dense_count;
    // every candidate list of this request has been read before the last barrier: clear them,
    // so that the workspace is all zero again for the dense walk
    __syncthreads();
    int32_t* clr = p.cand + (int64_t)b * p.T * p.k;
    for (int i = tid; i < p.T * p.k; i += TKW_THREADS) clr[i] = 0;
}

// ---- select and walk in one launch (k <= TKW_THREADS, rows that allow float4 loads) ----------
// Rows are listed in step-major order (every request's step 0 first), and the workgroups of step 0
// then walk their request. The dispatcher places the first F = min(rows, CUs) workgroups one per
// CU and the rest second on CUs in the same order, so the last of the first F hold a CU alone
// when the rows fit two per CU. Those take the step-0 rows (their rows finish soonest, and the
// walks run without a select on their CU); the others among the first F take steps 1, 2, ... in
// order. When all rows fit two per CU, the workgroups placed second take the remaining rows in
// reverse, so that the rows finishing last belong to the last steps. With more rows, the rest
// keep step order: the workgroups dispatched as others finish then take the latest steps. Any
// order is correct; this one makes the walks wait least. A step reads its row's candidate entries as soon
// as they are written (non-zero, see put_cand), and the row's -inf fill is complete by then (the
// fill stores are acknowledged before the first entry is written). The walk of a request thus
// starts as soon as its first row is selected, while the rows of later steps are still being read:
// in the two-launch form every walk waits for the last row of the whole batch. Workgroups are
// dispatched in index order and only the bs walkers wait, so a row's workgroup is always resident
// or dispatched once another finishes; each wait is still bounded in time (it then flags
// DSPARK_ERR_TIMEOUT and goes on).
struct FusedParams {
    SelectParams s;
    TopkWalkParams w;
    const uint32_t* never;  // a word that stays zero (test hook: waits that cannot end)
    uint32_t spin_ticks;
    int wait_unset;
    int first_slots;        // the device's compute units (at least bs)
};

// A candidate entry of step `row`: a device-scope load (no stale line of another call serves it).
__device__ __forceinline__ uint32_t load_entry(const TopkWalkParams& p, int64_t row, int j) {
    return (uint32_t)__hip_atomic_load(p.cand + row * p.k + min(j, p.k - 1), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide wait until every lane's entry `e` (loaded earlier) is written; reloads it meanwhile.
// The compiler barrier keeps the loads that use the entry below the loop.
__device__ __forceinline__ uint32_t wait_entry(const FusedParams& fp, uint32_t e, int64_t row,
                                               int j, int lane) {
    const WaitBound wait;
    while (true) {
        const uint64_t now = WaitBound::now();
        bool ok = e != 0;
        if (fp.wait_unset)
            ok = ok && __hip_atomic_load(fp.never, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
        if (__all(ok)) break;
        if (wait.expired(now, fp.spin_ticks)) {
            if (lane == 0) flag_error(fp.w.err, DSPARK_ERR_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
        e = load_entry(fp.w, row, j);
    }
    asm volatile("" ::: "memory");
    return e;
}

// PRUNE (greedy only): the lossless pruned walk, as in topk_walk_kernel. A step that is not
// certified is computed over every row with few registers (the next step's candidate rows stay
// where they are): each wave takes 8 rows per pass, two per 16-lane group.
template <int SAMPLE, int W1T, bool TIMED, bool PRUNE = false>
__global__ __launch_bounds__(SEL_THREADS, 4) void topk_fused_kernel(const FusedParams fp) {
    static_assert(!(PRUNE && SAMPLE), "the pruned walk is greedy");
    extern __shared__ __align__(16) unsigned char smem[];
    const TopkWalkParams& p = fp.w;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
    const int i = blockIdx.x, n = p.bs * p.T;
    const int F = n < fp.first_slots ? n : fp.first_slots;   // >= bs
    const int lin = i < F - p.bs ? i + p.bs
                    : i < F      ? i - (F - p.bs)
                    : n <= 2 * F ? F + (n - 1 - i)
                                 : i;
    const int t0 = lin / p.bs, b = lin - t0 * p.bs;
    select_row<true, TIMED, true>(fp.s, (int64_t)b * p.T + t0, smem);
    if (t0 != 0) return;
    __syncthreads();  // the select's LDS is free from here on

    // the walk of request b
    uint32_t* w1q = reinterpret_cast<uint32_t*>(smem) + wave * (RANK / 4);   // high digits
    uint32_t* w1l = w1q + SEL_WAVES * (RANK / 4);                            // low digits
    uint64_t* wkeys = reinterpret_cast<uint64_t*>(smem + 2 * SEL_WAVES * RANK);  // [2][waves]
    float* wmin = reinterpret_cast<float*>(wkeys + 2 * SEL_WAVES);              // [2][waves]
    const int64_t st0 = TK_WALK_STAMPS0 + (int64_t)b * 40;
    tk_stamp<TIMED>(p.stamps, st0);
    int prev = p.start[b];
    if (prev < 0 || prev >= p.V) {
        if (tid == 0) flag_error(p.err, DSPARK_ERR_INVALID_ARG);
        prev = 0;
    }
    uint64_t seed = 0, P0 = 0;
    float rtemp = 1.0f;
    if constexpr (SAMPLE) {
        seed = p.seeds[b];
        P0 = p.positions ? (uint64_t)p.positions[b] : 0;
        rtemp = inv_temperature(p.temps[b]);
    }
    const float w2_bound = PRUNE ? p.w2_bound[0] : 0.0f;
    int dense_count = 0;
    const int own = (lane & 15) * 4 + (lane >> 4);  // this lane's candidate within the wave's 64
    const int j = wave * WAVE + own;
    const bool has = j < p.k;
    const int64_t row0 = (int64_t)b * p.T;
    // Step t's candidate rows from its entry e (written): W2 row (whole lines per load, as in the
    // two-launch walk), scale and base logit.
    CandBlock blk;
    auto load_rows = [&](int t, uint32_t e) {
        const uint32_t ci = e - 1u;
        const uint32_t v = ci < (uint32_t)p.V ? ci : 0u;
        blk.v = v;
        blk.s = p.scale[v];
        blk.base = p.base[(row0 + t) * p.V + v];
        const int c = lane & 15;
#pragma unroll
        for (int r = 0; r < RANK / 16; ++r) {
            const uint32_t vi = (uint32_t)__shfl((int)v, (lane & 48) | r);
            blk.q[r] = reinterpret_cast<const int4*>(p.q + (int64_t)vi * RANK)[c];
        }
    };
    // The entry of the next step is loaded a step ahead, without waiting: when its step comes it
    // has usually been written already, and then the rows load without a dependent entry load.
    uint32_t e_next = 0;
    load_rows(0, wait_entry(fp, load_entry(p, row0, j), row0, j, lane));
    if (p.T > 1) e_next = load_entry(p, row0 + 1, j);
    for (int t = 0; t < p.T; ++t) {
        const int64_t row = row0 + t;
        const float4 w = load4_as_f32<W1T>(p.w1, (int64_t)prev * RANK + lane * 4);
        float a = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
        a = wave_max_nonneg_f32(a);
        const float inv = w1_code_scale(a);
        const float sb = w1_code_step(a);
        uint32_t lo, nib;
        w1q[lane] = pack_codes(w, inv, lo, nib);
        w1l[lane] = lo;
        tk_stamp<TIMED>(p.stamps, st0 + 1 + 2 * t);
        const int4 wc = reinterpret_cast<const int4*>(w1q)[lane & 15];
        const int4 wl = reinterpret_cast<const int4*>(w1l)[lane & 15];
        const int acc = cand_dot(blk, wc, wl, lane);
        const float l = walk_logit(blk.base, blk.s, sb, acc);
        const int64_t off = row * p.V + blk.v;
        uint64_t key;
        if constexpr (!SAMPLE) {
            if (has && p.out_f32) p.out_f32[off] = l;
            key = argmax_key(l, blk.v);
        } else {
            const uint32_t h = bf16_bits(l);
            if (has) p.out_bf16[off] = (uint16_t)h;
            const float xs = bf16_value(h) * rtemp;
            const float g = gumbel_from_word(noise_word(seed, P0 + (uint64_t)t, blk.v));
            key = argmax_key(xs + g, blk.v);
        }
        float min_base = INFINITY;
        if constexpr (PRUNE) min_base = has ? blk.base : INFINITY;
        // the next step's rows load while this step's argmax is combined
        if (t + 1 < p.T) {
            load_rows(t + 1, wait_entry(fp, e_next, row + 1, j, lane));
            if (t + 2 < p.T) e_next = load_entry(p, row + 2, j);
        }
        const uint64_t best = wave_max_u64(has ? key : 0ull);
        if (lane == 0) wkeys[(t & 1) * SEL_WAVES + wave] = best;
        if constexpr (PRUNE) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) min_base = fminf(min_base, __shfl_xor(min_base, o, WAVE));
            if (lane == 0) wmin[(t & 1) * SEL_WAVES + wave] = min_base;
        }
        __syncthreads();
        uint64_t m = wkeys[(t & 1) * SEL_WAVES];
#pragma unroll
        for (int w2 = 1; w2 < SEL_WAVES; ++w2) {
            const uint64_t o = wkeys[(t & 1) * SEL_WAVES + w2];
            m = o > m ? o : m;
        }
        if constexpr (PRUNE) {
            float kth = wmin[(t & 1) * SEL_WAVES];
#pragma unroll
            for (int w2 = 1; w2 < SEL_WAVES; ++w2) kth = fminf(kth, wmin[(t & 1) * SEL_WAVES + w2]);
            const float lstar = key_value(m);
            const float reach = w2_bound * a;        // bound on any row's |bias| this step
            const float margin = (fabsf(lstar) + fabsf(kth) + reach) * 0x1p-16f;
            // false for any NaN or infinity (then the difference or the margin is not finite)
            if (!(lstar - kth > reach + margin)) {
                // Every row of the step, scored as the dense walk scores it: per pass, lane
                // group g (lanes 16g .. 16g+15) takes rows r0 + 4i + g, i = 0..1, each lane one
                // 16-byte chunk of W2; lane 16g + i then finishes row r0 + 4i + g.
                const int g = lane >> 4, c = lane & 15;
                const int4 wc2 = reinterpret_cast<const int4*>(w1q)[c];
                const int4 wl2 = reinterpret_cast<const int4*>(w1l)[c];
                uint64_t bestd = 0;
#pragma unroll 1
                for (int r0 = wave * 8; r0 < p.V; r0 += SEL_WAVES * 8) {
                    int4 qv[2];
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        const int v = min(r0 + 4 * ii + g, p.V - 1);
                        qv[ii] = reinterpret_cast<const int4*>(p.q + (int64_t)v * RANK)[c];
                    }
                    const int vr = r0 + 4 * (c & 1) + g;           // the row this lane finishes
                    const int vc = min(vr, p.V - 1);
                    const float sr = p.scale[vc], br = p.base[row * p.V + vc];
                    int acc = 0;
#pragma unroll
                    for (int ii = 0; ii < 2; ++ii) {
                        int d = __builtin_amdgcn_sdot4(qv[ii].x, wc2.x, 0, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].y, wc2.y, d, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].z, wc2.z, d, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].w, wc2.w, d, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].x, wl2.x, d << 4, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].y, wl2.y, d, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].z, wl2.z, d, false);
                        d = __builtin_amdgcn_sdot4(qv[ii].w, wl2.w, d, false);
                        d = row16_sum_i32(d);
                        acc = (c & 1) == ii ? d : acc;
                    }
                    if (c < 2 && vr < p.V) {
                        const float l = walk_logit(br, sr, w1_code_step(a), acc);
                        if (p.out_f32) p.out_f32[row * p.V + vr] = l;
                        const uint64_t kd = argmax_key(l, (uint32_t)vr);
                        bestd = kd > bestd ? kd : bestd;
                    }
                }
                bestd = wave_max_u64(bestd);
                __syncthreads();                     // every wave has read this step's keys
                if (lane == 0) wkeys[(t & 1) * SEL_WAVES + wave] = bestd;
                __syncthreads();
                m = wkeys[(t & 1) * SEL_WAVES];
#pragma unroll
                for (int w2 = 1; w2 < SEL_WAVES; ++w2) {
                    const uint64_t o = wkeys[(t & 1) * SEL_WAVES + w2];
                    m = o > m ? o : m;
                }
                ++dense_count;
            }
        }
        // every candidate at -inf: the dense row is -inf throughout, whose first max is 0
        uint32_t token = (uint32_t)(m >> 32) <= ORDER_KEY_NEG_INF ? 0u : key_index(m);
        if (token >= (uint32_t)p.V) token = 0;
        if (tid == 0) p.tokens[b * p.T + t] = (int32_t)token;
        prev = (int)token;
        tk_stamp<TIMED>(p.stamps, st0 + 2 + 2 * t);
    }
    if constexpr (PRUNE)
        if (tid == 0 && p.dense_steps) p.dense_steps[b] = dense_count;
    // Every entry of this request has been read before the last barrier: clear them, so that the
    // workspace is all zero again.
    __syncthreads();
    int32_t* clr = p.cand + row0 * p.k;
    for (int e = tid; e < p.T * p.k; e += SEL_THREADS) clr[e] = 0;
}

static const void* pruned_fused_fn(int w1t) {
    if (w1t == DT_F32) return reinterpret_cast<const void*>(&topk_fused_kernel<0, DT_F32, false, true>);
    if (w1t == DT_BF16) return reinterpret_cast<const void*>(&topk_fused_kernel<0, DT_BF16, false, true>);
    return reinterpret_cast<const void*>(&topk_fused_kernel<0, DT_F16, false, true>);
}

template <int SAMPLE>
static const void* topk_fused_fn(int w1t, bool timed) {
    if (timed && w1t == DT_BF16) return reinterpret_cast<const void*>(&topk_fused_kernel<SAMPLE, DT_BF16, true>);
    if (w1t == DT_F32) return reinterpret_cast<const void*>(&topk_fused_kernel<SAMPLE, DT_F32, false>);
    if (w1t == DT_BF16) return reinterpret_cast<const void*>(&topk_fused_kernel<SAMPLE, DT_BF16, false>);
    return reinterpret_cast<const void*>(&topk_fused_kernel<SAMPLE, DT_F16, false>);
}

template <bool MULTI>
static const void* pruned_walk_fn(int w1t) {
    if (w1t == DT_F32) return reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_F32, MULTI, false, true>);
    if (w1t == DT_BF16) return reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_BF16, MULTI, false, true>);
    return reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_F16, MULTI, false, true>);
}

template <bool MULTI>
static const void* topk_walk_fn(int sample, int w1t, bool timed) {
    if (timed && !MULTI && w1t == DT_BF16)
        return sample ? reinterpret_cast<const void*>(&topk_walk_kernel<1, DT_BF16, false, true>)
                      : reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_BF16, false, true>);
    if (sample) {
        if (w1t == DT_F32) return reinterpret_cast<const void*>(&topk_walk_kernel<1, DT_F32, MULTI, false>);
        if (w1t == DT_BF16) return reinterpret_cast<const void*>(&topk_walk_kernel<1, DT_BF16, MULTI, false>);
        return reinterpret_cast<const void*>(&topk_walk_kernel<1, DT_F16, MULTI, false>);
    }
    if (w1t == DT_F32) return reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_F32, MULTI, false>);
    if (w1t == DT_BF16) return reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_BF16, MULTI, false>);
    return reinterpret_cast<const void*>(&topk_walk_kernel<0, DT_F16, MULTI, false>);
}

int launch_topk_walk(const TopkLaunch& a, hipStream_t stream) {
    const WalkLaunch& w = a.w;
    unsigned char* ws = static_cast<unsigned char*>(w.workspace);
    int32_t* cand = reinterpret_cast<int32_t*>(ws + WS_TOPK);

    SelectParams sp = {};
    sp.base = w.base;
    sp.cand = cand;
    sp.fill_bf16 = w.sample ? w.draft_logits : nullptr;
    sp.fill_f32 = w.sample ? nullptr : w.out_logits;
    sp.V = w.V;
    sp.k = a.k;
    const bool vec = (w.V % 4 == 0) && ((uintptr_t)w.base % 16 == 0);
    sp.stamps = reinterpret_cast<uint64_t*>(debug_knobs().stamps);
    const bool timed = sp.stamps != nullptr;
    const int w1t = w.w1_dtype == DSPARK_F32 ? DT_F32 : w.w1_dtype == DSPARK_BF16 ? DT_BF16 : DT_F16;

    TopkWalkParams kp = {};
    kp.q = w.q;
    kp.scale = w.scale;
    kp.w1 = w.w1;
    kp.base = w.base;
    kp.start = w.start;
    kp.tokens = w.tokens;
    kp.out_f32 = w.sample ? nullptr : w.out_logits;
    kp.out_bf16 = w.sample ? w.draft_logits : nullptr;
    kp.seeds = w.seeds;
    kp.positions = w.positions;
    kp.temps = w.temps;
    kp.cand = cand;
    kp.err = reinterpret_cast<uint32_t*>(ws + WS_ERR);
    kp.stamps = sp.stamps;
    kp.w2_bound = a.w2_bound;
    kp.dense_steps = a.dense_steps;
    kp.bs = w.bs;
    kp.T = w.T;
    kp.V = w.V;
    kp.k = a.k;

    // One launch pays when some rows are placed second on a CU: the walks then overlap their
    // select. With at most one row per CU every row finishes at about the same time and the walk
    // kernel alone, which loads each step's rows a step ahead, is faster.
    DeviceInfo dev;
    if (current_device_info(&dev) != DSPARK_OK) return DSPARK_ERR_NO_DEVICE;
    if (vec && a.k <= TKW_THREADS && (int64_t)w.bs * w.T > dev.cus &&
        !debug_knobs().topk_split) {
        // select and walk in one launch
        FusedParams fp = {};
        fp.s = sp;
        fp.w = kp;
        fp.never = reinterpret_cast<const uint32_t*>(ws + WS_ERR + 4);
        const DebugKnobs& dbg = debug_knobs();
        fp.spin_ticks = dbg.spin_ticks ? dbg.spin_ticks : DEFAULT_SPIN_TICKS;
        fp.wait_unset = dbg.wait_unset ? 1 : 0;
        fp.first_slots = dev.cus > w.bs ? dev.cus : w.bs;
        const void* fn = a.w2_bound ? pruned_fused_fn(w1t)
                       : w.sample   ? topk_fused_fn<1>(w1t, timed)
                                    : topk_fused_fn<0>(w1t, timed);
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, SEL_LDS_BYTES) !=
            hipSuccess) {
            (void)hipGetLastError();
        }
        void* fargs[] = {&fp};
        const hipError_t fe = launch_walk_kernel(fn, dim3((unsigned)(w.bs * w.T)),
                                                 dim3(SEL_THREADS), fargs,
                                                 (size_t)SEL_LDS_BYTES, stream);
        if (fe != hipSuccess) {
            (void)hipGetLastError();
            return DSPARK_ERR_LAUNCH;
        }
        return DSPARK_OK;
    }

    void* sargs[] = {&sp};
    const void* sel = vec ? (timed ? reinterpret_cast<const void*>(&topk_select_kernel<true, true>)
                                   : reinterpret_cast<const void*>(&topk_select_kernel<true, false>))
                          : reinterpret_cast<const void*>(&topk_select_kernel<false, false>);
    if (hipFuncSetAttribute(sel, hipFuncAttributeMaxDynamicSharedMemorySize, SEL_LDS_BYTES) !=
        hipSuccess) {
        (void)hipGetLastError();
    }
    hipError_t e = launch_walk_kernel(sel, dim3((unsigned)(w.bs * w.T)), dim3(SEL_THREADS), sargs,
                                      (size_t)SEL_LDS_BYTES, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return DSPARK_ERR_LAUNCH;
    }

    void* kargs[] = {&kp};
    const void* fn = a.w2_bound ? (a.k > TKW_THREADS ? pruned_walk_fn<true>(w1t)
                                                     : pruned_walk_fn<false>(w1t))
                   : a.k > TKW_THREADS ? topk_walk_fn<true>(w.sample, w1t, timed)
                                       : topk_walk_fn<false>(w.sample, w1t, timed);
    e = launch_walk_kernel(fn, dim3((unsigned)w.bs), dim3(TKW_THREADS),
                           kargs, 0, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return DSPARK_ERR_LAUNCH;
    }
    return DSPARK_OK;
}

// ---- load-time bound of the lossless pruned walk -----------------------------------------------
// B = max_v fl(s[v] * sum_k |q[v,k]|): one wave per row at a time (lane l sums the magnitudes of
// codes 4l .. 4l+3), the largest product folded into *bound with an unsigned atomic max of its
// bits (every product is >= 0, where IEEE order is unsigned order). *bound starts at zero.
__global__ __launch_bounds__(256) void w2_bound_zero_kernel(float* bound) { *bound = 0.0f; }

__global__ __launch_bounds__(256) void w2_bound_kernel(const int8_t* q, const float* s, int V,
                                                       float* bound) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = (int)(blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
    const int nwaves = (int)(gridDim.x * (blockDim.x / WAVE));
    float best = 0.0f;
    for (int v = wave; v < V; v += nwaves) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(q + (int64_t)v * RANK)[lane];
        int l1 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = (int)(int8_t)(w >> (8 * i));
            l1 += c < 0 ? -c : c;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l1 += __shfl_xor(l1, o, WAVE);
        best = fmaxf(best, s[v] * (float)l1);
    }
    if (lane == 0 && best > 0.0f)
        __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(bound), __float_as_uint(best),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int launch_w2_bound(const int8_t* q, const float* s, int64_t V, float* bound, hipStream_t stream) {
    w2_bound_zero_kernel<<<1, 1, 0, stream>>>(bound);
    const int64_t blocks = (V + 3) / 4 < 2048 ? (V + 3) / 4 : 2048;
    w2_bound_kernel<<<(unsigned)blocks, 256, 0, stream>>>(q, s, (int)V, bound);
    if (hipGetLastError() != hipSuccess) return DSPARK_ERR_LAUNCH;
    return DSPARK_OK;
}

}  // namespace dspark
