// K1: the dense Markov draft walk as one persistent kernel on gfx950.
//
// What it computes (vLLM PR #62958, int8 DSpark Markov walk, Overview and Details; vLLM PR
// #64476, Claims): for every request b and step t,
//     l[v]  = base[b,t,v] + s[v] * s1 * sum_k q[v,k] * q1[k],   q1/s1 = int8 codes of W1[prev_b]
//     greedy: token = argmax_v l[v];
//     sample: lb = bf16(l), token = argmax_v (lb[v] / temp_b + Gumbel(Philox(seed_b, P, v)))
// with torch.argmax order, and token becomes prev_b for step t+1.
//
// How it runs. One workgroup of 4 waves (one wave per SIMD) per compute unit owns a contiguous
// slice of W2 rows for the whole call; each lane owns whole rows (lane-per-row), so a row's
// 256-term dot product needs no cross-lane reduction:
//   * the first 2 x 256 rows of the slice live in VGPRs (2 rows x 64 dwords per lane),
//   * the next up to 2 x 256 rows live in LDS (16-byte chunks XOR-swizzled by row, so the
//     lanes of a wave reading one chunk index hit different banks),
//   * rows beyond are re-read from memory at every step (only when V exceeds what the grid
//     holds on chip).
// Per step: the gathered W1 rows are quantised to int8 codes with one absmax scale per row and
// placed in LDS, where every lane reads them as broadcasts; v_dot4_i32_i8 accumulates exact
// int32 sums; scale, base logit and sampler finish each row; wave-wide and workgroup-wide
// maxima of 64-bit argmax keys give the slice's best per request.
//
// Grid-wide combine, without read-modify-write contention: each workgroup stores its best key
// per request into a slot of its own (whole 128-byte lines); the workgroup that reduces
// request b waits until all slots of b are filled, takes their maximum, writes the token, and
// publishes the winning key in one result word; every workgroup waits for the result words it
// needs. The reducer clears the slots it read at once, and clears its result word of step t-1
// once every slot of step t is filled (each workgroup reads the results of step t-1 before it
// fills its slot of step t); the last step publishes no result. So the workspace is all-zero
// again when the kernel exits, without a final barrier. Every wait has a spin limit, after
// which DSPARK_ERR_TIMEOUT is recorded and the kernel runs to its end.
#include "device_common.hpp"
#include "internal.hpp"

namespace dspark {

constexpr int WALK_THREADS = 256;
constexpr int WALK_WAVES = WALK_THREADS / WAVE;      // 4: one per SIMD
constexpr int REG_J = 2;                             // row sets held in VGPRs
constexpr int LDS_J_MAX = 2;                         // row sets held in LDS
constexpr int PF_J = REG_J + LDS_J_MAX;              // row sets whose base logits are prefetched
constexpr int PF_DEPTH = 4;                          // requests of base logits in flight
constexpr int GATHER_CHUNK = 8;                      // W1 rows in flight per wave
constexpr int ROW_CHUNKS = RANK / 16;                // 16-byte chunks per int8 row
constexpr int LDS_ROWSET_BYTES = WALK_THREADS * RANK;  // one row per lane: 64 KiB
constexpr int LDS_FIXED_BYTES = MAX_BS * RANK        // int8 codes of the gathered W1 rows
                                + MAX_BS * 4         // their scales
                                + WALK_WAVES * MAX_BS * 8  // per-wave best keys
                                + MAX_BS * 4;        // tokens of the current step
constexpr int LDS_MIN_BYTES = 96 * 1024;             // > half the CU's LDS: one workgroup per CU
constexpr uint32_t DEFAULT_SPIN_LIMIT = 1u << 22;

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
    uint64_t* result;     // [16][64] winning keys
    uint64_t* slots;      // [T][num workgroups][stride] per-workgroup keys
    uint32_t* err;
    const uint32_t* never;  // a workspace word nothing writes (test hook)
    int bs, T, V;
    int rows_per_wg;
    int nj;        // row sets per lane (ceil(rows_per_wg / 256))
    int lds_j;     // of which LDS-resident (after the REG_J register sets)
    int stride;    // keys per workgroup slot
    uint32_t spin_limit;
    int wait_unset;
    uint64_t* stamps;  // instrumented builds: [num workgroups][STAMPS_PER_WG] clock stamps
};

// Instrumented builds record the constant-rate device clock (s_memrealtime, 100 MHz) at these
// points, per workgroup: kernel start, fill done, then per step: W1 codes ready, slice argmax
// done, own slot stored, reductions done, result words seen.
constexpr int STAMP_STEP0 = 2;
constexpr int STAMPS_PER_STEP = 5;
constexpr int STAMPS_PER_WG = STAMP_STEP0 + MAX_STEPS * STAMPS_PER_STEP;

template <int TIMED>
__device__ __forceinline__ void stamp(const WalkParams& p, int slot) {
    if constexpr (TIMED) {
        if (threadIdx.x == 0)
            p.stamps[(size_t)blockIdx.x * STAMPS_PER_WG + slot] = __builtin_amdgcn_s_memrealtime();
    }
}

// 16 int8 products of one 16-byte chunk into four independent int32 partial sums: v_dot4 has
// ~20 cycles of latency against ~4-5 cycles of issue, so one wave per SIMD needs >= 5
// independent accumulation chains to keep it busy.
__device__ __forceinline__ void dot16x4(const int4 a, const int4 b, int4& acc) {
    acc.x = __builtin_amdgcn_sdot4(a.x, b.x, acc.x, false);
    acc.y = __builtin_amdgcn_sdot4(a.y, b.y, acc.y, false);
    acc.z = __builtin_amdgcn_sdot4(a.z, b.z, acc.z, false);
    acc.w = __builtin_amdgcn_sdot4(a.w, b.w, acc.w, false);
}
__device__ __forceinline__ int hsum(const int4 a) { return (a.x + a.y) + (a.z + a.w); }

__device__ __forceinline__ uint32_t pack_codes(const float4 w, float inv) {
    const float v[4] = {w.x, w.y, w.z, w.w};
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float r = rintf(v[i] * inv);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        packed |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * i);
    }
    return packed;
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

template <int SAMPLE, int W1T, int TIMED = 0>
__global__ __launch_bounds__(WALK_THREADS, 1) void dense_walk_kernel(const WalkParams p) {
    stamp<TIMED>(p, 0);
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = tid / WAVE;
    const int nwg = gridDim.x;
    const int wg = blockIdx.x;
    const int row0 = wg * p.rows_per_wg;
    const int nrows = min(p.rows_per_wg, p.V - row0);

    unsigned char* lds_rows = smem;
    uint32_t* w1q = reinterpret_cast<uint32_t*>(smem + p.lds_j * LDS_ROWSET_BYTES);
    float* s1 = reinterpret_cast<float*>(w1q + MAX_BS * (RANK / 4));
    uint64_t* wkeys = reinterpret_cast<uint64_t*>(s1 + MAX_BS);
    int32_t* tok = reinterpret_cast<int32_t*>(wkeys + WALK_WAVES * MAX_BS);

    // ---- fill: this workgroup's W2 rows into VGPRs and LDS, their scales into VGPRs --------
    int4 qr[REG_J][ROW_CHUNKS];
#pragma unroll
    for (int j = 0; j < REG_J; ++j) {
        const int r = j * WALK_THREADS + tid;
        if (r < nrows) {
            const int4* src = reinterpret_cast<const int4*>(p.q + (int64_t)(row0 + r) * RANK);
#pragma unroll
            for (int c = 0; c < ROW_CHUNKS; ++c) qr[j][c] = src[c];
        } else {
#pragma unroll
            for (int c = 0; c < ROW_CHUNKS; ++c) qr[j][c] = make_int4(0, 0, 0, 0);
        }
    }
    for (int j = 0; j < p.lds_j; ++j) {
        const int r = (REG_J + j) * WALK_THREADS + tid;
        if (r < nrows) {
            const int4* src = reinterpret_cast<const int4*>(p.q + (int64_t)(row0 + r) * RANK);
            int4* dst = reinterpret_cast<int4*>(lds_rows + (size_t)(j * WALK_THREADS + tid) * RANK);
#pragma unroll
            for (int c = 0; c < ROW_CHUNKS; ++c) dst[c ^ (tid & 15)] = src[c];
        }
    }
    float sc[PF_J];  // scales of the register and LDS row sets
#pragma unroll
    for (int j = 0; j < PF_J; ++j) {
        const int r = j * WALK_THREADS + tid;
        sc[j] = r < nrows ? p.scale[row0 + r] : 0.0f;
    }
    if (tid < p.bs) {
        int s = p.start[tid];
        if (s < 0 || s >= p.V) {  // precondition violated: keep every gather in bounds
            if (wg == 0) flag_error(p.err, DSPARK_ERR_INVALID_ARG);
            s = 0;
        }
        tok[tid] = s;
    }

    // base logits of the first PF_J row sets, PF_DEPTH requests ahead of their use
    float pf[PF_DEPTH][PF_J];
    auto load_base = [&](float (&dst)[PF_J], int b, int t) {
        const float* br = p.base + ((int64_t)b * p.T + t) * p.V + row0;
#pragma unroll
        for (int j = 0; j < PF_J; ++j) {
            const int r = j * WALK_THREADS + tid;
            dst[j] = r < nrows ? br[r] : 0.0f;
        }
    };
#pragma unroll
    for (int u = 0; u < PF_DEPTH; ++u)
        if (u < p.bs) load_base(pf[u], u, 0);
    __syncthreads();
    stamp<TIMED>(p, 1);

    for (int t = 0; t < p.T; ++t) {
        // ---- gather W1[prev_b] (GATHER_CHUNK rows in flight per wave), int8 codes + scale ----
        for (int b0 = wave; b0 < p.bs; b0 += WALK_WAVES * GATHER_CHUNK) {
            float4 wv[GATHER_CHUNK];
#pragma unroll
            for (int u = 0; u < GATHER_CHUNK; ++u) {
                const int b = b0 + u * WALK_WAVES;
                if (b < p.bs)
                    wv[u] = load4_as_f32<W1T>(p.w1, (int64_t)tok[b] * RANK + lane * 4);
            }
#pragma unroll
            for (int u = 0; u < GATHER_CHUNK; ++u) {
                const int b = b0 + u * WALK_WAVES;
                if (b < p.bs) {
                    const float4 w = wv[u];
                    float a = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
                    a = wave_max_nonneg_f32(a);
                    const float inv = a > 0.0f ? 127.0f / a : 0.0f;
                    w1q[b * (RANK / 4) + lane] = pack_codes(w, inv);
                    if (lane == 0) s1[b] = a * (1.0f / 127.0f);
                }
            }
        }
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 0);

        // ---- per request: int8 GEMV over the slice, logits, sampler, slice-local argmax -----
        for (int b0 = 0; b0 < p.bs; b0 += PF_DEPTH) {
#pragma unroll
            for (int u = 0; u < PF_DEPTH; ++u) {
                const int b = b0 + u;
                if (b < p.bs) {
                    float cur[PF_J];
#pragma unroll
                    for (int j = 0; j < PF_J; ++j) cur[j] = pf[u][j];
                    if (b + PF_DEPTH < p.bs) load_base(pf[u], b + PF_DEPTH, t);

                    const float sb = s1[b];
                    const int64_t orow = ((int64_t)b * p.T + t) * p.V;
                    uint64_t seed = 0, P = 0;
                    float temp = 1.0f;
                    if constexpr (SAMPLE) {
                        seed = p.seeds[b];
                        P = (uint64_t)(p.positions ? p.positions[b] : 0) + (uint64_t)t;
                        temp = p.temps[b];
                    }
                    // logit of row v -> output store and argmax key
                    auto finish = [&](int v, float base_v, float scale_v, int acc) -> uint64_t {
                        const float l = base_v + (scale_v * sb) * (float)acc;
                        if constexpr (!SAMPLE) {
                            if (p.out_logits) p.out_logits[orow + v] = l;
                            return argmax_key(l, (uint32_t)v);
                        } else {
                            const uint32_t h = bf16_bits(l);
                            p.draft_logits[orow + v] = (uint16_t)h;
                            float x = bf16_value(h);
                            if (temp != 1.0f) x = x / temp;
                            const float g = gumbel_from_word(noise_word(seed, P, (uint32_t)v));
                            return argmax_key(x + g, (uint32_t)v);
                        }
                    };

                    const int4* wq = reinterpret_cast<const int4*>(w1q + b * (RANK / 4));
                    int4 acc[REG_J];
#pragma unroll
                    for (int j = 0; j < REG_J; ++j) acc[j] = make_int4(0, 0, 0, 0);
#pragma unroll
                    for (int c = 0; c < ROW_CHUNKS; ++c) {
                        const int4 w = wq[c];
#pragma unroll
                        for (int j = 0; j < REG_J; ++j) dot16x4(qr[j][c], w, acc[j]);
                    }
                    uint64_t best = 0;
#pragma unroll
                    for (int j = 0; j < REG_J; ++j) {
                        const int r = j * WALK_THREADS + tid;
                        if (r < nrows) {
                            const uint64_t key = finish(row0 + r, cur[j], sc[j], hsum(acc[j]));
                            best = key > best ? key : best;
                        }
                    }
                    // row sets beyond the registers: LDS-resident, then streamed from memory
                    for (int j = REG_J; j < p.nj; ++j) {
                        const int r = j * WALK_THREADS + tid;
                        if (r < nrows) {
                            int4 a4 = make_int4(0, 0, 0, 0), b4 = make_int4(0, 0, 0, 0);
                            if (j < REG_J + p.lds_j) {
                                const int4* src = reinterpret_cast<const int4*>(
                                    lds_rows + (size_t)((j - REG_J) * WALK_THREADS + tid) * RANK);
#pragma unroll
                                for (int c = 0; c < ROW_CHUNKS; c += 2) {
                                    dot16x4(src[c ^ (tid & 15)], wq[c], a4);
                                    dot16x4(src[(c + 1) ^ (tid & 15)], wq[c + 1], b4);
                                }
                            } else {
                                const int4* src = reinterpret_cast<const int4*>(
                                    p.q + (int64_t)(row0 + r) * RANK);
#pragma unroll 4
                                for (int c = 0; c < ROW_CHUNKS; c += 2) {
                                    dot16x4(src[c], wq[c], a4);
                                    dot16x4(src[c + 1], wq[c + 1], b4);
                                }
                            }
                            const int a = hsum(a4) + hsum(b4);
                            float bv = 0.0f, sv = 0.0f;
                            if (j < PF_J) {
#pragma unroll
                                for (int jj = REG_J; jj < PF_J; ++jj)
                                    if (jj == j) {
                                        bv = cur[jj];
                                        sv = sc[jj];
                                    }
                            } else {
                                bv = p.base[orow + row0 + r];
                                sv = p.scale[row0 + r];
                            }
                            const uint64_t key = finish(row0 + r, bv, sv, a);
                            best = key > best ? key : best;
                        }
                    }
                    best = wave_max_u64(best);
                    if (lane == 0) wkeys[wave * MAX_BS + b] = best;
                }
            }
        }
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 1);

        // the next step's first base logits load while the combine waits
        if (t + 1 < p.T) {
#pragma unroll
            for (int u = 0; u < PF_DEPTH; ++u)
                if (u < p.bs) load_base(pf[u], u, t + 1);
        }

        // ---- grid-wide combine: own slot -> reducer per request -> result words -------------
        if (wave == 0) {
            uint64_t* step_slots = p.slots + (size_t)t * nwg * p.stride;
            if (lane < p.bs) {
                uint64_t k = wkeys[lane];
#pragma unroll
                for (int w = 1; w < WALK_WAVES; ++w) {
                    const uint64_t o = wkeys[w * MAX_BS + lane];
                    k = o > k ? o : k;
                }
                st_dev(step_slots + (size_t)wg * p.stride + lane, k);
            }
            stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 2);
            for (int b = wg; b < p.bs; b += nwg) {
                uint64_t* col = step_slots + b;
                uint64_t best = 0;
                uint32_t spins = 0;
                while (true) {
                    // all slot loads of a round are in flight together (nwg <= 4 x 64)
                    uint64_t v[MAX_WORKGROUPS / WAVE];
#pragma unroll
                    for (int k = 0; k < MAX_WORKGROUPS / WAVE; ++k) {
                        const int w = lane + k * WAVE;
                        v[k] = w < nwg ? ld_dev(col + (size_t)w * p.stride) : 0;
                    }
                    bool all = true;
                    best = 0;
#pragma unroll
                    for (int k = 0; k < MAX_WORKGROUPS / WAVE; ++k) {
                        all = all && (v[k] != 0 || lane + k * WAVE >= nwg);
                        best = v[k] > best ? v[k] : best;
                    }
                    if (p.wait_unset)
                        all = all && __hip_atomic_load(p.never, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT) != 0;
                    if (__all(all)) break;
                    if (++spins > p.spin_limit) {
                        if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                best = wave_max_u64(best);
                if (best == 0) best = 1;  // only after a timeout: keep the result word non-zero
                uint32_t token = key_index(best);
                if (token >= (uint32_t)p.V) token = 0;
                if (lane == 0) {
                    p.tokens[b * p.T + t] = (int32_t)token;
                    if (t + 1 < p.T) st_dev(p.result + t * MAX_BS + b, best);
                    if (t > 0) st_dev(p.result + (t - 1) * MAX_BS + b, 0);
                }
#pragma unroll
                for (int k = 0; k < MAX_WORKGROUPS / WAVE; ++k) {
                    const int w = lane + k * WAVE;
                    if (w < nwg) st_dev(col + (size_t)w * p.stride, 0);
                }
            }
            stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 3);
            if (t + 1 < p.T) {
                uint64_t k = 0;
                uint32_t spins = 0;
                while (true) {
                    bool ok = true;
                    if (lane < p.bs) {
                        k = ld_dev(p.result + t * MAX_BS + lane);
                        ok = k != 0;
                    }
                    if (__all(ok)) break;
                    if (++spins > p.spin_limit) {
                        if (lane == 0) flag_error(p.err, DSPARK_ERR_TIMEOUT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (lane < p.bs) {
                    uint32_t token = key_index(k);
                    if (token >= (uint32_t)p.V) token = 0;
                    tok[lane] = (int32_t)token;
                }
            }
            stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 4);
        }
        __syncthreads();
    }
}

// -------------------------------------------------------------------------------------------
// Host side: the partition of W2 over the grid, and the launch.
// -------------------------------------------------------------------------------------------
int plan_walk(const DeviceInfo& dev, int64_t bs, int64_t T, int64_t V, dspark_walk_plan* plan) {
    (void)bs;
    (void)T;
    int cap = dev.cus < MAX_WORKGROUPS ? dev.cus : MAX_WORKGROUPS;
    const int dbg = debug_knobs().max_workgroups;
    if (dbg > 0 && dbg < cap) cap = dbg;
    if (cap < 1) return DSPARK_ERR_NO_DEVICE;
    int64_t rpw = (V + cap - 1) / cap;
    if (rpw < WALK_THREADS) rpw = V < WALK_THREADS ? V : WALK_THREADS;
    rpw = (rpw + 3) / 4 * 4;
    const int64_t nwg = (V + rpw - 1) / rpw;
    const int64_t nj = (rpw + WALK_THREADS - 1) / WALK_THREADS;
    int64_t lds_j = nj - REG_J;
    if (lds_j < 0) lds_j = 0;
    if (lds_j > LDS_J_MAX) lds_j = LDS_J_MAX;
    const int64_t reg_rows = rpw < REG_J * WALK_THREADS ? rpw : REG_J * WALK_THREADS;
    int64_t lds_rows = rpw - reg_rows;
    if (lds_rows > lds_j * WALK_THREADS) lds_rows = lds_j * WALK_THREADS;
    const int64_t str_rows = rpw - reg_rows - lds_rows;
    int64_t lds_bytes = lds_j * LDS_ROWSET_BYTES + LDS_FIXED_BYTES;
    if (lds_bytes < LDS_MIN_BYTES) lds_bytes = LDS_MIN_BYTES;
    if ((size_t)lds_bytes > dev.max_lds) return DSPARK_ERR_UNSUPPORTED;

    // whole-grid byte counts: rows are owned contiguously, the last workgroup may own fewer
    int64_t res = 0, str = 0;
    for (int64_t w = 0; w < nwg; ++w) {
        const int64_t n = (w + 1) * rpw <= V ? rpw : V - w * rpw;
        const int64_t on_chip = n < reg_rows + lds_rows ? n : reg_rows + lds_rows;
        res += on_chip;
        str += n - on_chip;
    }
    plan->device_cus = dev.cus;
    plan->num_workgroups = (int32_t)nwg;
    plan->rows_per_workgroup = (int32_t)rpw;
    plan->rows_in_registers = (int32_t)reg_rows;
    plan->rows_in_lds = (int32_t)lds_rows;
    plan->rows_streamed = (int32_t)str_rows;
    plan->resident_bytes = res * RANK;
    plan->streamed_bytes = str * RANK;
    plan->lds_bytes = (int32_t)lds_bytes;
    return DSPARK_OK;
}

template <int SAMPLE>
static const void* pick_kernel(int w1_dtype, bool timed) {
    if (timed)  // instrumented build: bf16 W1 only
        return reinterpret_cast<const void*>(&dense_walk_kernel<SAMPLE, DT_BF16, 1>);
    switch (w1_dtype) {
        case DSPARK_F32: return reinterpret_cast<const void*>(&dense_walk_kernel<SAMPLE, DT_F32>);
        case DSPARK_BF16: return reinterpret_cast<const void*>(&dense_walk_kernel<SAMPLE, DT_BF16>);
        default: return reinterpret_cast<const void*>(&dense_walk_kernel<SAMPLE, DT_F16>);
    }
}

// The kernel's waits need all its workgroups resident at once. The grid never exceeds the
// compute units, and each workgroup asks for more than half of a CU's LDS, so each CU holds at
// most one; with the device otherwise idle they are all resident. If they are not (other work
// holds CUs), the waits run into their spin limit and the call reports DSPARK_ERR_TIMEOUT
// instead of hanging. A cooperative launch would guarantee residency but costs ~20 us per
// launch on this stack, an order of magnitude above a plain launch.
int launch_dense_walk(const WalkLaunch& a, const dspark_walk_plan& plan, hipStream_t stream) {
    WalkParams p;
    p.q = a.q;
    p.scale = a.scale;
    p.w1 = a.w1;
    p.base = a.base;
    p.start = a.start;
    p.tokens = a.tokens;
    p.out_logits = a.out_logits;
    p.draft_logits = a.draft_logits;
    p.seeds = a.seeds;
    p.positions = a.positions;
    p.temps = a.temps;
    char* ws = static_cast<char*>(a.workspace);
    p.result = reinterpret_cast<uint64_t*>(ws + WS_RESULT);
    p.slots = reinterpret_cast<uint64_t*>(ws + WS_SLOTS);
    p.err = reinterpret_cast<uint32_t*>(ws + WS_ERR);
    p.never = reinterpret_cast<const uint32_t*>(ws + WS_ERR + 4);
    p.bs = a.bs;
    p.T = a.T;
    p.V = a.V;
    p.rows_per_wg = plan.rows_per_workgroup;
    p.nj = (plan.rows_per_workgroup + WALK_THREADS - 1) / WALK_THREADS;
    p.lds_j = (plan.rows_in_lds + WALK_THREADS - 1) / WALK_THREADS;
    p.stride = slot_stride(a.bs);
    const DebugKnobs& dbg = debug_knobs();
    p.spin_limit = dbg.spin_limit ? dbg.spin_limit : DEFAULT_SPIN_LIMIT;
    p.wait_unset = dbg.wait_unset ? 1 : 0;
    p.stamps = reinterpret_cast<uint64_t*>(dbg.stamps);
    const bool timed = p.stamps != nullptr && a.w1_dtype == DSPARK_BF16;

    const void* fn = a.sample ? pick_kernel<1>(a.w1_dtype, timed) : pick_kernel<0>(a.w1_dtype, timed);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, plan.lds_bytes) !=
        hipSuccess) {
        (void)hipGetLastError();
    }
    void* args[] = {&p};
    const hipError_t e = hipLaunchKernel(fn, dim3(plan.num_workgroups), dim3(WALK_THREADS), args,
                                         (size_t)plan.lds_bytes, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return DSPARK_ERR_LAUNCH;
    }
    return DSPARK_OK;
}

}  // namespace dspark
