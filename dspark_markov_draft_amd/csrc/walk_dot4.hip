// Dense walk, lane-per-row v_dot4 kernel (used for a single request, where every row of W2 is
// multiplied by one W1 row: a GEMV, which a matrix core would run at 1/16 use).
//
// What it computes (vLLM PR #62958, int8 DSpark Markov walk, Overview and Details; vLLM PR
// #64476, Claims): for every request b and step t,
//     l[v]  = base[b,t,v] + s[v] * s1 * sum_k q[v,k] * C[k],   C/s1 = the codes of W1[prev_b]
//     greedy: token = argmax_v l[v];
//     sample: lb = bf16(l), token = argmax_v (lb[v] / temp_b + Gumbel(Philox(seed_b, P, v)))
// with torch.argmax order, and token becomes prev_b for step t+1.
//
// One workgroup of 4 waves (one wave per SIMD) per compute unit owns a contiguous slice of W2
// rows for the whole call; each lane owns whole rows, so a row's 256-term dot product needs no
// cross-lane reduction:
//   * the first 2 x 256 rows of the slice live in VGPRs (2 rows x 64 dwords per lane),
//   * the next up to 2 x 256 rows live in LDS (16-byte chunks XOR-swizzled by row, so the
//     lanes of a wave reading one chunk index hit different banks),
//   * rows beyond are re-read from memory at every step.
// The W1 codes (two int8 digits per element) are LDS broadcasts; v_dot4_i32_i8 accumulates
// exact int32 sums in four independent chains per row and digit (its latency is ~20 cycles, its
// issue ~4), joined as 16 * high + low; scale, base logit and
// sampler finish each row; wave-wide and workgroup-wide maxima of 64-bit argmax keys give the
// slice's best, and combine_step() combines the slices across the grid.
#include "walk_common.hpp"

namespace dspark {

constexpr int REG_J = DOT4_REG_SETS;     // row sets held in registers
constexpr int LDS_J_MAX = 2;             // row sets held in LDS
constexpr int PF_J = REG_J + LDS_J_MAX;  // row sets whose base logits are prefetched
constexpr int PF_DEPTH = 2;              // requests of base logits in flight
constexpr int ROW_CHUNKS = RANK / 16;    // 16-byte chunks per int8 row


template <int SAMPLE, int W1T, int TIMED>
__global__ __launch_bounds__(WALK_THREADS, 1) void dense_walk_dot4_kernel(const WalkParams p) {
    stamp<TIMED>(p, 0);
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = tid / WAVE;
    const int row0 = blockIdx.x * p.rows_per_wg;
    const int nrows = min(p.rows_per_wg, p.V - row0);
    const int nj = p.total_units;
    const int lds_j = p.lds_units;

    unsigned char* lds_rows = smem;
    uint32_t* w1q = reinterpret_cast<uint32_t*>(smem + (size_t)lds_j * WALK_THREADS * RANK);
    uint32_t* w1l = w1q + W1Q_BYTES / 4;
    float* s1 = reinterpret_cast<float*>(w1l + W1L_BYTES / 4);
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
    for (int j = 0; j < lds_j; ++j) {
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
    load_start_tokens(p, tok);

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
        // wave 0 runs the combine, whose polls would wait behind any load it has in flight
        // (vector memory returns in issue order): its share of this step's first base logits is
        // issued here, behind the W1 row loads, instead of before the previous combine
        gather_w1_codes<W1T, LOW_BYTES>(p, tok, w1q, w1l, s1, wave, lane, [&] {
            if (wave == 0 && t > 0) {
#pragma unroll
                for (int u = 0; u < PF_DEPTH; ++u)
                    if (u < p.bs) load_base(pf[u], u, t);
            }
        });
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 0);

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
                    float rtemp = 1.0f;
                    if constexpr (SAMPLE) {
                        seed = p.seeds[b];
                        P = (uint64_t)(p.positions ? p.positions[b] : 0) + (uint64_t)t;
                        rtemp = inv_temperature(p.temps[b]);
                    }
                    // logit of row v -> output store, offered to this lane's running argmax (its
                    // rows come in increasing index order), or (inverse CDF) to its running
                    // softmax pair
                    RunningArgmax run;
                    RunningSoftmax soft;
                    const float kz = rtemp * LOG2E_F;
                    auto finish = [&](int v, float base_v, float scale_v, int acc) {
                        const float l = walk_logit(base_v, scale_v, sb, acc);
                        if constexpr (!SAMPLE) {
                            if (p.out_logits) p.out_logits[orow + v] = l;
                            run.offer(l, (uint32_t)v, true);
                        } else if constexpr (SAMPLE == 1) {
                            const uint32_t h = bf16_bits(l);
                            p.draft_logits[orow + v] = (uint16_t)h;
                            const float x = bf16_value(h) * rtemp;
                            const float g = gumbel_from_word(noise_word(seed, P, (uint32_t)v));
                            run.offer(x + g, (uint32_t)v, true);
                        } else {
                            const uint32_t h = bf16_bits(l);
                            p.draft_logits[orow + v] = (uint16_t)h;
                            soft.offer(bf16_value(h) * kz, true);
                        }
                    };

                    const int4* wq = reinterpret_cast<const int4*>(w1q + b * (RANK / 4));
                    const int4* wl = reinterpret_cast<const int4*>(w1l + b * (RANK / 4));
                    const int sw = b & 15;  // chunk c of this request's digits is at c ^ sw
                    // each row chunk (moved out of its AGPRs once) into a high and a low chain
                    int4 acc[REG_J], acl[REG_J];
#pragma unroll
                    for (int j = 0; j < REG_J; ++j) {
                        acc[j] = make_int4(0, 0, 0, 0);
                        acl[j] = make_int4(0, 0, 0, 0);
                    }
#pragma unroll
                    for (int c = 0; c < ROW_CHUNKS; ++c) {
                        // a compiler-only barrier every 4 chunks: the W1 chunks are read from
                        // LDS 4 at a time instead of all 16 up front, which keeps the register
                        // rows in VGPRs
                        if (c % 4 == 0) asm volatile("" ::: "memory");
                        const int4 w = wq[c ^ sw];
                        const int4 wlo = wl[c ^ sw];
#pragma unroll
                        for (int j = 0; j < REG_J; ++j) {
                            dot16x4(qr[j][c], w, acc[j]);
                            dot16x4(qr[j][c], wlo, acl[j]);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < REG_J; ++j) {
                        const int r = j * WALK_THREADS + tid;
                        if (r < nrows) finish(row0 + r, cur[j], sc[j], join_digits(hsum(acc[j]), hsum(acl[j])));
                    }
                    // row sets beyond the registers: LDS-resident, then streamed from memory
                    for (int j = REG_J; j < nj; ++j) {
                        const int r = j * WALK_THREADS + tid;
                        if (r < nrows) {
                            // each row chunk read once, into a high and a low chain
                            int4 a4 = make_int4(0, 0, 0, 0), b4 = make_int4(0, 0, 0, 0);
                            if (j < REG_J + lds_j) {
                                const int4* src = reinterpret_cast<const int4*>(
                                    lds_rows + (size_t)((j - REG_J) * WALK_THREADS + tid) * RANK);
#pragma unroll
                                for (int c = 0; c < ROW_CHUNKS; ++c) {
                                    const int4 x = src[c ^ (tid & 15)];
                                    dot16x4(x, wq[c ^ sw], a4);
                                    dot16x4(x, wl[c ^ sw], b4);
                                }
                            } else {
                                const int4* src = reinterpret_cast<const int4*>(
                                    p.q + (int64_t)(row0 + r) * RANK);
#pragma unroll 4
                                for (int c = 0; c < ROW_CHUNKS; ++c) {
                                    const int4 x = src[c];
                                    dot16x4(x, wq[c ^ sw], a4);
                                    dot16x4(x, wl[c ^ sw], b4);
                                }
                            }
                            const int a = join_digits(hsum(a4), hsum(b4));
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
                            finish(row0 + r, bv, sv, a);
                        }
                    }
                    if constexpr (SAMPLE == 2) {
                        wave_softmax(soft.m, soft.s);
                        if (lane == 0) wkeys[wave * MAX_BS + b] = pack_softmax(soft.m, soft.s);
                    } else {
                        const uint64_t best = wave_max_u64(run.key());
                        if (lane == 0) wkeys[wave * MAX_BS + b] = best;
                    }
                }
            }
        }
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 1);

        // the next step's first base logits load while the combine waits (wave 0: see above)
        if (t + 1 < p.T && wave != 0) {
#pragma unroll
            for (int u = 0; u < PF_DEPTH; ++u)
                if (u < p.bs) load_base(pf[u], u, t + 1);
        }
        if (wave == 0) {
            uint64_t k = 0;
            if constexpr (SAMPLE == 2) {
                if (lane < p.bs) {
                    RunningSoftmax a;
#pragma unroll
                    for (int w = 0; w < WALK_WAVES; ++w) {
                        const uint64_t o = wkeys[w * MAX_BS + lane];
                        a.merge(packed_m(o), packed_s(o));
                    }
                    k = pack_softmax(a.m, a.s);
                }
                combine_icdf_step<TIMED>(p, t, k, tok, lane);
            } else {
                if (lane < p.bs) {
                    // the four waves' keys: all read before any compare (one LDS round trip)
                    uint64_t o[WALK_WAVES];
#pragma unroll
                    for (int w = 0; w < WALK_WAVES; ++w) o[w] = wkeys[w * MAX_BS + lane];
                    asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
                    const uint64_t k01 = o[1] > o[0] ? o[1] : o[0];
                    const uint64_t k23 = o[3] > o[2] ? o[3] : o[2];
                    k = k23 > k01 ? k23 : k01;
                }
                combine_step<TIMED>(p, t, k, tok, lane);
            }
        }
        __syncthreads();
    }
}

const void* dot4_walk_kernel(int sample, int w1t, bool timed) {
#define DSPARK_DOT4(S, W, TI) reinterpret_cast<const void*>(&dense_walk_dot4_kernel<S, W, TI>)
    if (sample == 2) {
        switch (w1t) {
            case DT_F32: return DSPARK_DOT4(2, DT_F32, 0);
            case DT_BF16: return DSPARK_DOT4(2, DT_BF16, 0);
            default: return DSPARK_DOT4(2, DT_F16, 0);
        }
    }
    if (timed) return sample ? DSPARK_DOT4(1, DT_BF16, 1) : DSPARK_DOT4(0, DT_BF16, 1);
    if (sample) {
        switch (w1t) {
            case DT_F32: return DSPARK_DOT4(1, DT_F32, 0);
            case DT_BF16: return DSPARK_DOT4(1, DT_BF16, 0);
            default: return DSPARK_DOT4(1, DT_F16, 0);
        }
    }
    switch (w1t) {
        case DT_F32: return DSPARK_DOT4(0, DT_F32, 0);
        case DT_BF16: return DSPARK_DOT4(0, DT_BF16, 0);
        default: return DSPARK_DOT4(0, DT_F16, 0);
    }
#undef DSPARK_DOT4
}

}  // namespace dspark
