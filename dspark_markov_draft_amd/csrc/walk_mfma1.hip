// Dense walk for one request on the matrix cores.
//
// What it computes: as the other dense-walk kernels (vLLM PR #62958, int8 DSpark Markov walk,
// Overview and Details; vLLM PR #64476, Claims): l[v] = base[0,t,v] + s[v] * s1 * sum_k q[v,k]
// C[k] (C = 16 hi + lo, the two-digit W1 codes), then the first-maximum argmax (greedy) or the
// Gumbel-max of bf16(l) / temp + noise.
//
// One request makes each step a GEMV, and the lane-per-row v_dot4 kernel spends most of its
// step issuing VALU work: 64 v_dot4 per row plus a move per W2 word held in AGPRs. Here the
// workgroup's W2 rows sit in registers as the A operands of v_mfma_i32_16x16x64_i8 (which reads
// them from AGPRs directly), and the request's W1 digits are the B operand: the high digits in
// columns 0..7, the low digits in columns 8..15, so every column of the 16 x 16 result holds one
// of the two dot products of each of the tile's 16 rows. Lane l receives rows
// 4 (l / 16) .. 4 (l / 16) + 3 of the tile in column l % 16, so among four tiles it finishes one
// row of its own choosing (tile (l / 4) % 4, row 4 (l / 16) + l % 4); lane l ^ 8 holds the same
// rows in the other kind of column and sends it the other dot product with one DPP move. The
// matrix core does 8 times the MACs the method needs (each column holds one of 8 copies), which
// at 16 cycles per MFMA is 40 MFMAs, ~0.3 us per step for a 640-row slice; the VALU only
// finishes three rows per lane.
//
// The workgroup's rows form 16-row tiles dealt round-robin to its 4 waves (tile tw * 4 + wave):
// the first NREG slots of each wave in registers (NREG = 4, 8 or MFMA1_TILES, the fewest that
// hold the slice: every slot is multiplied and finished), up to MFMA1_LDS_TILES more in LDS (a
// K-block of a tile is 64 consecutive 16-byte lane slots there, read without bank conflicts).
// A lane holds, for tile slot tw and K-block kb, bytes kb * 64 + g * 16 .. +15 of its row
// (g = lane / 16), and the W1 codes are read from LDS in the same order: any order of K serves
// if A and B share it, and this one makes each fill instruction read 64 contiguous bytes of each
// of 16 rows (16 cache lines per 1 KB, where the multi-request kernel's order touches 32). Everything else (the per-step W1 gather, base-logit prefetch, the
// running argmax and the grid-wide combine) is the v_dot4 kernel's, so both give the same exact
// int32 sums, logits and tokens.
#include "walk_common.hpp"

namespace dspark {

typedef int v4i1 __attribute__((ext_vector_type(4)));

constexpr int M1_TILE_LDS_BYTES = 4 * WAVE * 16;

// LDS: slices of more than MFMA1_TILES tiles per wave (the LDS tile slots exist); without it the
// kernel has only its NREG register slots, and no code or registers for the others.
template <int SAMPLE, int W1T, int TIMED, int LDS, int NREG>
__global__ __launch_bounds__(WALK_THREADS, 1) void dense_walk_mfma1_kernel(const WalkParams p) {
    static_assert(NREG == MFMA1_TILES || !LDS, "LDS slots follow a full set of register slots");
    constexpr int M1_SLOTS = NREG + (LDS ? MFMA1_LDS_TILES : 0);   // tile slots per wave
    constexpr int M1_GROUPS = (M1_SLOTS + 3) / 4;   // rows each lane finishes per step, at most
    static_assert(M1_GROUPS <= MFMA1_MAX_GROUPS, "LDS for wave 0's base logits");
    stamp<TIMED>(p, 0);
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int c = lane & 15;   // A: row within the tile
    const int g = lane >> 4;   // K group; result rows 4g .. 4g+3
    const int ts = (lane >> 2) & 3;   // which of four tiles this lane finishes a row of
    const int ri = lane & 3;          // and which of its four result rows
    const int row0 = blockIdx.x * p.rows_per_wg;
    const int nrows = min(p.rows_per_wg, p.V - row0);
    const int vend = row0 + nrows;
    const int ntiles = (nrows + 15) / 16;
    // tile slots per wave holding rows; the LDS variant multiplies all its MFMA1_LDS_TILES LDS
    // slots (branch-free), those past nslots hold copies of the slice's first row, not finished
    const int ntl = LDS ? p.lds_units : 0;
    const int nslots = NREG + ntl;

    unsigned char* lds_tiles = smem;
    uint32_t* w1q = reinterpret_cast<uint32_t*>(
        smem + (size_t)(LDS ? MFMA1_LDS_TILES : 0) * WALK_WAVES * M1_TILE_LDS_BYTES);
    float* s1 = reinterpret_cast<float*>(w1q + W1Q_BYTES / 4);
    uint64_t* wkeys = reinterpret_cast<uint64_t*>(s1 + MAX_BS);
    int32_t* tok = reinterpret_cast<int32_t*>(wkeys + WALK_WAVES * MAX_BS);
    uint32_t* w1l = reinterpret_cast<uint32_t*>(tok + MAX_BS);   // the request's low digits
    // wave 0's base logits of the next step, copied by wave 1 (argmax walks without LDS tiles)
    float* pf0 = reinterpret_cast<float*>(w1l + RANK / 4);

    // ---- step 0's W1 codes, by the last wave before its share of the fill ----------------
    // The start token is known at launch, so its row is gathered while the other waves' fill
    // streams in (an out-of-range token reads row 0, as load_start_tokens() makes it); this
    // wave's fill then queues behind two short memory round trips instead of the step waiting
    // for a gather after the whole fill.
    if (wave == WALK_WAVES - 1) {
        int s0 = p.start[0];
        if (s0 < 0 || s0 >= p.V) s0 = 0;
        float sb;
        uint32_t lo;
        const uint32_t codes =
            w1_row_quantise(load4_as_f32<W1T>(p.w1, (int64_t)s0 * RANK + lane * 4), sb, lo);
        w1q[w1q_chunk_dword(0, lane >> 2) + (lane & 3)] = codes;
        w1l[w1q_chunk_dword(0, lane >> 2) + (lane & 3)] = lo;
        if (lane == 0) s1[0] = sb;
    }
    // ---- fill: this wave's tiles as A operands; zero past the slice -----------------------
    v4i1 qa[NREG][4];
#pragma unroll
    for (int tw = 0; tw < NREG; ++tw) {
        const int tl = tw * WALK_WAVES + wave;
        const int row = row0 + tl * 16 + c;
        const bool have = tl < ntiles && row < vend;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            qa[tw][kb] = have ? *reinterpret_cast<const v4i1*>(p.q + (int64_t)row * RANK + kb * 64 + g * 16)
                              : (v4i1){0, 0, 0, 0};
    }
    // LDS slots, copied by DMA straight from memory (a K-block is the 64 consecutive 16-byte lane
    // slots one global_load_lds writes). Rows past the slice copy the slice's first row: their
    // products are never finished.
    for (int tw = NREG; tw < M1_SLOTS; ++tw) {
        const int tl = tw * WALK_WAVES + wave;
        int row = row0 + tl * 16 + c;
        if (!(tw < nslots && tl < ntiles && row < vend)) row = row0;
        unsigned char* dst = lds_tiles + (size_t)((tw - NREG) * WALK_WAVES + wave) * M1_TILE_LDS_BYTES;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            __builtin_amdgcn_global_load_lds(
                (__attribute__((address_space(1))) void*)(p.q + (int64_t)row * RANK + kb * 64 + g * 16),
                (__attribute__((address_space(3))) void*)(dst + kb * WAVE * 16), 16, 0, 0);
    }
    // the rows this lane finishes: group gi takes tile slot 4 gi + ts, row 4 g + ri of it
    int vrow[M1_GROUPS];
    bool vok[M1_GROUPS];
    float sc[M1_GROUPS];
#pragma unroll
    for (int gi = 0; gi < M1_GROUPS; ++gi) {
        const int tw = 4 * gi + ts;
        vrow[gi] = row0 + (tw * WALK_WAVES + wave) * 16 + 4 * g + ri;
        vok[gi] = tw < nslots && vrow[gi] < vend;
        sc[gi] = vok[gi] ? p.scale[vrow[gi]] : 0.0f;
    }
    load_start_tokens(p, tok);

    float pf[M1_GROUPS];   // base logits of the next step to be scored
    auto load_base = [&](int t) {
        const float* br = p.base + (int64_t)t * p.V;
#pragma unroll
        for (int gi = 0; gi < M1_GROUPS; ++gi) pf[gi] = vok[gi] ? br[vrow[gi]] : 0.0f;
    };
    // Wave 0 runs the combine, and loads it issues before would delay its key store and polls
    // (vector memory completes in issue order), so in the argmax walks without LDS tiles wave 1
    // copies wave 0's base logits of the next step into LDS by DMA and waits for them before the
    // step's barrier. (Measured: 32.0 -> 31.7 us at T = 7, 61.5 -> 60.6 at T = 16; with LDS
    // tiles, where wave 1 has more to copy, 1 us slower at T = 16, so not there.)
    constexpr bool W0_LDS = SAMPLE != 2 && !LDS;
    auto copy_base_w0 = [&](int t) {
        const float* br = p.base + (int64_t)t * p.V;
#pragma unroll
        for (int gi = 0; gi < M1_GROUPS; ++gi) {
            const int tw = 4 * gi + ts;
            const int r = row0 + tw * WALK_WAVES * 16 + 4 * g + ri;   // wave 0's row
            const bool ok = tw < nslots && r < vend;
            __builtin_amdgcn_global_load_lds(
                (__attribute__((address_space(1))) void*)(br + (ok ? r : row0)),
                (__attribute__((address_space(3))) void*)(pf0 + gi * WAVE), 4, 0, 0);
        }
    };
    load_base(0);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's tile copies have landed, and every wave's
    __syncthreads();                  // after the barrier
    stamp<TIMED>(p, 1);

    uint64_t seed = 0;
    uint64_t pos0 = 0;
    float rtemp = 1.0f;
    if constexpr (SAMPLE) {
        seed = p.seeds[0];
        pos0 = (uint64_t)(p.positions ? p.positions[0] : 0);
        rtemp = inv_temperature(p.temps[0]);
    }
    const float kz = rtemp * LOG2E_F;   // inverse CDF: z = lb * log2(e) / temp

    for (int t = 0; t < p.T; ++t) {
        // every wave's base logits of this step were issued before the previous combine: the
        // first poll round waits behind them (vector memory returns in issue order), which costs
        // little, as the combine waits for the last workgroup anyway, while the W1 row of wave 0's
        // gather has nothing queued ahead of it
        if (t > 0) {
            gather_w1_codes<W1T, LOW_BYTES>(p, tok, w1q, w1l, s1, wave, lane, [&] {});
            __syncthreads();
        }
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 0);

        float cur[M1_GROUPS];
        if (W0_LDS && wave == 0 && t > 0) {
#pragma unroll
            for (int gi = 0; gi < M1_GROUPS; ++gi) cur[gi] = vok[gi] ? pf0[gi * WAVE + lane] : 0.0f;
        } else {
#pragma unroll
            for (int gi = 0; gi < M1_GROUPS; ++gi) cur[gi] = pf[gi];
        }
        v4i1 bop[4];
        const uint32_t* wd = c < 8 ? w1q : w1l;   // column c: high digits, or low from 8 on
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            bop[kb] = *reinterpret_cast<const v4i1*>(wd + w1q_chunk_dword(0, kb * 4 + g));
        const float sb = s1[0];

        // every register slot's MFMAs first (slots past the slice hold zero codes), then the LDS
        // slots', then the finish
        v4i1 acc[M1_SLOTS];
#pragma unroll
        for (int tw = 0; tw < NREG; ++tw) {
            acc[tw] = (v4i1){0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc[tw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[tw][kb], bop[kb], acc[tw], 0, 0, 0);
        }
#pragma unroll
        for (int tw = NREG; tw < M1_SLOTS; ++tw) {
            acc[tw] = (v4i1){0, 0, 0, 0};
            const v4i1* src = reinterpret_cast<const v4i1*>(
                lds_tiles + (size_t)((tw - NREG) * WALK_WAVES + wave) * M1_TILE_LDS_BYTES);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc[tw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(src[kb * WAVE + lane], bop[kb],
                                                                acc[tw], 0, 0, 0);
        }
        const int64_t orow = (int64_t)t * p.V;
        const uint64_t P = pos0 + (uint64_t)t;
        // Gumbel noise: the four lanes of a quad (ri = 0..3) finish the four rows of one 4-row
        // group in each row group gi, and one Philox call yields those four words. So lane ri
        // draws the call of group ri + 4k alone, and the quad shares the words below, instead of
        // every lane drawing every group's call for one word of it.
        constexpr int NCALL = (M1_GROUPS + 3) / 4;
        uint4 nw[SAMPLE == 1 ? NCALL : 1];
        if constexpr (SAMPLE == 1) {
#pragma unroll
            for (int k = 0; k < NCALL; ++k) {
                int vr = vrow[0];   // (a lane past the last group draws group 0's call, unused)
#pragma unroll
                for (int gi = 1; gi < M1_GROUPS; ++gi) vr = ri + 4 * k == gi ? vrow[gi] : vr;
                nw[k] = philox4x32_10((uint32_t)vr >> 2, (uint32_t)P, (uint32_t)(P >> 32), 0u,
                                      (uint32_t)seed, (uint32_t)(seed >> 32));
            }
        }
        // word ri of the call that quad lane s drew: broadcast within the quad, then chosen
        auto quad_word = [&](const uint4 w, int s) -> uint32_t {
            uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                switch (s) {
                    case 0: x[i] = dpp_u32<0x00>(x[i]); break;
                    case 1: x[i] = dpp_u32<0x55>(x[i]); break;
                    case 2: x[i] = dpp_u32<0xAA>(x[i]); break;
                    default: x[i] = dpp_u32<0xFF>(x[i]); break;
                }
            }
            return ri == 0 ? x[0] : ri == 1 ? x[1] : ri == 2 ? x[2] : x[3];
        };
        RunningArgmax run;
        RunningSoftmax soft;
#pragma unroll
        for (int gi = 0; gi < M1_GROUPS; ++gi) {
            // this lane's row of tile slot 4 gi + ts: component ri of that slot's result
            int a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tw = 4 * gi + j;
                const v4i1 x = tw < M1_SLOTS ? acc[tw] : (v4i1){0, 0, 0, 0};
                int s = x[0];
                s = ri == 1 ? x[1] : s;
                s = ri == 2 ? x[2] : s;
                s = ri == 3 ? x[3] : s;
                a[j] = s;
            }
            // this lane's product (column l % 16: high digits for ts < 2) and, for lane l ^ 8,
            // the product of the row that lane finishes (tile slot 4 gi + (ts ^ 2), the other
            // kind of column), exchanged by a rotation of each 16-lane row by 8
            int mine = a[0], theirs = a[2];
            mine = ts == 1 ? a[1] : mine;
            theirs = ts == 1 ? a[3] : theirs;
            mine = ts == 2 ? a[2] : mine;
            theirs = ts == 2 ? a[0] : theirs;
            mine = ts == 3 ? a[3] : mine;
            theirs = ts == 3 ? a[1] : theirs;
            const int other = __builtin_amdgcn_update_dpp(theirs, theirs, DPP_ROW_ROR8, 0xF, 0xF, false);
            const int dot = ts < 2 ? join_digits(mine, other) : join_digits(other, mine);
            const int v = vrow[gi];
            const float l = walk_logit(cur[gi], sc[gi], sb, dot);
            if constexpr (!SAMPLE) {
                if (p.out_logits && vok[gi]) p.out_logits[orow + v] = l;
                run.offer(l, (uint32_t)v, vok[gi]);
            } else if constexpr (SAMPLE == 1) {
                const uint32_t h = bf16_bits(l);
                if (vok[gi]) p.draft_logits[orow + v] = (uint16_t)h;
                const float x = bf16_value(h) * rtemp;
                const float gn = gumbel_from_word(quad_word(nw[gi / 4], gi % 4));
                run.offer(x + gn, (uint32_t)v, vok[gi]);
            } else {
                const uint32_t h = bf16_bits(l);
                if (vok[gi]) p.draft_logits[orow + v] = (uint16_t)h;
                soft.offer(bf16_value(h) * kz, vok[gi]);
            }
        }
        if constexpr (SAMPLE == 2) {
            wave_softmax(soft.m, soft.s);
            if (lane == 0) wkeys[wave * MAX_BS] = pack_softmax(soft.m, soft.s);
        } else {
            const uint64_t best = wave_max_u64(run.key());
            if (lane == 0) wkeys[wave * MAX_BS] = best;
        }
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 1);

        // the next step's base logits load while the combine waits (wave 0's: above)
        if (t + 1 < p.T) {
            if (!W0_LDS || wave != 0) load_base(t + 1);
            if (W0_LDS && wave == 1) {
                copy_base_w0(t + 1);
                __builtin_amdgcn_s_waitcnt(0);   // landed before the step's last barrier
            }
        }
        if (wave == 0) {
            uint64_t k = 0;
            if constexpr (SAMPLE == 2) {
                RunningSoftmax a;
#pragma unroll
                for (int w = 0; w < WALK_WAVES; ++w) {
                    const uint64_t o = wkeys[w * MAX_BS];
                    a.merge(packed_m(o), packed_s(o));
                }
                k = pack_softmax(a.m, a.s);
                combine_icdf_step<TIMED>(p, t, k, tok, lane);
            } else {
                if (lane == 0) {
                    uint64_t o[WALK_WAVES];
#pragma unroll
                    for (int w = 0; w < WALK_WAVES; ++w) o[w] = wkeys[w * MAX_BS];
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

template <int LDS, int NREG>
static const void* mfma1_kernel_for(int sample, int w1t, bool timed) {
#define DSPARK_MFMA1(S, W, TI) reinterpret_cast<const void*>(&dense_walk_mfma1_kernel<S, W, TI, LDS, NREG>)
    if (sample == 2) {
        switch (w1t) {
            case DT_F32: return DSPARK_MFMA1(2, DT_F32, 0);
            case DT_BF16: return DSPARK_MFMA1(2, DT_BF16, 0);
            default: return DSPARK_MFMA1(2, DT_F16, 0);
        }
    }
    if (timed) return sample ? DSPARK_MFMA1(1, DT_BF16, 1) : DSPARK_MFMA1(0, DT_BF16, 1);
    if (sample) {
        switch (w1t) {
            case DT_F32: return DSPARK_MFMA1(1, DT_F32, 0);
            case DT_BF16: return DSPARK_MFMA1(1, DT_BF16, 0);
            default: return DSPARK_MFMA1(1, DT_F16, 0);
        }
    }
    switch (w1t) {
        case DT_F32: return DSPARK_MFMA1(0, DT_F32, 0);
        case DT_BF16: return DSPARK_MFMA1(0, DT_BF16, 0);
        default: return DSPARK_MFMA1(0, DT_F16, 0);
    }
#undef DSPARK_MFMA1
}

const void* mfma1_walk_kernel(int sample, int w1t, bool timed, bool lds_tiles, int reg_slots) {
    if (lds_tiles) return mfma1_kernel_for<1, MFMA1_TILES>(sample, w1t, timed);
    if (reg_slots <= 4) return mfma1_kernel_for<0, 4>(sample, w1t, timed);
    if (reg_slots <= 8) return mfma1_kernel_for<0, 8>(sample, w1t, timed);
    return mfma1_kernel_for<0, MFMA1_TILES>(sample, w1t, timed);
}

}  // namespace dspark
