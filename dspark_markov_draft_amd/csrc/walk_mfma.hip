// Dense walk, matrix-core kernel (used for two or more requests, where each step is a GEMM of
// W2 [V x 256] with the requests' W1 codes [256 x bs]).
//
// What it computes: as the v_dot4 kernel (vLLM PR #62958, int8 DSpark Markov walk, Overview
// and Details; vLLM PR #64476, Claims): l[v] = base[b,t,v] + s[v] * s1_b * sum_k q[v,k] C_b[k]
// (C = 16 hi + lo, the two-digit W1 codes), then the first-maximum argmax (greedy), the
// Gumbel-max of bf16(l) / temp + noise (sample), or (inverse CDF) each lane's running softmax
// pair of z = bf16(l) * log2(e) / temp, merged per request and handed to combine_icdf_step().
//
// v_mfma_i32_16x16x64_i8 multiplies a 16 x 64 int8 tile by a 64 x 16 int8 tile into 16 x 16
// int32. Lane l supplies row l % 16 of A and column l % 16 of B, each for the k-chunk of lane
// group l / 16, and receives D[(l / 16) * 4 + i][l % 16], i < 4. Here A = 16 rows of W2 and
// B = the W1 digits of 16 requests; lane group g carries bytes g*64 + kb*16 .. +15 of the row in
// K-block kb, so over the four K-blocks a lane holds one contiguous 64-byte quarter of its row.
// Each tile's accumulator takes the high digits' 4 MFMAs, is shifted left by 4, and takes the
// low digits' 4 MFMAs: 16 * (high sum) + (low sum), the exact integer of the other kernels. The
// low digits sit in LDS as nibbles (8 KB for 64 requests) and are widened to int8 when read.
//
// The workgroup's rows form 16-row tiles dealt round-robin to its waves: 8 waves (two per SIMD)
// with 5 or 4 tiles each in registers for slices of up to 624 rows, otherwise 4 waves that keep
// up to 8 tiles (128 rows) in VGPRs as ready A operands, further tiles in LDS (laid out so a
// K-block read is 64 consecutive 16-byte lane slots), and stream any rest from memory. Per
// step and 16-request tile: 8 MFMAs per W2 tile; each lane then finishes 4 consecutive rows of
// one request (one float4 of base logits, one Philox call for the 4 noise words), keeps its
// best key, the four lanes of a request in a wave merge theirs with two lane swaps, and the
// workgroup's best per request goes to combine_step().
//
// The base logits of a 16-request tile (16 rows of the workgroup's slice) are copied into LDS
// by global_load_lds DMA before the tile is used (one latency per request tile instead of one
// per W2 tile): with two staging buffers the next request tile's copy runs under the current
// one's compute, and the first tile of step t+1 is fetched while the combine of step t waits.
// Staging rows are padded to an odd number of 16-byte units, so the 16 requests a wave reads
// at once fall into different LDS banks. The kernel needs V % 4 == 0 and 16-byte aligned rows
// (the host runs the v_dot4 kernel otherwise): every 4-row group is then wholly inside or
// wholly outside the slice, and its base logits, scales and outputs move as one vector.
#include "walk_common.hpp"

namespace dspark {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

constexpr int TILE_ROWS = 16;
constexpr int NT_REG = 8;                       // W2 tiles per wave held in VGPRs
constexpr int TILE_LDS_BYTES = 4 * WAVE * 16;   // one tile: 4 K-blocks x 64 lanes x 16 bytes
constexpr int MAX_RT = MAX_BS / 16;             // 16-request tiles
static_assert(mfma_static_max_slots(4) == NT_REG + mfma_static_lds_slots(mfma_static_max_slots(4), 4),
              "STAT tile slots");
// copy instructions per wave for one request tile with STAT: one after each tile slot, and the
// rest (a build with fewer slots) after the last
__host__ __device__ constexpr int stat_copy_slots(int waves) {
    return MFMA_STATIC_COPY_UNITS / WAVE / waves;
}
static_assert(MFMA_STATIC_COPY_UNITS % (WAVE * 8) == 0 && stat_copy_slots(4) == mfma_static_max_slots(4) &&
                  stat_copy_slots(8) == mfma_static_max_slots(8),
              "STAT copy slots");
// the workgroup's best key per request (argmax), or each wave's softmax pair per request
// (inverse CDF)
__host__ __device__ constexpr int lkey_bytes(int sample, int waves) {
    return (sample == 2 ? waves : 1) * MAX_BS * 8;
}
constexpr int LKEY_BYTES = lkey_bytes(2, WALK_WAVES);   // the dynamic layout reserves the larger

// dynamic LDS besides the W2 tiles: W1 digits, their steps, row scales, wave keys, tokens
__host__ __device__ constexpr int mfma_fixed_lds(int rows_per_wg) {
    return W1Q_BYTES + W1N_BYTES + MAX_BS * 4 + ((rows_per_wg * 4 + 15) / 16) * 16 + LKEY_BYTES +
           MAX_BS * 4;
}

// STAT (slices of up to MFMA_STATIC_ROWS rows): every LDS buffer is a static array of its own
// (two staging buffers, the LDS tiles, W1 codes, scales, lane keys, tokens) and there is no
// dynamic LDS. The compiler then knows that the DMA into one staging buffer cannot touch the
// other one or any other LDS data, and reads them while the DMA runs. With dynamic LDS it has
// to assume that any LDS read may alias the DMA's target, and waits for every DMA in flight
// before each LDS read, which serialises the next request tile's copy with the current tile's
// compute. NT: the tile slots per wave with STAT (mfma_static_slots()). NW: the waves, 4 (one
// per SIMD), or 8 with STAT (two per SIMD, half the registers each: while one waits, for its
// memory or in the issue of a copy, the other computes).
template <int SAMPLE, int W1T, int TIMED, int STAT, int OUTL, int NT, int NW>
__global__ __launch_bounds__(NW * WAVE, 1) void dense_walk_mfma_kernel(const WalkParams p) {
    static_assert(NW == 4 || (NW == 8 && STAT), "waves");
    constexpr int NTHREADS = NW * WAVE;
    constexpr int NT_STAT = NT;
    constexpr int LDS_SLOTS = STAT ? mfma_static_lds_slots(NT, NW) : 0;   // of the NT
    constexpr int STAT_COPY_SLOTS = stat_copy_slots(NW);
    stamp<TIMED>(p, 0);
    extern __shared__ __align__(16) unsigned char smem[];
    // the staging buffers and row scales are padded for the past-the-end tile slots (below)
    __shared__ __align__(16) float stage_a[STAT ? MFMA_STATIC_STAGE_FLOATS : 4];
    __shared__ __align__(16) float stage_b[STAT ? MFMA_STATIC_STAGE_FLOATS : 4];
    // W2 tile slots per wave in registers (the rest of the NT_STAT slots with STAT are in LDS)
    constexpr int NTR = STAT ? NT_STAT - LDS_SLOTS : NT_REG;
    __shared__ __align__(16) unsigned char tiles_s[LDS_SLOTS ? LDS_SLOTS * NW * TILE_LDS_BYTES : 16];
    __shared__ __align__(16) uint32_t w1q_s[STAT ? W1Q_BYTES / 4 : 4];
    __shared__ __align__(16) uint32_t w1n_s[STAT ? W1N_BYTES / 4 : 4];
    __shared__ __align__(16) float s1_s[STAT ? MAX_BS : 4];
    __shared__ __align__(16) float scl_s[STAT ? MFMA_STATIC_SLOT_ROWS : 4];
    __shared__ __align__(16) uint64_t lkeys_s[STAT ? lkey_bytes(SAMPLE, NW) / 8 : 2];
    __shared__ __align__(16) int32_t tok_s[STAT ? MAX_BS : 4];
    __shared__ __align__(16) uint64_t rq_seed[SAMPLE == 1 ? MAX_BS : 2];
    __shared__ __align__(16) uint64_t rq_pos[SAMPLE == 1 ? MAX_BS : 2];
    __shared__ __align__(16) float rq_rtemp[SAMPLE ? MAX_BS : 4];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);   // uniform: scalar branches
    const int c = lane & 15;   // A: row within the tile; B/D: request within the request tile
    const int g = lane >> 4;   // k-chunk group; D: rows g*4 .. g*4+3
    const int row0 = blockIdx.x * p.rows_per_wg;
    const int nrows = min(p.rows_per_wg, p.V - row0);
    const int vend = row0 + nrows;
    const int ntiles = (nrows + TILE_ROWS - 1) / TILE_ROWS;   // tiles of this workgroup
    const int ntw = p.total_units;                             // tile slots per wave
    const int lds_tw = p.lds_units;

    // dynamic layout (without STAT): LDS tiles, staging buffers, W1 high digits, low digits,
    // their steps, row scales, wave keys, tokens
    unsigned char* const d_tiles = smem;
    float* const d_stage = reinterpret_cast<float*>(smem + (size_t)lds_tw * NW * TILE_LDS_BYTES);
    const int ss = p.stage_stride;
    const int nbuf = p.stage_bufs;   // 1 or 2 (the host guarantees at least one)
    uint32_t* const d_w1q = reinterpret_cast<uint32_t*>(d_stage + (size_t)p.stage_bufs * 16 * ss);
    uint32_t* const d_w1n = d_w1q + W1Q_BYTES / 4;
    float* const d_s1 = reinterpret_cast<float*>(d_w1n + W1N_BYTES / 4);
    float* const d_scl = d_s1 + MAX_BS;
    uint64_t* const d_lkeys = reinterpret_cast<uint64_t*>(d_scl + ((p.rows_per_wg * 4 + 15) / 16) * 4);
    unsigned char* lds_tiles = STAT ? tiles_s : d_tiles;
    float* const buf0 = STAT ? stage_a : d_stage;
    float* const buf1 = STAT ? stage_b : d_stage + (size_t)16 * ss;
    uint32_t* w1q = STAT ? w1q_s : d_w1q;
    uint32_t* w1n = STAT ? w1n_s : d_w1n;
    float* s1 = STAT ? s1_s : d_s1;
    float* scl = STAT ? scl_s : d_scl;
    uint64_t* lkeys = STAT ? lkeys_s : d_lkeys;
    int32_t* tok = STAT ? tok_s : reinterpret_cast<int32_t*>(d_lkeys + LKEY_BYTES / 8);

    // ---- fill: W2 tiles as A operands (VGPRs, then LDS), row scales into LDS ---------------
    auto load_a = [&](int tl, int kb) -> v4i {
        const int row = row0 + tl * TILE_ROWS + c;
        if (row >= vend) return (v4i){0, 0, 0, 0};
        return *reinterpret_cast<const v4i*>(p.q + (int64_t)row * RANK + g * 64 + kb * 16);
    };
    v4i qa[NTR][4];
#pragma unroll
    for (int tw = 0; tw < NTR; ++tw) {
        const int tl = tw * NW + wave;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) qa[tw][kb] = tl < ntiles ? load_a(tl, kb) : (v4i){0, 0, 0, 0};
    }
    // with STAT every LDS slot is written (zero codes past the slice's tiles): the tile loop
    // multiplies all of them
    for (int tw = NTR; tw < NTR + (STAT ? LDS_SLOTS : lds_tw); ++tw) {
        const int tl = tw * NW + wave;
        const bool have = tl < ntiles && tw < NTR + lds_tw;
        if (have || STAT) {
            v4i* dst = reinterpret_cast<v4i*>(
                lds_tiles + (size_t)((tw - NTR) * NW + wave) * TILE_LDS_BYTES);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                dst[kb * WAVE + lane] = have ? load_a(tl, kb) : (v4i){0, 0, 0, 0};
        }
    }
    for (int i = tid; i < (STAT ? MFMA_STATIC_SLOT_ROWS : ntiles * TILE_ROWS); i += NTHREADS)
        scl[i] = i < nrows ? p.scale[row0 + i] : 0.0f;
    load_start_tokens(p, tok);
    if (tid < MAX_BS) lkeys[tid] = 0;   // the per-request key words start empty
    if constexpr (SAMPLE) {
        // read once here rather than at every request tile, where each read was a round trip
        if (tid < p.bs) {
            if constexpr (SAMPLE == 1) {
                rq_seed[tid] = p.seeds[tid];
                rq_pos[tid] = (uint64_t)(p.positions ? p.positions[tid] : 0);
            }
            rq_rtemp[tid] = inv_temperature(p.temps[tid]);
        }
    }
    __syncthreads();
    stamp<TIMED>(p, 1);

    const int nrt = (p.bs + 15) / 16;

    // DMA of base[rt*16 .. rt*16+15, t, row0 .. vend) into staging buffer `buf`: each wave
    // instruction moves 64 lanes x 16 bytes to consecutive LDS; row segments are whole 16-byte
    // units (V and row0 are multiples of 4) and lanes past a segment's end stay idle.
    const int units = nrows / 4;
    // STAT: the copy of a request tile is one flat list of full instructions over the buffer's
    // 16-byte units. Unit L is unit L % upr of row L / upr (upr: units per padded row), and
    // instruction j (units 64j .. 64j+63) belongs to wave j % NW, so each wave has at most
    // STAT_COPY_SLOTS of them and can issue them one at a time between its tile slots: a wave
    // that issues many copies back to back while HBM is busy stalls in the issue itself. Pad
    // units, and units past the tile's last valid request (last instruction only), copy an
    // in-bounds unit of the slice; no valid row ever reads them. The division is a multiply and
    // shift, exact for L < 2^12 and upr <= 157 (the error stays below 2^-8 < 1/upr).
    const int upr = ss / 4;
    const uint32_t upr_inv = (1u << 20) / (uint32_t)upr + 1u;
    auto copy_job = [&](int rt, int t, float* dst_buf, int j) {
        const int nv = min(16, p.bs - rt * 16);              // valid requests of the tile (>= 1)
        if (j * WAVE >= nv * upr) return;                     // past the tile's instructions
        int L = j * WAVE + lane;                              // < MFMA_STATIC_COPY_UNITS
        // computed where issued: hoisted out of the step loop, the addresses of every slot's
        // copy would hold registers the tile loop needs
        asm volatile("" : "+v"(L));
        const int r = (int)(((uint32_t)L * upr_inv) >> 20);
        const int u = L - r * upr;
        const int rc = min(r, nv - 1), uc = min(u, units - 1);
        const float* src = p.base + ((int64_t)(rt * 16 + rc) * p.T + t) * p.V + row0 + 4 * uc;
        __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(dst_buf + j * WAVE * 4),
                                         16, 0, 0);
    };
    auto stage_base = [&](int rt, int t, float* dst_buf) {
        if constexpr (STAT) {
            for (int s = 0; s < STAT_COPY_SLOTS; ++s) copy_job(rt, t, dst_buf, s * NW + wave);
            return;
        }
        for (int r = 0; r < 16; ++r) {
            const int b = rt * 16 + r;
            if (b >= p.bs) break;
            const float* src = p.base + ((int64_t)b * p.T + t) * p.V + row0;
            float* dst = dst_buf + (size_t)r * ss;
            for (int u0 = wave * WAVE; u0 < units; u0 += NTHREADS) {
                if (u0 + lane < units)
                    __builtin_amdgcn_global_load_lds((global_void_ptr)(src + 4 * (u0 + lane)),
                                                     (lds_void_ptr)(dst + 4 * u0), 16, 0, 0);
            }
        }
    };
    stage_base(0, 0, buf0);
    // The same copy issued by waves 1-3 only: wave 0 runs the combine right after, and a copy it
    // issued would delay its slot store (a wave issuing copies while HBM is busy stalls in the
    // issue) and its polls (they would complete behind the copy, in issue order).
    auto stage_base_w123 = [&](int rt, int t, float* dst_buf) {
        if (wave == 0) return;
        if constexpr (STAT) {
            for (int j = wave - 1; j < STAT_COPY_SLOTS * NW; j += NW - 1)
                copy_job(rt, t, dst_buf, j);
            return;
        }
        for (int r = 0; r < 16; ++r) {
            const int b = rt * 16 + r;
            if (b >= p.bs) break;
            const float* src = p.base + ((int64_t)b * p.T + t) * p.V + row0;
            float* dst = dst_buf + (size_t)r * ss;
            for (int u0 = (wave - 1) * WAVE; u0 < units; u0 += NTHREADS - WAVE) {
                if (u0 + lane < units)
                    __builtin_amdgcn_global_load_lds((global_void_ptr)(src + 4 * (u0 + lane)),
                                                     (lds_void_ptr)(dst + 4 * u0), 16, 0, 0);
            }
        }
    };

    for (int t = 0; t < p.T; ++t) {
        gather_w1_codes<W1T, LOW_NIBBLES, STAT ? 4 : 2, NW>(p, tok, w1q, w1n, s1, wave, lane, [] {});
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 0);

        // one request tile: its base logits are in `cur`; the next tile's copy goes to `nxt`
        auto request_tile = [&](int rt, float* cur, float* nxt) __attribute__((always_inline)) {
            if (nbuf == 1 && rt > 0) {
                __syncthreads();   // every wave is done with the previous request tile
                stage_base(rt, t, cur);
            }
            // This tile's base logits have landed: this wave's copies, then (barrier) every other
            // wave's; past the barrier every wave is also done with the buffer that the next
            // copy overwrites. With STAT the tile's MFMAs, which need no base logit, are issued
            // before this wait and run while the copy lands; the next tile's copy is issued
            // after it (the wait counts every load in flight).
            auto landed = [&]() {
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                stamp<TIMED>(p, STAMP_TILE0 + (t * STAMP_TILES + rt) * 2);
            };
            if constexpr (!STAT) landed();
            const bool prefetch = nbuf == 2 && rt + 1 < nrt;
            if (!STAT && prefetch) stage_base(rt + 1, t, nxt);
            const float* sbase = cur + (size_t)c * ss;
            const int b = rt * 16 + c;
            const bool vb = b < p.bs;
            // Column c of the result depends only on column c of B, and the columns of requests
            // past bs are dropped: their digits are read (in bounds: the arrays hold 64
            // requests) without a branch, whatever the LDS holds there.
            auto high_op = [&](int kb) -> v4i {
                return *reinterpret_cast<const v4i*>(w1q + w1q_chunk_dword(b, g * 4 + kb));
            };
            // low digits, widened from their nibbles
            auto low_op = [&](int kb) -> v4i {
                const uint4 x = unpack_low_digits(
                    *reinterpret_cast<const uint2*>(w1n + w1n_chunk_dword(b, g * 4 + kb)));
                return (v4i){(int)x.x, (int)x.y, (int)x.z, (int)x.w};
            };
            // both digits' B operands of the request tile, read together (one LDS wait)
            v4i bop[4], bol[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bop[kb] = high_op(kb);
                bol[kb] = low_op(kb);
            }
            const float sb = vb ? s1[b] : 0.0f;
            uint64_t seed = 0, P = 0;
            float rtemp = 1.0f;
            if constexpr (SAMPLE) {
                if (vb) {
                    // volatile: read here, not hoisted out of the step loop, where every request
                    // tile's values would hold registers through the whole walk
                    if constexpr (SAMPLE == 1) {
                        seed = *reinterpret_cast<volatile uint64_t*>(&rq_seed[b]);
                        P = *reinterpret_cast<volatile uint64_t*>(&rq_pos[b]) + (uint64_t)t;
                    }
                    rtemp = *reinterpret_cast<volatile float*>(&rq_rtemp[b]);
                }
            }
            const PhiloxRun prun = philox_run(seed, P);
            const float kz = rtemp * LOG2E_F;   // inverse CDF: z = lb * log2(e) / temp
            // Rows vt .. vt+3 of request b from the accumulator of one tile: their logits (and
            // bf16 rows and noise when sampling), the quantity the argmax compares, and in `out`
            // the bits store4 writes (fp32 logits, or two words of bf16 pairs). The group is
            // wholly inside the slice or wholly past its end (partial last tile); past-the-end
            // groups (and, with STAT, slots past the slice's tiles: the arrays are padded for
            // them) and requests past bs read in-bounds LDS, are computed, and are dropped.
            auto scores4 = [&](const v4i acc, int vt, float (&sc)[4], uint32_t (&out)[4]) {
                const int off = vt - row0;
                const float4 sv = *reinterpret_cast<const float4*>(scl + off);
                const float4 bv = *reinterpret_cast<const float4*>(sbase + off);
                const bool ok = vb && vt < vend;
                float l[4];
                l[0] = walk_logit(bv.x, sv.x, sb, acc[0]);
                l[1] = walk_logit(bv.y, sv.y, sb, acc[1]);
                l[2] = walk_logit(bv.z, sv.z, sb, acc[2]);
                l[3] = walk_logit(bv.w, sv.w, sb, acc[3]);
                if constexpr (!SAMPLE) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sc[i] = l[i];
                        out[i] = __float_as_uint(l[i]);
                    }
                } else if constexpr (SAMPLE == 2) {
                    out[0] = bf16x2_bits(l[0], l[1]);
                    out[1] = bf16x2_bits(l[2], l[3]);
                    out[2] = out[3] = 0;
                    sc[0] = bf16_lo(out[0]) * kz;
                    sc[1] = bf16_hi(out[0]) * kz;
                    sc[2] = bf16_lo(out[1]) * kz;
                    sc[3] = bf16_hi(out[1]) * kz;
                } else {
                    out[0] = bf16x2_bits(l[0], l[1]);
                    out[1] = bf16x2_bits(l[2], l[3]);
                    out[2] = out[3] = 0;
                    const float x[4] = {bf16_lo(out[0]), bf16_hi(out[0]), bf16_lo(out[1]),
                                        bf16_hi(out[1])};
                    // vt is a multiple of 4: one Philox call yields the words of all 4 rows
                    const uint4 w = philox_run_words(prun, (uint32_t)vt >> 2);
                    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[i] = x[i] * rtemp + gumbel_from_word(words[i]);
                }
                return ok;
            };
            // writes what scores4 left in `out` (greedy: only when the caller asked for logits).
            // The row offset is computed here, not once per request tile: held through the tile,
            // its two registers were spilled.
            auto store4 = [&](int vt, bool ok, const uint32_t (&out)[4]) {
                int bo = vb ? b : 0;
                asm volatile("" : "+v"(bo));
                const int64_t orow = ((int64_t)bo * p.T + t) * p.V;
                if constexpr (!SAMPLE) {
                    if (p.out_logits != nullptr && ok)
                        *reinterpret_cast<uint4*>(p.out_logits + orow + vt) =
                            make_uint4(out[0], out[1], out[2], out[3]);
                } else {
                    if (ok)
                        *reinterpret_cast<uint2*>(p.draft_logits + orow + vt) =
                            make_uint2(out[0], out[1]);
                }
            };

            // Every tile of this wave in increasing row order: register tiles (all their MFMAs
            // first, each into its own accumulator, so the matrix core runs ahead while the VALU
            // finishes tile after tile), then LDS tiles, then streamed ones.
            auto for_tiles = [&](auto&& fin, auto&& after, auto&& half_end) {
                if constexpr (STAT) {
                    // At most NT_STAT tile slots per wave, all on chip: every slot's MFMAs are
                    // issued first and every slot is finished, with no branch on the tile, so
                    // the compiler can overlap one tile's LDS reads with another's arithmetic.
                    // Slots past the slice's tiles hold zero codes and their rows are past vend.
                    auto a_op = [&](int tw, int kb) -> v4i {
                        if (tw < NTR) return qa[tw][kb];
                        return reinterpret_cast<const v4i*>(
                            lds_tiles + (size_t)((tw - NTR) * NW + wave) *
                                            TILE_LDS_BYTES)[kb * WAVE + lane];
                    };
                    // The sampling kernel takes the slots in two halves (half the accumulators
                    // live at a time), the greedy kernel in one pass. A pass: the high digits'
                    // MFMAs, every accumulator times 16, the low digits' MFMAs (K-block by
                    // K-block, so that consecutive MFMAs feed different accumulators), then the
                    // finish. The first pass's MFMAs run before the wait for this tile's base
                    // logits. The next tile's copy instructions are spread: one behind each
                    // finished slot of the first pass, and in a later pass one behind each
                    // group of its MFMAs (a copy whose issue stalls while HBM is busy then stalls
                    // the wave only while the matrix core works through the group before it).
                    constexpr int HALF = SAMPLE == 1 ? (NT_STAT + 1) / 2 : NT_STAT;
#pragma unroll
                    for (int h0 = 0; h0 < NT_STAT; h0 += HALF) {
                        constexpr int n = HALF;
                        const bool first = h0 == 0;
                        v4i accs[n];
#pragma unroll
                        for (int i = 0; i < n; ++i) accs[i] = (v4i){0, 0, 0, 0};
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const v4i bh = bop[kb];
#pragma unroll
                            for (int i = 0; i < n; ++i)
                                if (h0 + i < NT_STAT)
                                    accs[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                        a_op(h0 + i, kb), bh, accs[i], 0, 0, 0);
                            if (!first && kb < n && h0 + kb < NT_STAT) after(h0 + kb);
                        }
#pragma unroll
                        for (int i = 0; i < n; ++i) accs[i] = accs[i] << 4;
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const v4i bl = bol[kb];
#pragma unroll
                            for (int i = 0; i < n; ++i)
                                if (h0 + i < NT_STAT)
                                    accs[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                                        a_op(h0 + i, kb), bl, accs[i], 0, 0, 0);
                            if (!first && 4 + kb < n && h0 + 4 + kb < NT_STAT) after(h0 + 4 + kb);
                        }
                        if (!first) {
                            // a pass of more than 8 slots: its last copy instructions
#pragma unroll
                            for (int i = 8; i < n; ++i)
                                if (h0 + i < NT_STAT) after(h0 + i);
                        }
                        if (first) landed();
#pragma unroll
                        for (int i = 0; i < n; ++i) {
                            const int tw = h0 + i;
                            if (tw < NT_STAT) {
                                fin(accs[i], row0 + (tw * NW + wave) * TILE_ROWS + g * 4, tw);
                                if (first) after(tw);
                            }
                        }
                        half_end(h0);
                    }
                    return;
                }
                v4i accs[NTR];
#pragma unroll
                for (int tw = 0; tw < NTR; ++tw) {
                    accs[tw] = (v4i){0, 0, 0, 0};
                    if (tw * NW + wave < ntiles) {
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
                            accs[tw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[tw][kb], bop[kb],
                                                                             accs[tw], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int tw = 0; tw < NTR; ++tw) {
                    if (tw * NW + wave < ntiles) {
                        accs[tw] = accs[tw] << 4;
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
                            accs[tw] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[tw][kb], bol[kb],
                                                                             accs[tw], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int tw = 0; tw < NTR; ++tw) {
                    const int tl = tw * NW + wave;
                    if (tl < ntiles) fin(accs[tw], row0 + tl * TILE_ROWS + g * 4, tw);
                }
                for (int tw = NTR; tw < ntw; ++tw) {
                    const int tl = tw * NW + wave;
                    if (tl < ntiles) {
                        // the tile's A operands read once (from LDS or memory) for both digits
                        v4i a4[4];
                        if (tw < NTR + lds_tw) {
                            const v4i* src = reinterpret_cast<const v4i*>(
                                lds_tiles + (size_t)((tw - NTR) * NW + wave) * TILE_LDS_BYTES);
#pragma unroll
                            for (int kb = 0; kb < 4; ++kb) a4[kb] = src[kb * WAVE + lane];
                        } else {
#pragma unroll
                            for (int kb = 0; kb < 4; ++kb) a4[kb] = load_a(tl, kb);
                        }
                        v4i acc = {0, 0, 0, 0};
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
                            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a4[kb], bop[kb], acc, 0, 0, 0);
                        acc = acc << 4;
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb)
                            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a4[kb], bol[kb], acc, 0, 0, 0);
                        fin(acc, row0 + tl * TILE_ROWS + g * 4, tw);
                    }
                }
            };

            // Fast pass: a running (value, row) maximum per lane with plain float compares. A
            // lane meets its rows in increasing order, so a strictly larger value replacing the
            // best keeps the first of equal values (and -0 equals +0), as torch.argmax does.
            // NaN is the one case a float compare cannot order; a lane that meets one (or a
            // false alarm such as inf - inf in its check sum) sends its wave through the exact
            // pass below, which builds the order-preserving key of every value.
            // Four running maxima, one per row of the group, so that the compare-and-select
            // chains are independent; merged afterwards by value, then lowest row. The check sum
            // of all scores is NaN if any score is (or on an inf - inf false alarm). With STAT
            // the stores wait until every slot of a half is scored (stores in between would
            // split the code into blocks the compiler schedules one at a time).
            float run_v[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            uint32_t run_i[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
            float chk = 0.0f;
            RunningSoftmax soft;   // inverse CDF: this lane's pair of request b
            constexpr bool HOLD = STAT && (SAMPLE || OUTL);   // outputs held for a half
            constexpr int HALF_SLOTS = SAMPLE == 1 ? (NT_STAT + 1) / 2 : NT_STAT;
            uint32_t held[HOLD ? HALF_SLOTS : 1][4];
            for_tiles([&](const v4i acc, int vt, int tw) {
                float sc[4];
                uint32_t out[4];
                const bool ok = scores4(acc, vt, sc, out);
                if constexpr (HOLD) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) held[tw % HALF_SLOTS][i] = out[i];
                } else if constexpr (!STAT) {
                    store4(vt, ok, out);
                }
                if constexpr (SAMPLE == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) soft.offer(sc[i], ok);
                } else {
                    chk += ok ? (sc[0] + sc[1]) + (sc[2] + sc[3]) : 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = ok ? sc[i] : -INFINITY;
                        if (x > run_v[i]) {
                            run_v[i] = x;
                            run_i[i] = (uint32_t)(vt + i);
                        }
                    }
                }
            }, [&](int tw) {
                // this wave's share of the next request tile's copy, spread over the slots
                if constexpr (STAT) {
                    if (prefetch) {
                        copy_job(rt + 1, t, nxt, tw * NW + wave);
                        if (tw == NT_STAT - 1) {
#pragma unroll
                            for (int s = NT_STAT; s < STAT_COPY_SLOTS; ++s)
                                copy_job(rt + 1, t, nxt, s * NW + wave);
                        }
                    }
                }
            }, [&](int h0) {
                if constexpr (HOLD) {
                    if (SAMPLE || p.out_logits != nullptr) {
#pragma unroll
                        for (int i = 0; i < HALF_SLOTS; ++i) {
                            const int tw = h0 + i;
                            const int vt = row0 + (tw * NW + wave) * TILE_ROWS + g * 4;
                            if (tw < NT_STAT) store4(vt, vb && vt < vend, held[i]);
                        }
                    }
                }
            });
            if constexpr (SAMPLE == 2) {
                // request c's pair over this wave's rows: the four lanes of the request (row
                // groups g at lanes c + 16 g) merged by two lane exchanges, stored by g = 0
#pragma unroll
                for (int o = 32; o >= 16; o >>= 1)
                    soft.merge(__shfl_xor(soft.m, o, WAVE), __shfl_xor(soft.s, o, WAVE));
                if (g == 0) lkeys[wave * MAX_BS + rt * 16 + c] = pack_softmax(soft.m, soft.s);
                return;
            }
            const bool nan_seen = chk != chk;
            float bv = run_v[0];
            uint32_t bi = run_i[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) {
                // an empty chain has index 0xFFFFFFFF and value -inf: it never wins
                if (run_v[i] > bv || (run_v[i] == bv && run_i[i] < bi)) {
                    bv = run_v[i];
                    bi = run_i[i];
                }
            }
            uint64_t best;
            if (bi != 0xFFFFFFFFu) {
                best = argmax_key(bv, bi);
            } else {
                // every row of this lane was -inf (or it had none): its first row wins
                const int vt0 = row0 + wave * TILE_ROWS + g * 4;
                best = (vb && wave < ntiles && vt0 < vend) ? argmax_key(-INFINITY, (uint32_t)vt0) : 0ull;
            }
            if (__any(nan_seen)) {
                // The exact pass, rare (a NaN score): every tile once more, its W2 rows read
                // from memory (the same codes as the on-chip copies) in a loop that is not
                // unrolled, so that it adds little code.
                best = 0;
#pragma unroll 1
                for (int tw = 0; tw < ntw; ++tw) {
                    const int tl = tw * NW + wave;
                    if (tl >= ntiles) break;
                    v4i acc = {0, 0, 0, 0};
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(load_a(tl, kb), bop[kb], acc, 0, 0, 0);
                    acc = acc << 4;
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(load_a(tl, kb), bol[kb], acc, 0, 0, 0);
                    const int vt = row0 + tl * TILE_ROWS + g * 4;
                    float sc[4];
                    uint32_t out[4];
                    const bool ok = scores4(acc, vt, sc, out);
                    const uint64_t keep = ok ? ~0ull : 0ull;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint64_t k = argmax_key(sc[i], (uint32_t)(vt + i)) & keep;
                        best = k > best ? k : best;
                    }
                }
            }
            // the workgroup's best per request: every lane's key into one LDS word per request
            // by an atomic maximum (keys order as the values they carry; 0 is no row). Merging
            // the four lanes of a request in registers first put a dependent cross-lane chain
            // at the end of every request tile, ~5 us per walk at 64 requests.
            __hip_atomic_fetch_max(&lkeys[rt * 16 + c], best, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            stamp<TIMED>(p, STAMP_TILE0 + (t * STAMP_TILES + rt) * 2 + 1);
        };
        for (int rt = 0; rt < nrt; ++rt) {
            // the buffer each tile reads is named in the code (not picked by an index), so that
            // with STAT the compiler can tell it apart from the one the DMA writes
            if (nbuf == 1 || (rt & 1) == 0)
                request_tile(rt, buf0, buf1);
            else
                request_tile(rt, buf1, buf0);
        }
        __syncthreads();
        stamp<TIMED>(p, STAMP_STEP0 + t * STAMPS_PER_STEP + 1);
        // the first request tile of step t+1 streams in while the combine of step t waits
        if (nbuf && t + 1 < p.T) stage_base_w123(0, t + 1, buf0);

        if (wave == 0) {
            uint64_t k = 0;
            if constexpr (SAMPLE == 2) {
                // request `lane`'s pair over the whole slice: the four waves' merged
                RunningSoftmax a;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const uint64_t o = lkeys[w * MAX_BS + lane];
                    a.merge(packed_m(o), packed_s(o));
                }
                k = lane < p.bs ? pack_softmax(a.m, a.s) : 0ull;
            } else {
                // the workgroup's key of request `lane`, cleared for the next step (whose first
                // update follows the barrier after the combine)
                k = lkeys[lane];
                lkeys[lane] = 0;
                if (lane >= p.bs) k = 0;
            }
            if constexpr (SAMPLE == 2)
                combine_icdf_step<TIMED>(p, t, k, tok, lane);
            else
                combine_step<TIMED>(p, t, k, tok, lane);
        }
        __syncthreads();
    }
}

// OUTL: a greedy kernel with STAT holds its logits for the optional fp32 output (every other
// kernel writes its outputs as before); one without (OUTL = 0) is used when none is asked for
template <int STAT, int OUTL, int NT, int NW>
static const void* mfma_kernel_for(int sample, int w1t, bool timed) {
#define DSPARK_MFMA(S, W, TI) \
    reinterpret_cast<const void*>(&dense_walk_mfma_kernel<S, W, TI, STAT, (S ? 1 : OUTL), NT, NW>)
    if (sample == 2) {   // inverse CDF (no instrumented build)
        switch (w1t) {
            case DT_F32: return DSPARK_MFMA(2, DT_F32, 0);
            case DT_BF16: return DSPARK_MFMA(2, DT_BF16, 0);
            default: return DSPARK_MFMA(2, DT_F16, 0);
        }
    }
    if (timed) return sample ? DSPARK_MFMA(1, DT_BF16, 1) : DSPARK_MFMA(0, DT_BF16, 1);
    if (sample) {
        switch (w1t) {
            case DT_F32: return DSPARK_MFMA(1, DT_F32, 0);
            case DT_BF16: return DSPARK_MFMA(1, DT_BF16, 0);
            default: return DSPARK_MFMA(1, DT_F16, 0);
        }
    }
    switch (w1t) {
        case DT_F32: return DSPARK_MFMA(0, DT_F32, 0);
        case DT_BF16: return DSPARK_MFMA(0, DT_BF16, 0);
        default: return DSPARK_MFMA(0, DT_F16, 0);
    }
#undef DSPARK_MFMA
}

template <int NW>
static const void* mfma_static_kernel(int sample, int w1t, bool timed, bool out_logits, int slots) {
    constexpr int F = mfma_static_max_slots(NW), S = mfma_static_small_slots(NW);
    if (slots <= S)
        return out_logits ? mfma_kernel_for<1, 1, S, NW>(sample, w1t, timed)
                          : mfma_kernel_for<1, 0, S, NW>(sample, w1t, timed);
    return out_logits ? mfma_kernel_for<1, 1, F, NW>(sample, w1t, timed)
                      : mfma_kernel_for<1, 0, F, NW>(sample, w1t, timed);
}

const void* mfma_walk_kernel(int sample, int w1t, bool timed, bool static_stage, bool out_logits,
                             int slots, int waves) {
    if (!static_stage) return mfma_kernel_for<0, 1, 10, WALK_WAVES>(sample, w1t, timed);
    return waves == 8 ? mfma_static_kernel<8>(sample, w1t, timed, out_logits, slots)
                      : mfma_static_kernel<WALK_WAVES>(sample, w1t, timed, out_logits, slots);
}

int mfma_fixed_lds_bytes(int rows_per_wg) { return mfma_fixed_lds(rows_per_wg); }

}  // namespace dspark
