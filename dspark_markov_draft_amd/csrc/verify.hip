// Verification of a drafted block against the target model's logits, on the stored bf16 draft
// distribution (vLLM PR #62958, Details: rejection sampling works on exactly the bf16 rows the
// draft sampled from; vLLM PR #64476, Validation: block verification keeps the target
// distribution). Two published verifiers:
//   token (Leviathan, Kalman, Matias, ICML 2023, Algorithm 1): keep draft token i while
//     u_i <= min(1, p_i(x_i) / q_i(x_i)); the first rejected step draws from max(p_i - q_i, 0);
//   block (Sun et al., "Block Verification Accelerates Speculative Decoding", ICLR 2025,
//     Algorithm 2): w_0 = 1, w_i = min(w_{i-1} p_{i-1}(x_{i-1}) / q_{i-1}(x_{i-1}), 1),
//     h_i = R_i / (R_i + 1 - w_i) with R_i = sum_x max(w_i p_i(x) - q_i(x), 0) (i < T),
//     h_T = w_T; the kept length tau is the largest i with u_{i-1} <= h_i; the next token is
//     drawn from p_T (tau = T) or from max(w_tau p_tau - q_tau, 0).
// q_t = softmax(bf16 draft row t / temp), p_t = softmax(target row t / temp), t = 0..T. The
// next token is the inverse-CDF draw with uniforms[b, T]: the first index whose running mass
// exceeds u * (total mass).
//
// Every pass streams rows from HBM in chunks of CH consecutive vocabulary entries, one chunk per
// workgroup, so a launch has bs * rows * V / CH workgroups (thousands at the pages' shapes).
// Thread i of a chunk handles entries (j * 256 + i) * 4 .. +3 for j < CH / 1024: a float4 of the
// target row and four bf16 of the draft row, each wave instruction reading 4 KB / 2 KB of
// consecutive memory. Per-request decisions run in small kernels between the passes:
//   1. stats:    per (row, chunk): max and sum of 2^(z - max) of z = logit * log2(e) / temp,
//                for the target row and the draft row;
//   2. decide:   per request: combine the chunks, the ratios p_t(x_t) / q_t(x_t) at the drafted
//                tokens, the weights w_t; in token mode the kept length;
//   3. residual: (block mode) per (row i in 1..T-1, chunk): sum of max(w_i p_i - q_i, 0);
//   4. choose:   (block mode) per request: h_i and the kept length;
//   5. mass:     per (chunk): mass of the next token's distribution r on row tau;
//   6. draw:     per request: the chunk where the running mass crosses u * total, an in-order
//                scan of that chunk, the outputs; the request's workspace words are cleared.
#include "internal.hpp"
#include "device_common.hpp"

namespace dspark {

namespace {

constexpr int VT = 256;                  // threads per workgroup
constexpr int VWAVES = VT / WAVE;
constexpr float LOG2E_F = 1.44269504088896340736f;

// Per-request state in the workspace.
struct VerifyState {
    float mp[MAX_STEPS + 1], sp[MAX_STEPS + 1];   // target rows: max z and sum 2^(z - max)
    float mq[MAX_STEPS], sq[MAX_STEPS];           // draft rows
    float w[MAX_STEPS + 1];                       // weights w_0..w_T (all 1 in token mode)
    float prob[MAX_STEPS];                        // acceptance probability of each step
    int tau;                                      // kept length
};
static_assert(sizeof(VerifyState) <= VERIFY_STATE_BYTES, "state fits its slot");

struct VerifyParams {
    const uint16_t* draft;     // [bs, T, V] bf16 bits
    const int32_t* tokens;     // [bs, T]
    const float* target;       // [bs, T + 1, V]
    const float* temps;        // [bs]
    const float* uniforms;     // [bs, T + 1]
    int32_t* accepted;         // [bs]
    int32_t* out_tokens;       // [bs, T + 1]
    float* accept_prob;        // [bs, T] or null
    uint32_t* err;
    VerifyState* state;        // [bs]
    float4* stats;             // [bs][T + 1][C]: (mp, sp, mq, sq) per chunk
    float* resid;              // [bs][T][C]
    float2* mass;              // [bs][CM]: (mass of r, mass of p_tau) per chunk of MASS_J * 1024
    int bs, T, V, mode, C, CM;
};

// The next token's pass (masses per chunk, then the draw's in-order scan of one chunk) uses
// chunks of MASS_J * 1024 entries: more workgroups for the one row per request it reads, and a
// short scan. Up to MASS_MAX_CHUNKS chunks per row.
constexpr int MASS_J = 2;
constexpr int MASS_GROUPS = 4;                       // the draw's selection: chunks per lane
constexpr int MASS_MAX_CHUNKS = MASS_GROUPS * WAVE;
static_assert((int64_t)MASS_MAX_CHUNKS * MASS_J * 1024 >= DSPARK_MAX_V, "chunks of the largest V");

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// 2^x by the hardware instruction alone (exp2f adds a range reduction that keeps results
// below 2^-126 as denormals; this flushes them to 0). Used only for terms that are added to a
// sum that holds the maximum's own term 1, or compared with terms of their own size, where
// such values change nothing; the per-entry masses that decide which tokens can be drawn use
// exp2f.
__device__ __forceinline__ float exp2_sum_term(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) pairs: s = sum of 2^(z - m) over the entries seen, m their maximum (-inf, 0: none).
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) {
        m = M;
        s = 0.0f;
        return;
    }
    s = s * exp2f(m - M) + s2 * exp2f(m2 - M);
    m = M;
}

__device__ __forceinline__ void wave_ms(float& m, float& s) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, WAVE);
        const float s2 = __shfl_xor(s, o, WAVE);
        ms_merge(m, s, m2, s2);
    }
}

// Block-wide (m, s) and sums: wave results through LDS, combined by every thread in wave order.
__device__ __forceinline__ void block_ms(float& m, float& s, float* lds) {
    wave_ms(m, s);
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    __syncthreads();
    if (lane == 0) {
        lds[2 * wave] = m;
        lds[2 * wave + 1] = s;
    }
    __syncthreads();
    m = lds[0];
    s = lds[1];
#pragma unroll
    for (int w = 1; w < VWAVES; ++w) ms_merge(m, s, lds[2 * w], lds[2 * w + 1]);
}

__device__ __forceinline__ float block_sum(float v, float* lds) {
    v = wave_sum(v);
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    __syncthreads();
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    float t = lds[0];
#pragma unroll
    for (int w = 1; w < VWAVES; ++w) t += lds[w];
    return t;
}

// Four entries x0 .. x0+3 of a target row (fp32) and of a draft row (bf16), -inf past V.
template <int VEC>
__device__ __forceinline__ void load_entries(const float* trow, const uint16_t* drow, int64_t x0,
                                             int V, float (&zp)[4], float (&zq)[4]) {
    if (VEC && x0 + 3 < V) {
        const float4 a = *reinterpret_cast<const float4*>(trow + x0);
        zp[0] = a.x; zp[1] = a.y; zp[2] = a.z; zp[3] = a.w;
        if (drow) {
            const uint2 d = *reinterpret_cast<const uint2*>(drow + x0);
            zq[0] = bf16_lo(d.x); zq[1] = bf16_hi(d.x); zq[2] = bf16_lo(d.y); zq[3] = bf16_hi(d.y);
        } else {
            zq[0] = zq[1] = zq[2] = zq[3] = -INFINITY;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bool in = x0 + k < V;
        zp[k] = in ? trow[x0 + k] : -INFINITY;
        zq[k] = (in && drow) ? bf16_value(drow[x0 + k]) : -INFINITY;
    }
}

// The J groups of four entries a thread reads from a chunk (group j at x0 + 4 (j VT + thread)).
// A chunk wholly inside the row takes the vector loads with no per-group branch, so that all of
// them are in flight together; a per-group choice between vector and element loads made the
// compiled code wait for each group's loads before issuing the next.
template <int J, int VEC>
__device__ __forceinline__ void load_chunk(const float* trow, const uint16_t* drow, int64_t base,
                                           int V, float (&zp)[J][4], float (&zq)[J][4]) {
    if (VEC && base + (int64_t)J * VT * 4 <= V) {
        float4 a[J];
        uint2 d[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t x0 = base + (int64_t)(j * VT + threadIdx.x) * 4;
            a[j] = *reinterpret_cast<const float4*>(trow + x0);
            if (drow) d[j] = *reinterpret_cast<const uint2*>(drow + x0);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            zp[j][0] = a[j].x; zp[j][1] = a[j].y; zp[j][2] = a[j].z; zp[j][3] = a[j].w;
            if (drow) {
                zq[j][0] = bf16_lo(d[j].x); zq[j][1] = bf16_hi(d[j].x);
                zq[j][2] = bf16_lo(d[j].y); zq[j][3] = bf16_hi(d[j].y);
            } else {
                zq[j][0] = zq[j][1] = zq[j][2] = zq[j][3] = -INFINITY;
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
        load_entries<VEC>(trow, drow, base + (int64_t)(j * VT + threadIdx.x) * 4, V, zp[j], zq[j]);
}

// ---- 1. row statistics ------------------------------------------------------------------
template <int J, int VEC>
__global__ __launch_bounds__(VT) void verify_stats_kernel(const VerifyParams p) {
    __shared__ float lds[2 * VWAVES];
    const int c = blockIdx.x, row = blockIdx.y;
    const int b = row / (p.T + 1), t = row - b * (p.T + 1);
    const float k = LOG2E_F / p.temps[b];
    const float* trow = p.target + (int64_t)row * p.V;
    const uint16_t* drow = t < p.T ? p.draft + ((int64_t)b * p.T + t) * p.V : nullptr;
    const int64_t base = (int64_t)c * (J * VT * 4);
    float zp[J][4], zq[J][4];
    load_chunk<J, VEC>(trow, drow, base, p.V, zp, zq);
    float mp = -INFINITY, mq = -INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            zp[j][e] *= k;
            zq[j][e] *= k;
            mp = fmaxf(mp, zp[j][e]);
            mq = fmaxf(mq, zq[j][e]);
        }
    // (a row part with no finite entry subtracts 0: its -inf entries give exactly 0)
    const float mpc = mp == -INFINITY ? 0.0f : mp, mqc = mq == -INFINITY ? 0.0f : mq;
    float sp = 0.0f, sq = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sp += exp2_sum_term(zp[j][e] - mpc);
            sq += exp2_sum_term(zq[j][e] - mqc);
        }
    block_ms(mp, sp, lds);
    block_ms(mq, sq, lds);
    if (threadIdx.x == 0) p.stats[(int64_t)row * p.C + c] = make_float4(mp, sp, mq, sq);
}

// probability of entry z (already scaled) in a row with statistics (m, s)
__device__ __forceinline__ float prob_of(float z, float m, float inv_s) {
    return exp2f(z - m) * inv_s;
}

// ---- 2. per-request decisions after the statistics -----------------------------------------
__global__ __launch_bounds__(VT) void verify_decide_kernel(const VerifyParams p) {
    __shared__ float ms[MAX_STEPS + 1][4];
    __shared__ float ratio[MAX_STEPS];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    // combine each row's chunks: wave w takes rows w, w + 4, ...
    for (int t = wave; t <= p.T; t += VWAVES) {
        const float4* st = p.stats + ((int64_t)b * (p.T + 1) + t) * p.C;
        float mp = -INFINITY, sp = 0.0f, mq = -INFINITY, sq = 0.0f;
        for (int c = lane; c < p.C; c += WAVE) {
            const float4 v = st[c];
            ms_merge(mp, sp, v.x, v.y);
            ms_merge(mq, sq, v.z, v.w);
        }
        wave_ms(mp, sp);
        wave_ms(mq, sq);
        if (lane == 0) {
            ms[t][0] = mp; ms[t][1] = sp; ms[t][2] = mq; ms[t][3] = sq;
        }
    }
    __syncthreads();
    const float k = LOG2E_F / p.temps[b];
    // the drafted token's probabilities, one thread per step
    if ((int)threadIdx.x < p.T) {
        const int t = threadIdx.x;
        int x = p.tokens[b * p.T + t];
        if (x < 0 || x >= p.V) {
            __hip_atomic_store(p.err, (uint32_t)(-DSPARK_ERR_INVALID_ARG), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            x = 0;
        }
        const float zp = p.target[((int64_t)b * (p.T + 1) + t) * p.V + x] * k;
        const float zq = bf16_value(p.draft[((int64_t)b * p.T + t) * p.V + x]) * k;
        const float pp = prob_of(zp, ms[t][0], 1.0f / ms[t][1]);
        const float qq = prob_of(zq, ms[t][2], 1.0f / ms[t][3]);
        ratio[t] = qq > 0.0f ? pp / qq : (pp > 0.0f ? INFINITY : 0.0f);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        VerifyState& s = p.state[b];
        for (int t = 0; t <= p.T; ++t) {
            s.mp[t] = ms[t][0];
            s.sp[t] = ms[t][1];
            if (t < p.T) {
                s.mq[t] = ms[t][2];
                s.sq[t] = ms[t][3];
            }
        }
        const float* u = p.uniforms + (int64_t)b * (p.T + 1);
        if (p.mode == 0) {
            int tau = p.T;
            for (int t = 0; t < p.T; ++t) {
                const float a = fminf(ratio[t], 1.0f);
                s.prob[t] = a;
                if (tau == p.T && !(u[t] <= a)) tau = t;
            }
            for (int t = 0; t <= p.T; ++t) s.w[t] = 1.0f;
            s.tau = tau;
        } else {
            float w = 1.0f;
            s.w[0] = w;
            for (int t = 1; t <= p.T; ++t) {
                w = w > 0.0f ? fminf(w * ratio[t - 1], 1.0f) : 0.0f;
                s.w[t] = w;
            }
        }
    }
}

// ---- 3. block mode: residual sums R_i, rows 1..T-1 ----------------------------------------
template <int J, int VEC>
__global__ __launch_bounds__(VT) void verify_residual_kernel(const VerifyParams p) {
    __shared__ float lds[VWAVES];
    const int c = blockIdx.x, row = blockIdx.y;
    const int b = row / (p.T - 1), i = 1 + row - b * (p.T - 1);
    const VerifyState& s = p.state[b];
    const float k = LOG2E_F / p.temps[b];
    const float mp = s.mp[i], ip = 1.0f / s.sp[i], mq = s.mq[i], iq = 1.0f / s.sq[i], w = s.w[i];
    const float* trow = p.target + ((int64_t)b * (p.T + 1) + i) * p.V;
    const uint16_t* drow = p.draft + ((int64_t)b * p.T + i) * p.V;
    const int64_t base = (int64_t)c * (J * VT * 4);
    float zp[J][4], zq[J][4];
    load_chunk<J, VEC>(trow, drow, base, p.V, zp, zq);
    float R = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d = w * (exp2_sum_term(zp[j][e] * k - mp) * ip) -
                            exp2_sum_term(zq[j][e] * k - mq) * iq;
            R += d > 0.0f ? d : 0.0f;
        }
    R = block_sum(R, lds);
    if (threadIdx.x == 0) p.resid[((int64_t)b * p.T + i) * p.C + c] = R;
}

// ---- 4. block mode: h_i and the kept length ------------------------------------------------
__global__ __launch_bounds__(VT) void verify_choose_kernel(const VerifyParams p) {
    __shared__ float R[MAX_STEPS];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    for (int i = 1 + wave; i < p.T; i += VWAVES) {
        const float* r = p.resid + ((int64_t)b * p.T + i) * p.C;
        float v = 0.0f;
        for (int c = lane; c < p.C; c += WAVE) v += r[c];
        v = wave_sum(v);
        if (lane == 0) R[i] = v;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        VerifyState& s = p.state[b];
        const float* u = p.uniforms + (int64_t)b * (p.T + 1);
        int tau = 0;
        for (int i = 1; i <= p.T; ++i) {
            float h;
            if (i < p.T) {
                const float den = R[i] + 1.0f - s.w[i];
                h = den > 0.0f ? R[i] / den : 1.0f;
            } else {
                h = s.w[p.T];
            }
            s.prob[i - 1] = h;
            if (u[i - 1] <= h) tau = i;
        }
        s.tau = tau;
    }
}

// r(x) of the next token's distribution on row tau: p_T (tau = T), else max(w p - q, 0)
struct NextDist {
    float mp, ip, mq, iq, w, k;
    bool last;
    __device__ __forceinline__ void at(float xp, float xq, float& r, float& pr) const {
        pr = prob_of(xp * k, mp, ip);
        if (last) {
            r = pr;
        } else {
            const float d = w * pr - prob_of(xq * k, mq, iq);
            r = d > 0.0f ? d : 0.0f;
        }
    }
};

__device__ __forceinline__ NextDist next_dist(const VerifyParams& p, int b) {
    const VerifyState& s = p.state[b];
    const int tau = s.tau;
    NextDist d;
    d.last = tau == p.T;
    d.k = LOG2E_F / p.temps[b];
    d.mp = s.mp[tau];
    d.ip = 1.0f / s.sp[tau];
    d.mq = d.last ? 0.0f : s.mq[tau];
    d.iq = d.last ? 0.0f : 1.0f / s.sq[tau];
    d.w = s.w[tau];
    return d;
}

// ---- 5. mass of the next token's distribution per chunk ------------------------------------
template <int J, int VEC>
__global__ __launch_bounds__(VT) void verify_mass_kernel(const VerifyParams p) {
    __shared__ float lds[VWAVES];
    const int c = blockIdx.x, b = blockIdx.y;
    const NextDist d = next_dist(p, b);
    const int tau = p.state[b].tau;
    const float* trow = p.target + ((int64_t)b * (p.T + 1) + tau) * p.V;
    const uint16_t* drow = d.last ? nullptr : p.draft + ((int64_t)b * p.T + tau) * p.V;
    const int64_t base = (int64_t)c * (J * VT * 4);
    float zp[J][4], zq[J][4];
    load_chunk<J, VEC>(trow, drow, base, p.V, zp, zq);
    float mr = 0.0f, mpt = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float r, pr;
            d.at(zp[j][e], zq[j][e], r, pr);
            mr += r;
            mpt += pr;
        }
    mr = block_sum(mr, lds);
    mpt = block_sum(mpt, lds);
    if (threadIdx.x == 0) p.mass[(int64_t)b * p.CM + c] = make_float2(mr, mpt);
}

// ---- 6. the draw, the outputs, and the request's workspace words cleared -------------------
template <int J, int VEC>
__global__ __launch_bounds__(VT) void verify_draw_kernel(const VerifyParams p) {
    __shared__ float part[VWAVES];
    __shared__ int found;
    __shared__ int chunk_sel;
    __shared__ float local_target;
    __shared__ int use_p;
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
    const VerifyState& s = p.state[b];
    const int tau = s.tau;
    const NextDist d = next_dist(p, b);
    const float2* mass = p.mass + (int64_t)b * p.CM;
    if (wave == 0) {
        // total mass (r; p_tau if r has none), then the first chunk with mass where the running
        // mass passes u * total: wave 0, chunk g * 64 + lane in lane `lane` of group g, running
        // masses by a scan of each group over the lanes, in chunk order
        float mr[MASS_GROUPS], mpt[MASS_GROUPS];
        float tr = 0.0f, tp = 0.0f;
#pragma unroll
        for (int g = 0; g < MASS_GROUPS; ++g) {
            const int c = g * WAVE + lane;
            const float2 v = c < p.CM ? mass[c] : make_float2(0.0f, 0.0f);
            mr[g] = v.x;
            mpt[g] = v.y;
            tr += v.x;
            tp += v.y;
        }
        float tot = wave_sum(tr);
        const int up = tot > 0.0f ? 0 : 1;
        if (up) tot = wave_sum(tp);
        const float target = p.uniforms[(int64_t)b * (p.T + 1) + p.T] * tot;
        float mg[MASS_GROUPS];   // the masses in use, chosen value by value (no array select)
#pragma unroll
        for (int g = 0; g < MASS_GROUPS; ++g) mg[g] = up ? mpt[g] : mr[g];
        float run = 0.0f;          // mass of the groups before
        int sel = -1, last = 0;
        float before = 0.0f, before_last = 0.0f;
        auto group = [&](int g, float m) {
            float incl = m;
#pragma unroll
            for (int o = 1; o < WAVE; o <<= 1) {
                const float v = __shfl_up(incl, o, WAVE);
                if (lane >= o) incl += v;
            }
            const float excl = run + (incl - m);   // running mass before this lane's chunk
            const uint64_t cross = __ballot(m > 0.0f && excl + m > target);
            if (sel < 0 && cross != 0) {
                const int f = __builtin_ctzll(cross);
                sel = g * WAVE + f;
                before = __shfl(excl, f, WAVE);
            }
            const uint64_t has = __ballot(m > 0.0f);
            if (has != 0) {
                const int l = 63 - __builtin_clzll(has);
                last = g * WAVE + l;
                before_last = __shfl(excl, l, WAVE);
            }
            run += __shfl(incl, WAVE - 1, WAVE);
        };
        static_assert(MASS_GROUPS == 4, "groups");
        group(0, mg[0]);
        group(1, mg[1]);
        group(2, mg[2]);
        group(3, mg[3]);
        if (sel < 0) {   // rounding: the running mass never passed the target
            sel = last;
            before = before_last;
        }
        if (lane == 0) {
            chunk_sel = sel;
            local_target = target - before;
            use_p = up;
            found = 0x7FFFFFFF;
        }
    }
    __syncthreads();
    const int c = chunk_sel;
    const float lt = local_target;
    const bool up = use_p != 0;
    const float* trow = p.target + ((int64_t)b * (p.T + 1) + tau) * p.V;
    const uint16_t* drow = d.last ? nullptr : p.draft + ((int64_t)b * p.T + tau) * p.V;
    const int64_t base = (int64_t)c * (J * VT * 4);
    // in-order scan of the chunk: group j covers entries base + j * 1024 .. +1023, thread i
    // its four entries (j * 256 + i) * 4 .. +3
    float run = 0.0f;
    int last_pos = -1;   // last entry of the chunk with mass (fallback)
    for (int j = 0; j < J; ++j) {
        const int64_t x0 = base + (int64_t)(j * VT + threadIdx.x) * 4;
        float zp[4], zq[4];
        load_entries<VEC>(trow, drow, x0, p.V, zp, zq);
        float r[4];
        float mine = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float rr, pr;
            d.at(zp[e], zq[e], rr, pr);
            r[e] = up ? pr : rr;
            if (r[e] > 0.0f) last_pos = (int)(x0 + e);
            mine += r[e];
        }
        // exclusive prefix of `mine` over the workgroup (wave scan, then the waves in order)
        float incl = mine;
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const float v = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += v;
        }
        __syncthreads();
        if (lane == WAVE - 1) part[wave] = incl;
        __syncthreads();
        float before = run;
        float total = 0.0f;
#pragma unroll
        for (int w = 0; w < VWAVES; ++w) {
            if (w < wave) before += part[w];
            total += part[w];
        }
        before += incl - mine;
        float cum = before;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            cum += r[e];
            if (r[e] > 0.0f && cum > lt) {
                atomicMin(&found, (int)(x0 + e));
                break;
            }
        }
        run += total;
        __syncthreads();
        if (found != 0x7FFFFFFF) break;
    }
    // rounding: if nothing passed the target inside the chunk (the scan then covered all of
    // it), the draw is the chunk's last entry with mass
    __shared__ int last_sel;
    if (threadIdx.x == 0) last_sel = -1;
    __syncthreads();
    if (found == 0x7FFFFFFF && last_pos >= 0) atomicMax(&last_sel, last_pos);
    __syncthreads();
    if (threadIdx.x == 0) {
        int y = found != 0x7FFFFFFF ? found : last_sel;
        if (y < 0 || y >= p.V) y = 0;
        p.accepted[b] = tau;
        for (int i = 0; i <= p.T; ++i) {
            int o = -1;
            if (i < tau) {
                o = p.tokens[b * p.T + i];
                if (o < 0 || o >= p.V) o = 0;
            } else if (i == tau) {
                o = y;
            }
            p.out_tokens[b * (p.T + 1) + i] = o;
        }
        if (p.accept_prob)
            for (int i = 0; i < p.T; ++i) p.accept_prob[b * p.T + i] = s.prob[i];
    }
    __syncthreads();
    // clear this request's workspace words (the next call, or a walk on the same workspace,
    // finds them zero)
    {
        float4* st = p.stats + (int64_t)b * (p.T + 1) * p.C;
        for (int i = threadIdx.x; i < (p.T + 1) * p.C; i += VT) st[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        float* rs = p.resid + (int64_t)b * p.T * p.C;
        for (int i = threadIdx.x; i < p.T * p.C; i += VT) rs[i] = 0.0f;
        float2* ms = p.mass + (int64_t)b * p.CM;
        for (int i = threadIdx.x; i < p.CM; i += VT) ms[i] = make_float2(0.f, 0.f);
        uint32_t* sw = reinterpret_cast<uint32_t*>(&p.state[b]);
        for (int i = threadIdx.x; i < (int)(VERIFY_STATE_BYTES / 4); i += VT) sw[i] = 0u;
    }
}

// chunk of CH = J * 1024 entries: the largest of 8192 / 4096 / 2048 whose statistics pass
// still has at least 2048 workgroups, so small batches spread over the whole chip
int verify_groups(int bs, int T, int V) {
    const int64_t rows = (int64_t)bs * (T + 1);
    for (int J = 8; J > 2; J /= 2)
        if (rows * ((V + J * 1024 - 1) / (J * 1024)) >= 2048) return J;
    return 2;
}

template <int J, int VEC>
int launch_verify_j(const VerifyParams& p_in, hipStream_t s) {
    VerifyParams p = p_in;
    void* args[] = {&p};
    const dim3 blk(VT);
    auto go = [&](const void* fn, dim3 grid) {
        return launch_walk_kernel(fn, grid, blk, args, 0, s) == hipSuccess;
    };
    bool ok = go(reinterpret_cast<const void*>(&verify_stats_kernel<J, VEC>),
                 dim3(p.C, p.bs * (p.T + 1)));
    ok = ok && go(reinterpret_cast<const void*>(&verify_decide_kernel), dim3(p.bs));
    if (p.mode == 1 && p.T > 1)
        ok = ok && go(reinterpret_cast<const void*>(&verify_residual_kernel<J, VEC>),
                      dim3(p.C, p.bs * (p.T - 1)));
    if (p.mode == 1) ok = ok && go(reinterpret_cast<const void*>(&verify_choose_kernel), dim3(p.bs));
    ok = ok && go(reinterpret_cast<const void*>(&verify_mass_kernel<MASS_J, VEC>), dim3(p.CM, p.bs));
    ok = ok && go(reinterpret_cast<const void*>(&verify_draw_kernel<MASS_J, VEC>), dim3(p.bs));
    if (!ok) {
        (void)hipGetLastError();
        return DSPARK_ERR_LAUNCH;
    }
    return DSPARK_OK;
}

}  // namespace

static size_t up16(size_t n) { return (n + 15) / 16 * 16; }

// workspace regions after the error word: states [bs], chunk statistics [bs][T + 1][C] (float4),
// residual sums [bs][T][C], next-token masses [bs][CM] (float2), each 16-byte aligned
struct VerifyLayout {
    size_t state, stats, resid, mass, end;
    VerifyLayout(int64_t bs, int64_t T, int64_t C, int64_t CM) {
        state = VERIFY_WS_STATE;
        stats = state + (size_t)bs * VERIFY_STATE_BYTES;
        resid = stats + up16((size_t)bs * (T + 1) * C * 16);
        mass = resid + up16((size_t)bs * T * C * 4);
        end = mass + up16((size_t)bs * CM * 8);
    }
};

size_t verify_workspace_bytes(int64_t bs, int64_t T, int64_t V) {
    const int64_t most = (V + 2047) / 2048;   // the smallest chunk: the most chunks
    const VerifyLayout L(bs, T, most, most);
    return (L.end + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN;
}

int launch_verify(const VerifyLaunch& a, hipStream_t stream) {
    VerifyParams p;
    p.draft = a.draft_logits;
    p.tokens = a.draft_tokens;
    p.target = a.target_logits;
    p.temps = a.temperature;
    p.uniforms = a.uniforms;
    p.accepted = a.accepted;
    p.out_tokens = a.out_tokens;
    p.accept_prob = a.accept_prob;
    p.bs = a.bs;
    p.T = a.T;
    p.V = a.V;
    p.mode = a.mode;
    const int J = verify_groups(a.bs, a.T, a.V);
    p.C = (a.V + J * 1024 - 1) / (J * 1024);
    p.CM = (a.V + MASS_J * 1024 - 1) / (MASS_J * 1024);
    if (p.CM > MASS_MAX_CHUNKS) return DSPARK_ERR_UNSUPPORTED;
    char* ws = static_cast<char*>(a.workspace);
    const VerifyLayout L(a.bs, a.T, p.C, p.CM);
    p.err = reinterpret_cast<uint32_t*>(ws + WS_ERR);
    p.state = reinterpret_cast<VerifyState*>(ws + L.state);
    p.stats = reinterpret_cast<float4*>(ws + L.stats);
    p.resid = reinterpret_cast<float*>(ws + L.resid);
    p.mass = reinterpret_cast<float2*>(ws + L.mass);
    const bool vec = (a.V % 4 == 0) && ((uintptr_t)a.target_logits % 16 == 0) &&
                     ((uintptr_t)a.draft_logits % 8 == 0);
    switch (J * 2 + (vec ? 1 : 0)) {
        case 17: return launch_verify_j<8, 1>(p, stream);
        case 16: return launch_verify_j<8, 0>(p, stream);
        case 9: return launch_verify_j<4, 1>(p, stream);
        case 8: return launch_verify_j<4, 0>(p, stream);
        case 5: return launch_verify_j<2, 1>(p, stream);
        default: return launch_verify_j<2, 0>(p, stream);
    }
}

}  // namespace dspark
