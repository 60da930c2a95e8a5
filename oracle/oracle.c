/*
 * Plain CPU oracle for the DSpark Markov draft walk.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library. The HIP library never calls it, and the two share no
 * code: no kernels, headers, helpers or tables.
 *
 * What is computed, and where the pages say so:
 *  - vLLM PR #62958 (int8 DSpark Markov walk), Overview: the draft block is walked left to
 *    right; each step adds W2 @ W1[prev] to that step's base logits (W2 is V x 256), then takes
 *    the argmax or a sample, and the chosen token is the next step's prev. W2 is stored as int8
 *    with one fp32 scale per row.
 *  - PR #62958, Details: probabilistic drafting stores the bf16 logits it sampled from in
 *    draft_logits; its Gumbel noise words are Philox outputs whose key is the request's seed and
 *    whose counter holds the draft position.
 *    The rank is 256.
 *  - vLLM PR #64476 (Markov bias in the Gumbel kernel), Claims: the combine follows
 *    torch.argmax (the first NaN wins, otherwise the first maximum); the temperature divide is
 *    skipped at 1.0, which changes no bit.
 *  - vLLM PR #49969 "[Spec Decode] Add top-k DSpark Markov projection", Purpose: the top-k
 *    candidates are taken from the base logits once per draft position, the bias is evaluated
 *    only for them, the results are scattered into a dense row that is -inf elsewhere, and the
 *    unchanged greedy or Gumbel sampler runs on that row.
 *  - Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 *    SC'11, Figure 2 / Section 3.3 (the Philox S-box, key schedule and round count).
 *
 * Readings taken where the pages are silent (each is also noted at its function):
 *  - quantisation is symmetric absmax: s = absmax / 127 in fp32, q = rint(w / s) clamped to
 *    [-127, 127]; an all-zero row has s = 0, q = 0; non-finite W2 is an error;
 *  - the bias is the exact dequantised product s[v] * q[v,k] times W1[prev,k], summed in fp64;
 *    the logit is base + bias rounded once to fp32, and every argmax decision is taken on fp32;
 *  - sampling: lb = bf16(l) (round to nearest even), score = lb / temp + g with
 *    g = -log(-log(u)), u = (2 * (x >> 9) + 1) * 2^-24 and x the Philox word for
 *    counter (v >> 2, lo32(P), hi32(P), 0), key (lo32(seed), hi32(seed)), word v & 3,
 *    P = position offset + step; the score is rounded once to fp32;
 *  - top-k: the k largest base logits, ties at the boundary broken toward the lower index.
 *
 * Floating point: every float -> double conversion is exact; dot products accumulate in fp64
 * in index order. Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NONFINITE (-6)

/* ---------------------------------------------------------------------------------------- */
/* Quantisation (PR #62958, Overview: int8 W2 with one fp32 scale per row).                  */
/* Reading: symmetric absmax, s = absmax/127 in IEEE fp32, q = rint(w/s) (half to even) in    */
/* [-127, 127]. Zero row: s = 0, q = 0. Any non-finite element: error (PR #62958, Details:    */
/* inputs the kernel does not handle are rejected with an explicit error, not computed).     */
/* ---------------------------------------------------------------------------------------- */
int oracle_quantize_w2(const float* w2, int64_t V, int64_t R, int8_t* q, float* s) {
    if (!w2 || !q || !s || V < 0 || R <= 0) return ORACLE_ERR_ARG;
    for (int64_t v = 0; v < V; ++v) {
        const float* row = w2 + v * R;
        float amax = 0.0f;
        for (int64_t k = 0; k < R; ++k) {
            if (!isfinite(row[k])) return ORACLE_ERR_NONFINITE;
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            s[v] = 0.0f;
            for (int64_t k = 0; k < R; ++k) q[v * R + k] = 0;
            continue;
        }
        float sv = amax / 127.0f;
        s[v] = sv;
        for (int64_t k = 0; k < R; ++k) {
            float r = rintf(row[k] / sv);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[v * R + k] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------------------- */
/* Philox4x32-10 (Salmon et al., SC'11): ten rounds of the 4x32 Philox S-box with the Weyl     */
/* key schedule. One round maps (c0, c1, c2, c3) under key (k0, k1) to                        */
/*   (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)),                        */
/* and the key is bumped by (W0, W1) between rounds.                                          */
/* ---------------------------------------------------------------------------------------- */
static const uint32_t PHILOX_M0 = 0xD2511F53u;
static const uint32_t PHILOX_M1 = 0xCD9E8D57u;
static const uint32_t PHILOX_W0 = 0x9E3779B9u;
static const uint32_t PHILOX_W1 = 0xBB67AE85u;

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The noise word for vocabulary entry v of draft position P of a request with this seed    */
/* (PR #62958, Details: Philox with the request seed and draft position as inputs).         */
/* Reading: counter (v >> 2, lo32(P), hi32(P), 0), key (lo32(seed), hi32(seed)), word v & 3. */
uint32_t oracle_noise_word(uint64_t seed, uint64_t P, int64_t v) {
    uint32_t ctr[4] = {(uint32_t)((uint64_t)v >> 2), (uint32_t)P, (uint32_t)(P >> 32), 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[v & 3];
}

/* Reading: u = (2 * (x >> 9) + 1) / 2^24, the midpoint of one of 2^23 equal cells of (0, 1);  */
/* exact in fp32 and never 0 or 1.                                                            */
double oracle_uniform(uint32_t x) {
    return (2.0 * (double)(x >> 9) + 1.0) / 16777216.0;
}

/* Standard Gumbel variate by inversion of its CDF exp(-exp(-g)): g = -log(-log(u)), in fp64. */
double oracle_gumbel(uint32_t x) {
    double u = oracle_uniform(x);
    return -log(-log(u));
}

/* ---------------------------------------------------------------------------------------- */
/* bf16 with round to nearest, ties to even (PR #62958, Details: draft_logits are bf16).       */
/* NaN stays NaN (quiet), overflow goes to +-inf.                                            */
/* ---------------------------------------------------------------------------------------- */
uint16_t oracle_bf16_rne(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    uint32_t r = u + 0x7FFFu + lsb;
    return (uint16_t)(r >> 16);
}

float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------------------------------------------------------------------------------------- */
/* torch.argmax order (PR #64476, Claims and Validation: the first NaN wins, otherwise the     */
/* first maximum). -0.0 and +0.0 compare equal, as they do under C's ==.                      */
/* ---------------------------------------------------------------------------------------- */
int64_t oracle_argmax_f32(const float* x, int64_t n) {
    if (n <= 0) return -1;
    for (int64_t i = 0; i < n; ++i)
        if (isnan(x[i])) return i;
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i)
        if (x[i] > x[best]) best = i;
    return best;
}

/* ---------------------------------------------------------------------------------------- */
/* Top-k candidates (PR #49969, Purpose: select the top-k candidates from the base logits once */
/* for all draft positions). Reading: the k largest values; at equal values the lower index   */
/* ranks first. Output order: (value descending, index ascending). NaN input is an error.     */
/* ---------------------------------------------------------------------------------------- */
typedef struct {
    float val;
    int32_t idx;
} oracle_vi;

static int oracle_cmp_vi(const void* a, const void* b) {
    const oracle_vi* x = (const oracle_vi*)a;
    const oracle_vi* y = (const oracle_vi*)b;
    if (x->val > y->val) return -1;
    if (x->val < y->val) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx) ? 1 : 0;
}

int oracle_topk(const float* row, int64_t V, int64_t k, int32_t* cand) {
    if (!row || !cand || k < 1 || k > V) return ORACLE_ERR_ARG;
    oracle_vi* tmp = (oracle_vi*)malloc((size_t)V * sizeof(oracle_vi));
    if (!tmp) return ORACLE_ERR_ARG;
    for (int64_t v = 0; v < V; ++v) {
        if (isnan(row[v])) {
            free(tmp);
            return ORACLE_ERR_ARG;
        }
        tmp[v].val = row[v] == 0.0f ? 0.0f : row[v]; /* -0 ranks with +0 */
        tmp[v].idx = (int32_t)v;
    }
    qsort(tmp, (size_t)V, sizeof(oracle_vi), oracle_cmp_vi);
    for (int64_t i = 0; i < k; ++i) cand[i] = tmp[i].idx;
    free(tmp);
    return ORACLE_OK;
}

double oracle_icdf_uniform(uint64_t seed, uint64_t P);
int64_t oracle_icdf_draw(const uint16_t* lb, int64_t V, float temp, double u);

/* ---------------------------------------------------------------------------------------- */
/* One draft step of one request (PR #62958, Overview; PR #64476, Claims; PR #49969, Purpose). */
/*   l[v] = fp32( base[v] + sum_k s[v] * q[v,k] * W1[prev,k] )   for every v (dense), or for    */
/*          v in cand with l = -inf elsewhere (top-k);                                         */
/*   greedy:  token = argmax(l);                                                             */
/*   sample:  lb = bf16(l); score = fp32(lb / temp + g(v)) (no divide at temp 1.0);           */
/*            token = argmax(score).                                                          */
/*   sample == 2 (inverse CDF): lb = bf16(l); token = oracle_icdf_draw(lb, temp, u(seed, P));  */
/*            score receives float(lb).                                                        */
/* logits receives l (fp32, dense). lb and score, if given, receive the bf16 row and the      */
/* scores. Returns the token, or a negative status.                                           */
/* ---------------------------------------------------------------------------------------- */
int64_t oracle_step(const int8_t* q, const float* s, const float* w1, int64_t V, int64_t R,
                    const float* base_row, int64_t prev, const int32_t* cand, int64_t k,
                    int sample, uint64_t seed, uint64_t P, float temp, float* logits,
                    uint16_t* lb, float* score) {
    if (!q || !s || !w1 || !base_row || !logits || V <= 0 || R <= 0) return ORACLE_ERR_ARG;
    if (prev < 0 || prev >= V) return ORACLE_ERR_ARG;
    if (sample && (!lb || !score)) return ORACLE_ERR_ARG;
    const float* w = w1 + prev * R;

    if (cand) {
        for (int64_t v = 0; v < V; ++v) logits[v] = -INFINITY;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < k; ++i) {
            int64_t v = cand[i];
            double bias = 0.0;
            for (int64_t j = 0; j < R; ++j)
                bias += (double)s[v] * (double)q[v * R + j] * (double)w[j];
            logits[v] = (float)((double)base_row[v] + bias);
        }
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t v = 0; v < V; ++v) {
            double bias = 0.0;
            for (int64_t j = 0; j < R; ++j)
                bias += (double)s[v] * (double)q[v * R + j] * (double)w[j];
            logits[v] = (float)((double)base_row[v] + bias);
        }
    }

    if (!sample) return oracle_argmax_f32(logits, V);
    if (sample == 2) {
        /* inverse-CDF sampling: the stored row, then one draw (see oracle_icdf_draw) */
        for (int64_t v = 0; v < V; ++v) {
            lb[v] = oracle_bf16_rne(logits[v]);
            score[v] = oracle_bf16_to_f32(lb[v]);
        }
        return oracle_icdf_draw(lb, V, temp, oracle_icdf_uniform(seed, P));
    }

#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < V; ++v) {
        uint16_t h = oracle_bf16_rne(logits[v]);
        lb[v] = h;
        double x = (double)oracle_bf16_to_f32(h);
        if (temp != 1.0f) x = x / (double)temp;
        double g = oracle_gumbel(oracle_noise_word(seed, P, v));
        score[v] = (float)(x + g);
    }
    return oracle_argmax_f32(score, V);
}

/* ---------------------------------------------------------------------------------------- */
/* The whole walk for bs requests over T steps: the token chosen at step t is prev at t+1,     */
/* start_tokens[b] is prev at t = 0 (PR #62958, Overview). k = 0: full vocabulary; k > 0:     */
/* top-k candidates of base[b,t,:] (PR #49969, Purpose). positions may be NULL (offset 0).    */
/* logits / lb may be NULL; when given they are [bs, T, V].                                   */
/* ---------------------------------------------------------------------------------------- */
int oracle_walk(const int8_t* q, const float* s, const float* w1, const float* base,
                const int32_t* start, int64_t bs, int64_t T, int64_t V, int64_t R, int64_t k,
                int sample, const uint64_t* seeds, const int64_t* positions, const float* temps,
                int32_t* tokens, float* logits, uint16_t* lb) {
    if (!q || !s || !w1 || !base || !start || !tokens || bs < 1 || T < 1 || V < 1 || R < 1)
        return ORACLE_ERR_ARG;
    if (k < 0 || k > V) return ORACLE_ERR_ARG;
    if (sample && (!seeds || !temps)) return ORACLE_ERR_ARG;

    float* l_row = (float*)malloc((size_t)V * sizeof(float));
    uint16_t* lb_row = (uint16_t*)malloc((size_t)V * sizeof(uint16_t));
    float* sc_row = (float*)malloc((size_t)V * sizeof(float));
    int32_t* cand = k > 0 ? (int32_t*)malloc((size_t)k * sizeof(int32_t)) : NULL;
    int status = ORACLE_OK;
    if (!l_row || !lb_row || !sc_row || (k > 0 && !cand)) status = ORACLE_ERR_ARG;

    for (int64_t b = 0; b < bs && status == ORACLE_OK; ++b) {
        int64_t prev = start[b];
        for (int64_t t = 0; t < T; ++t) {
            const float* base_row = base + (b * T + t) * V;
            if (k > 0) {
                status = oracle_topk(base_row, V, k, cand);
                if (status != ORACLE_OK) break;
            }
            uint64_t P = (uint64_t)(positions ? positions[b] : 0) + (uint64_t)t;
            int64_t tok = oracle_step(q, s, w1, V, R, base_row, prev, k > 0 ? cand : NULL, k,
                                      sample, sample ? seeds[b] : 0, P,
                                      sample ? temps[b] : 1.0f, l_row, lb_row, sc_row);
            if (tok < 0) {
                status = (int)tok;
                break;
            }
            tokens[b * T + t] = (int32_t)tok;
            if (logits) memcpy(logits + (b * T + t) * V, l_row, (size_t)V * sizeof(float));
            if (lb && sample) memcpy(lb + (b * T + t) * V, lb_row, (size_t)V * sizeof(uint16_t));
            prev = tok;
        }
    }
    free(l_row);
    free(lb_row);
    free(sc_row);
    free(cand);
    return status;
}

/* Threads the vocabulary loops may use (OpenMP); 1 when built without OpenMP. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ======================================================================================== */
/* Verification of a drafted block against the target model's logits.                      */
/*                                                                                          */
/* The pages: probabilistic drafting stores the bf16 logits it sampled from in draft_logits  */
/* so that rejection sampling works on exactly that distribution (vLLM PR #62958, Details),  */
/* and block verification keeps the target distribution across draft steps (vLLM PR #64476, */
/* Validation). They give neither algorithm; these are the published ones:                   */
/*  - mode 0, token verification: speculative sampling, Leviathan, Kalman, Matias, "Fast      */
/*    Inference from Transformers via Speculative Decoding", ICML 2023, Algorithm 1 (and      */
/*    Chen et al., "Accelerating Large Language Model Decoding with Speculative Sampling",    */
/*    2023, Algorithm 2): draft token i is kept with probability min(1, p_i(x_i) / q_i(x_i)) */
/*    until the first rejection, which is replaced by a draw from the normalised             */
/*    max(p_i - q_i, 0); if every draft token is kept, one more token is drawn from p_T.     */
/*  - mode 1, block verification: Sun, Mendlovic, Leviathan, Aharoni, Beirami, Ro, Suresh,   */
/*    "Block Verification Accelerates Speculative Decoding", ICLR 2025, Algorithm 2: with    */
/*    weights w_0 = 1, w_i = min(w_{i-1} p_{i-1}(x_{i-1}) / q_{i-1}(x_{i-1}), 1), and        */
/*    h_i = R_i / (R_i + 1 - w_i), R_i = sum_x max(w_i p_i(x) - q_i(x), 0) for i < T,         */
/*    h_T = w_T, the kept length is the largest i with eta_i <= h_i (0 if none); the next     */
/*    token is drawn from p_T if all T are kept, else from the normalised                    */
/*    max(w_tau p_tau - q_tau, 0).                                                           */
/* Rows (0-based): q_t = softmax(bf16 draft_logits[b,t] / temp) is the distribution draft    */
/* token t was drawn from (the walk's Gumbel-max over the stored bf16 row samples exactly    */
/* this), p_t = softmax(target_logits[b,t] / temp), t = 0..T (row T scores the position      */
/* after the block).                                                                         */
/* Readings where the pages are silent:                                                      */
/*  - one temperature per request divides both the draft and the target logits;            */
/*  - the random draws are inputs: uniforms[b, i] (i < T) is the acceptance draw of step i   */
/*    (eta_{i+1} in the block paper's 1-based notation), uniforms[b, T] draws the final      */
/*    token by inverting the CDF of its (unnormalised) distribution r in vocabulary order:   */
/*    the first y with r(0) + ... + r(y) > u * sum(r); a draw is kept when u <= its          */
/*    acceptance probability;                                                                */
/*  - ratios with q = 0: p / q is +inf (min gives 1) when p > 0, and 0 when p = 0; a weight  */
/*    of 0 stays 0; h_i = 1 where R_i + 1 - w_i = 0 (then R_i = 0 and w_i = 1, and the       */
/*    algorithm's outputs do not depend on h_i);                                             */
/*  - a final distribution of total mass 0 (a rejection where p_tau <= w q_tau everywhere, */
/*    reachable only through rounding) is replaced by p_tau.                                 */
/* Everything is fp64: z = logit / temp, probabilities exp(z - max z) / sum exp(z - max z).  */
/* ======================================================================================== */
static void oracle_probs_row(const double* z, int64_t V, double* prob) {
    double m = -INFINITY;
    for (int64_t x = 0; x < V; ++x)
        if (z[x] > m) m = z[x];
    double sum = 0.0;
    for (int64_t x = 0; x < V; ++x) {
        prob[x] = (m == -INFINITY) ? 0.0 : exp(z[x] - m);
        sum += prob[x];
    }
    for (int64_t x = 0; x < V; ++x) prob[x] = sum > 0.0 ? prob[x] / sum : 0.0;
}

/* p / q for the ratio of a drafted token (q = 0: +inf when p > 0, else 0) */
static double oracle_ratio(double p, double q) {
    if (q > 0.0) return p / q;
    return p > 0.0 ? INFINITY : 0.0;
}

/* Index drawn from the unnormalised distribution r by inverse CDF with uniform u. */
static int64_t oracle_inverse_cdf(const double* r, int64_t V, double u) {
    double mass = 0.0;
    for (int64_t x = 0; x < V; ++x) mass += r[x];
    const double target = u * mass;
    double c = 0.0;
    int64_t last = -1;
    for (int64_t x = 0; x < V; ++x) {
        c += r[x];
        if (r[x] > 0.0) last = x;
        if (c > target) return x;
    }
    return last;
}

int oracle_verify(const uint16_t* draft_logits, const int32_t* draft_tokens,
                  const float* target_logits, const float* temps, const float* uniforms,
                  int64_t bs, int64_t T, int64_t V, int mode, int32_t* accepted,
                  int32_t* out_tokens, double* accept_prob) {
    if (!draft_logits || !draft_tokens || !target_logits || !temps || !uniforms || !accepted ||
        !out_tokens || bs < 1 || T < 1 || V < 1 || (mode != 0 && mode != 1))
        return ORACLE_ERR_ARG;
    double* z = (double*)malloc((size_t)V * sizeof(double));
    double* P = (double*)malloc((size_t)(T + 1) * (size_t)V * sizeof(double));
    double* Q = (double*)malloc((size_t)T * (size_t)V * sizeof(double));
    double* r = (double*)malloc((size_t)V * sizeof(double));
    double* w = (double*)malloc((size_t)(T + 1) * sizeof(double));
    double* h = (double*)malloc((size_t)(T + 1) * sizeof(double));
    int status = ORACLE_OK;
    if (!z || !P || !Q || !r || !w || !h) status = ORACLE_ERR_ARG;

    for (int64_t b = 0; b < bs && status == ORACLE_OK; ++b) {
        const double temp = (double)temps[b];
        const int32_t* X = draft_tokens + b * T;
        const float* u = uniforms + b * (T + 1);
        if (!(temp > 0.0) || !isfinite(temp)) { status = ORACLE_ERR_ARG; break; }
        for (int64_t t = 0; t < T; ++t)
            if (X[t] < 0 || X[t] >= V) status = ORACLE_ERR_ARG;
        if (status != ORACLE_OK) break;
        /* the rows' probabilities */
        for (int64_t t = 0; t <= T && status == ORACLE_OK; ++t) {
            const float* row = target_logits + (b * (T + 1) + t) * V;
            for (int64_t x = 0; x < V; ++x) {
                if (isnan(row[x])) status = ORACLE_ERR_ARG;
                z[x] = (double)row[x] / temp;
            }
            oracle_probs_row(z, V, P + t * V);
        }
        for (int64_t t = 0; t < T && status == ORACLE_OK; ++t) {
            const uint16_t* row = draft_logits + (b * T + t) * V;
            for (int64_t x = 0; x < V; ++x) {
                const float f = oracle_bf16_to_f32(row[x]);
                if (isnan(f)) status = ORACLE_ERR_ARG;
                z[x] = (double)f / temp;
            }
            oracle_probs_row(z, V, Q + t * V);
        }
        if (status != ORACLE_OK) break;

        int64_t tau;
        double weight;
        if (mode == 0) {
            /* token verification: keep while u_i <= min(1, p_i(x_i) / q_i(x_i)) */
            tau = T;
            for (int64_t i = 0; i < T; ++i) {
                double a = oracle_ratio(P[i * V + X[i]], Q[i * V + X[i]]);
                if (a > 1.0) a = 1.0;
                h[i + 1] = a;
                if (tau == T && !((double)u[i] <= a)) tau = i;
            }
            weight = 1.0;
        } else {
            /* block verification */
            w[0] = 1.0;
            for (int64_t i = 1; i <= T; ++i) {
                double wi = 0.0;
                if (w[i - 1] > 0.0) {
                    wi = w[i - 1] * oracle_ratio(P[(i - 1) * V + X[i - 1]], Q[(i - 1) * V + X[i - 1]]);
                    if (wi > 1.0) wi = 1.0;
                }
                w[i] = wi;
            }
            for (int64_t i = 1; i <= T; ++i) {
                if (i < T) {
                    double R = 0.0;
                    for (int64_t x = 0; x < V; ++x) {
                        const double d = w[i] * P[i * V + x] - Q[i * V + x];
                        if (d > 0.0) R += d;
                    }
                    const double den = R + 1.0 - w[i];
                    h[i] = den > 0.0 ? R / den : 1.0;
                } else {
                    h[i] = w[T];
                }
            }
            tau = 0;
            for (int64_t i = 1; i <= T; ++i)
                if ((double)u[i - 1] <= h[i]) tau = i;
            weight = w[tau];
        }
        /* the token after the kept prefix */
        const double* Pt = P + tau * V;
        double mass = 0.0;
        for (int64_t x = 0; x < V; ++x) {
            r[x] = (tau == T) ? Pt[x] : weight * Pt[x] - Q[tau * V + x];
            if (r[x] < 0.0) r[x] = 0.0;
            mass += r[x];
        }
        if (!(mass > 0.0))
            for (int64_t x = 0; x < V; ++x) r[x] = Pt[x];
        const int64_t y = oracle_inverse_cdf(r, V, (double)u[T]);

        accepted[b] = (int32_t)tau;
        for (int64_t i = 0; i <= T; ++i)
            out_tokens[b * (T + 1) + i] = i < tau ? X[i] : (i == tau ? (int32_t)y : -1);
        if (accept_prob)
            for (int64_t i = 0; i < T; ++i) accept_prob[b * T + i] = h[i + 1];
    }
    free(z);
    free(P);
    free(Q);
    free(r);
    free(w);
    free(h);
    return status;
}

/* ======================================================================================== */
/* Lossless top-k pruning of W2 for the greedy walk (vLLM PR #62958, Details, names a PR      */
/* that prunes W2 with top-k, losslessly; the pages give no algorithm). Reading: at each step  */
/* only the W2 rows of the k largest base logits are multiplied, and the step is accepted only */
/* if no other row can reach the best candidate's logit; otherwise the step is computed over  */
/* the whole vocabulary. The walk's result is then by definition the dense greedy walk's       */
/* (oracle_walk), which is what its outputs are checked against. The one quantity the pruned  */
/* walk adds is this load-time bound on every row's bias per unit of W1 magnitude:            */
/*     B = max_v fl32( s[v] * fl32(sum_k |q[v,k]|) ),                                         */
/* so that |deq(W2)[v] . w| <= sum_k |s[v] q[v,k]| |w_k| <= B * max_k |w_k| for every row v.   */
/* The integer sum is exact in fp32 (at most 256 * 127); one product is rounded.               */
/* ======================================================================================== */
float oracle_w2_l1_bound(const int8_t* q, const float* s, int64_t V, int64_t R) {
    float best = 0.0f;
    for (int64_t v = 0; v < V; ++v) {
        int32_t l1 = 0;
        for (int64_t k = 0; k < R; ++k) l1 += q[v * R + k] < 0 ? -q[v * R + k] : q[v * R + k];
        const float c = s[v] * (float)l1;
        if (c > best) best = c;
    }
    return best;
}

/* ======================================================================================== */
/* Inverse-CDF sampling inside the walk (vLLM PR #62958 and #64476, Details, name a PR that    */
/* fuses the Markov sampling loop by inverse CDF; the pages give no further detail).          */
/* Reading: the step rounds its logits to bf16 and stores them (as the Gumbel walk does, so    */
/* that verification works on the distribution drawn from), then draws the token from         */
/* softmax(float(lb) / temp) by inverting its CDF in vocabulary order with one uniform per     */
/* (request, step): the first index v whose running mass sum_{x<=v} exp(z_x - m) exceeds      */
/* u * sum_x exp(z_x - m), z = float(lb) / temp, m = max z (fp64). The uniform comes from the  */
/* same generator as the Gumbel noise on a disjoint counter: word 0 of Philox4x32-10 with     */
/* counter (0, lo32(P), hi32(P), 1) and key (lo32(seed), hi32(seed)) (the Gumbel counters     */
/* have 0 in their last word), mapped by oracle_uniform.                                      */
/* ======================================================================================== */
double oracle_icdf_uniform(uint64_t seed, uint64_t P) {
    uint32_t ctr[4] = {0u, (uint32_t)P, (uint32_t)(P >> 32), 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return oracle_uniform(out[0]);
}

/* The inverse-CDF draw from the stored bf16 row lb with uniform u (see above). Rows must hold a */
/* finite entry and no NaN or +inf. Returns the index, or -1 for such a row.                     */
int64_t oracle_icdf_draw(const uint16_t* lb, int64_t V, float temp, double u) {
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        const double z = (double)oracle_bf16_to_f32(lb[v]) / (double)temp;
        if (isnan(z) || z == INFINITY) return -1;
        if (z > m) m = z;
    }
    if (m == -INFINITY) return -1;
    double total = 0.0;
    for (int64_t v = 0; v < V; ++v) total += exp((double)oracle_bf16_to_f32(lb[v]) / (double)temp - m);
    const double target = u * total;
    double c = 0.0;
    int64_t last = -1;
    for (int64_t v = 0; v < V; ++v) {
        const double e = exp((double)oracle_bf16_to_f32(lb[v]) / (double)temp - m);
        c += e;
        if (e > 0.0) last = v;
        if (c > target) return v;
    }
    return last;
}
