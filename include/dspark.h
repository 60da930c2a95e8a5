/*
 * dspark.h - C ABI of the MI355X (gfx950) DSpark Markov draft walk.
 *
 * The operation (vLLM PR #62958, int8 DSpark Markov walk, Overview): for each request the
 * draft block is walked left to right; at step t
 *
 *     logits_t = base_logits[t] + dequant(W2) @ W1[prev],        W1, W2: V x 256
 *
 * then the step takes the first-maximum argmax (greedy) or a Gumbel-max sample, and the
 * chosen token is prev for step t + 1 (prev at t = 0 is the request's start token). W2 is
 * held as int8 with one fp32 scale per row (same page, Overview). Probabilistic drafting
 * stores the bf16 logits it sampled from, and its Gumbel noise comes from Philox4x32-10 with the
 * request's seed as key and its draft position in the counter (same page, Details). Argmax follows torch.argmax: the first NaN
 * wins, else the first maximum (vLLM PR #64476, Claims and Validation). The top-k variant
 * takes the k best base logits once per draft position, biases only those, and scatters them
 * into a row that is -inf elsewhere before the unchanged sampler runs (vLLM PR #49969
 * "[Spec Decode] Add top-k DSpark Markov projection", Purpose).
 *
 * Conventions for every entry point:
 *  - All tensors are row-major and contiguous, in device memory of the current HIP device,
 *    owned by the caller. The library never frees caller memory and keeps no pointer after a
 *    call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream). Walk calls only enqueue work on it
 *    and return; they never wait on the device, so they may be captured into a HIP graph.
 *  - A negative return value is an error from enum dspark_status. Argument errors are found on
 *    the host before any device work: nothing is enqueued and no output is written.
 *  - Supported envelope (PR #62958, Details): rank 256; 1 <= T <= 16 draft steps;
 *    1 <= bs <= 64 requests; 1 <= V <= 270336; W1 and W2 in fp32, bf16 or fp16; base logits in
 *    fp32. Larger inputs are rejected with DSPARK_ERR_UNSUPPORTED.
 *  - Documented preconditions, not checked (checking would need a device sync): start tokens
 *    lie in [0, V); W1 is finite; temperatures are finite and > 0; positions are >= 0.
 *    NaN base logits are allowed in the dense walks and follow torch.argmax.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dspark_status {
    DSPARK_OK = 0,
    DSPARK_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer */
    DSPARK_ERR_UNSUPPORTED = -2,  /* outside the supported envelope */
    DSPARK_ERR_WORKSPACE = -3,    /* workspace missing or smaller than dspark_walk_workspace_bytes */
    DSPARK_ERR_NO_DEVICE = -4,    /* no HIP device, or not a device this library was built for */
    DSPARK_ERR_LAUNCH = -5,       /* a HIP launch or copy failed */
    DSPARK_ERR_NONFINITE = -6,    /* dspark_quantize_w2 met a NaN or infinity in W2 */
    DSPARK_ERR_TIMEOUT = -7       /* a walk's grid-wide wait hit its time bound (see dspark_workspace_status) */
};

enum dspark_dtype { DSPARK_F32 = 0, DSPARK_BF16 = 1, DSPARK_F16 = 2 };

#define DSPARK_RANK 256
#define DSPARK_MAX_STEPS 16
#define DSPARK_MAX_BS 64
#define DSPARK_MAX_V 270336
#define DSPARK_MAX_TOPK 2048

/* Text for a status code. Never NULL; static storage. */
const char* dspark_status_string(int status);

/*
 * Quantise W2 to int8 codes and one fp32 scale per row (PR #62958, Overview). Reading of the
 * unstated recipe: symmetric absmax, per row
 *     s[v] = max_k |W2[v,k]| / 127            (IEEE fp32 division)
 *     q[v,k] = clamp(rint(W2[v,k] / s[v]), -127, 127)   (IEEE division, round half to even)
 * and an all-zero row gets s = 0, q = 0.
 *   w2        [V, rank] in w2_dtype (DSPARK_F32 / BF16 / F16), 16-byte aligned
 *   w2_q      [V, rank] int8 out, 16-byte aligned
 *   w2_scale  [V] fp32 out
 * Load-time call: it synchronises `stream` once to learn whether W2 held a NaN or infinity,
 * and then returns DSPARK_ERR_NONFINITE with w2_q / w2_scale unspecified. Calls that overlap
 * on one device must not run concurrently (they share the device-side flag).
 */
int dspark_quantize_w2(const void* w2, int w2_dtype, int64_t V, int64_t rank, int8_t* w2_q,
                       float* w2_scale, void* stream);

/*
 * Bytes of workspace a walk call needs (k = 0 for the dense walks, else the top-k k).
 * The caller allocates it on the device and zeroes it ONCE; every walk call leaves it zeroed
 * again, so repeated calls need no memset. A workspace must not be used by two calls that can
 * run at the same time.
 */
size_t dspark_walk_workspace_bytes(int64_t bs, int64_t T, int64_t V, int64_t k);

/* How the dense walk will split W2 over the current device (for reports and tests). */
typedef struct dspark_walk_plan {
    int32_t device_cus;          /* compute units of the current device */
    int32_t num_workgroups;      /* persistent workgroups, at most one per compute unit */
    int32_t rows_per_workgroup;  /* contiguous W2 rows owned by each workgroup (last may own fewer) */
    int32_t rows_in_registers;   /* per workgroup, held in the vector register file for the whole call */
    int32_t rows_in_lds;         /* per workgroup, held in LDS for the whole call */
    int32_t rows_streamed;       /* per workgroup, re-read from memory at every step */
    int64_t resident_bytes;      /* int8 W2 bytes held on chip (whole grid) */
    int64_t streamed_bytes;      /* int8 W2 bytes re-read per step (whole grid) */
    int32_t lds_bytes;           /* dynamic LDS per workgroup */
    int32_t path;                /* DSPARK_PATH_DOT4, DSPARK_PATH_MFMA or DSPARK_PATH_MFMA1 */
    int32_t reg_units;           /* register row sets (dot4) or 16-row tiles per wave (MFMA kernels) */
    int32_t lds_units;           /* LDS row sets (dot4) or tiles per wave (MFMA) */
    int32_t total_units;         /* all row sets / tiles per wave (the rest are streamed) */
    int32_t stage_bufs;          /* MFMA: LDS buffers staging a 16-request tile's base logits */
    int32_t stage_stride;        /* MFMA: floats per request row in such a buffer */
    int32_t waves_per_workgroup; /* 4 (one per SIMD), or 8 for the MFMA kernel with static LDS */
} dspark_walk_plan;

/* Which kernel runs a dense walk: a few requests are GEMVs, more make every step a GEMM (int8
 * matrix cores, 16 requests per tile: DSPARK_PATH_MFMA, from 3 requests greedy and 4 sampling).
 * One request runs on the matrix cores too when each workgroup's slice is at most 1152 rows
 * (every supported V on a 256-CU device), with the two digits of its W1 codes in the two halves
 * of the 16 columns (DSPARK_PATH_MFMA1); otherwise, and for 2 (greedy) or 2-3 (sampling) requests, the
 * lane-per-row v_dot4 kernel runs (DSPARK_PATH_DOT4).
 * The plan queries below report the greedy walk's plan. */
enum dspark_path { DSPARK_PATH_DOT4 = 1, DSPARK_PATH_MFMA = 2, DSPARK_PATH_MFMA1 = 3 };

int dspark_walk_plan_query(int64_t bs, int64_t T, int64_t V, dspark_walk_plan* plan);

/* The same plan for a hypothetical gfx950 device with `cus` compute units and `max_lds` bytes of
 * LDS per workgroup. Pure host logic (no HIP call); for tests and capacity planning. */
int dspark_walk_plan_for(int32_t cus, int64_t max_lds, int64_t bs, int64_t T, int64_t V,
                         dspark_walk_plan* plan);

/*
 * Greedy walk (PR #62958, Overview and Validation: greedy drafting, first-maximum argmax).
 *   w2_q [V, 256] int8 and w2_scale [V] fp32 from dspark_quantize_w2 (w2_q 16-byte aligned)
 *   w1 [V, 256] in w1_dtype, 16-byte aligned
 *   base_logits [bs, T, V] fp32, 16-byte aligned
 *   start_tokens [bs] int32: prev at step 0
 *   draft_tokens [bs, T] int32 out
 *   out_logits [bs, T, V] fp32 out, or NULL: the logits the argmax ran on
 *   workspace of dspark_walk_workspace_bytes(bs, T, V, 0) bytes, zeroed once at allocation
 * Numerics: the bias is (s[v] * s1) * sum_k q[v,k] * C[k], where the gathered W1 row is coded
 * per step as C = rint(W1[prev] * 2032 / absmax), integers in [-2032, 2032] with step
 * s1 = absmax / 2032 (each element within s1 / 2 of W1), held as two int8 digits
 * C = 16 hi + lo; the sum is exact in int32 and every kernel computes the same one. Logits are
 * fp32.
 */
int dspark_walk_greedy(const int8_t* w2_q, const float* w2_scale, const void* w1, int w1_dtype,
                       const float* base_logits, const int32_t* start_tokens, int64_t bs,
                       int64_t T, int64_t V, int64_t rank, int32_t* draft_tokens,
                       float* out_logits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The greedy walk without a caller workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation. It
 * computes exactly what dspark_walk_greedy computes (same kernels, same bits) and allocates
 * nothing: its workspace is a library-held device array of 2,232,320 bytes, sized for the
 * largest walk (bs 64, T 16), one copy per GPU, held until the process ends. Arguments as
 * dspark_walk_greedy, without workspace and workspace_bytes, plus
 *   error_word: a device uint32 the caller zeroes, where a walk records an error as
 *       -dspark_status (DSPARK_ERR_TIMEOUT, or DSPARK_ERR_INVALID_ARG for a start token outside
 *       [0, V)); or NULL, where such errors are not reported.
 * Each call first clears the part of the array it uses (a fill kernel on `stream`), then walks.
 * All calls on one GPU share its array: calls that overlap on one GPU (other streams, other
 * threads) race and must not be made. Shapes beyond the array's size cannot occur within the
 * supported envelope; they would return DSPARK_ERR_UNSUPPORTED.
 */
int dspark_walk_greedy_noalloc(const int8_t* w2_q, const float* w2_scale, const void* w1,
                               int w1_dtype, const float* base_logits,
                               const int32_t* start_tokens, int64_t bs, int64_t T, int64_t V,
                               int64_t rank, int32_t* draft_tokens, float* out_logits,
                               uint32_t* error_word, void* stream);

/*
 * Probabilistic walk (PR #62958, Details; PR #64476, Claims).
 * Arguments as dspark_walk_greedy, plus
 *   seeds [bs] uint64: per-request Philox key (lo32, hi32)
 *   positions [bs] int64 or NULL: draft-position offset; step t uses P = positions[b] + t
 *   temperature [bs] fp32 (> 0)
 *   draft_logits [bs, T, V] bf16 bits out (required, 16-byte aligned): lb = bf16(logits), the
 *       row the sample is drawn from
 * Sample: x = Philox4x32-10(counter (v >> 2, lo32 P, hi32 P, 0), key seed)[v & 3],
 * u = (2 (x >> 9) + 1) 2^-24, g = -log(-log u), token = argmax_v (lb[v] / temperature + g)
 * with torch.argmax order. The quotient is taken as lb[v] * (1 / temperature) with the
 * reciprocal rounded once (within one fp32 ulp of lb[v] / temperature; exact at 1.0).
 */
int dspark_walk_sample(const int8_t* w2_q, const float* w2_scale, const void* w1, int w1_dtype,
                       const float* base_logits, const int32_t* start_tokens, int64_t bs,
                       int64_t T, int64_t V, int64_t rank, const uint64_t* seeds,
                       const int64_t* positions, const float* temperature,
                       int32_t* draft_tokens, uint16_t* draft_logits, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Probabilistic walk drawing each token by inverse CDF instead of Gumbel-max (vLLM PR #62958
 * and #64476, Details, name a PR that fuses the Markov sampling loop by inverse CDF; the pages
 * give no further detail). Arguments and outputs as dspark_walk_sample: the same bf16 row lb is
 * stored in draft_logits, and the token is drawn from softmax(lb / temperature) by inverting its
 * CDF in vocabulary order with one uniform per (request, step): the first index whose running
 * mass exceeds u times the total, u = (2 (x >> 9) + 1) 2^-24 with x word 0 of Philox4x32-10 at
 * counter (0, lo32 P, hi32 P, 1), key the request's seed, P = positions[b] + t (the Gumbel
 * noise uses counters whose last word is 0). Base logits must hold no NaN or +inf, and each
 * step a finite logit. One request runs on the one-request matrix-core kernel, more on the
 * lane-per-row kernel. Each step takes three grid-wide exchanges: the slices' softmax pairs to
 * one reducer per request, its choice of slice to every workgroup, the chosen slice's token
 * to every workgroup.
 */
int dspark_walk_sample_icdf(const int8_t* w2_q, const float* w2_scale, const void* w1,
                            int w1_dtype, const float* base_logits, const int32_t* start_tokens,
                            int64_t bs, int64_t T, int64_t V, int64_t rank,
                            const uint64_t* seeds, const int64_t* positions,
                            const float* temperature, int32_t* draft_tokens,
                            uint16_t* draft_logits, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Top-k walk (PR #49969, Purpose). For each (request, step) the k largest base logits are the
 * candidates (at equal values the lower index ranks first); the Markov bias is evaluated for
 * candidates only; every other entry of the row is -inf; then greedy (sample = 0) or Gumbel
 * (sample = 1, arguments as dspark_walk_sample) runs on the dense row, with noise keyed by the
 * vocabulary index.
 *   draft_logits: sample = 1: bf16 [bs, T, V] (required); sample = 0: fp32 [bs, T, V] or NULL
 *   1 <= k <= min(V, DSPARK_MAX_TOPK); base logits must not hold NaN (result undefined)
 * With k <= 512, V % 4 == 0 (16-byte aligned base rows) and more (request, step) rows than the
 * device has compute units, the select and the walk run in one launch: each request's walk
 * starts once its first row is selected and waits (bounded in time, as the dense walks' waits)
 * for the rows of later steps. Otherwise two launches: every row's select, then the walks. Both
 * forms give the same results.
 */
int dspark_walk_topk(const int8_t* w2_q, const float* w2_scale, const void* w1, int w1_dtype,
                     const float* base_logits, const int32_t* start_tokens, int64_t bs,
                     int64_t T, int64_t V, int64_t rank, int64_t k, int sample,
                     const uint64_t* seeds, const int64_t* positions, const float* temperature,
                     int32_t* draft_tokens, void* draft_logits, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Lossless top-k pruning of W2 for the greedy walk (vLLM PR #62958, Details, names a PR that
 * prunes W2 with top-k without loss; the pages give no algorithm). Reading: at each step only the
 * W2 rows of the k largest base logits are multiplied (the candidates of dspark_walk_topk), and
 * the step keeps their argmax only if no other row can reach it: every other row v has
 * base[v] <= kth, the smallest candidate base logit, and |bias(v)| <= B * max_k |W1[prev,k]|,
 * so the step is certified when the best candidate logit exceeds kth + B * max|W1[prev]| (with a
 * relative margin of 2^-16 for rounding). A step that is not certified is computed over the whole
 * vocabulary. The tokens are therefore those of dspark_walk_greedy on the same inputs.
 *
 * dspark_w2_prune_bound (load time, after dspark_quantize_w2): *bound = B =
 *   max_v fl32(w2_scale[v] * sum_k |w2_q[v,k]|), into a device fp32 word. Enqueues two kernels.
 *
 * dspark_walk_greedy_pruned: arguments as dspark_walk_greedy, plus
 *   k           candidates per step, 1 <= k <= min(V, DSPARK_MAX_TOPK)
 *   w2_bound    device fp32 word holding B for these w2_q / w2_scale
 *   out_logits  [bs, T, V] fp32 or NULL: the logits of the rows each step evaluated (the
 *               candidates, or every row of a step that was not certified), -inf elsewhere
 *   dense_steps [bs] int32 or NULL: per request, the number of steps computed over every row
 *   workspace of dspark_walk_workspace_bytes(bs, T, V, k) bytes (as dspark_walk_topk)
 * Base logits must not hold NaN (as dspark_walk_topk). It runs on the top-k walk's kernels, in
 * one launch or two under the same conditions as dspark_walk_topk.
 */
int dspark_w2_prune_bound(const int8_t* w2_q, const float* w2_scale, int64_t V, int64_t rank,
                          float* bound, void* stream);

int dspark_walk_greedy_pruned(const int8_t* w2_q, const float* w2_scale, const void* w1,
                              int w1_dtype, const float* base_logits,
                              const int32_t* start_tokens, int64_t bs, int64_t T, int64_t V,
                              int64_t rank, int64_t k, const float* w2_bound,
                              int32_t* draft_tokens, float* out_logits, int32_t* dense_steps,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Verification of drafted blocks against the target model, on the stored bf16 draft rows
 * (vLLM PR #62958, Details: rejection sampling works on exactly the distribution the draft
 * sampled from; vLLM PR #64476, Validation: block verification keeps the target distribution).
 * The pages give no algorithm; the two modes are published ones:
 *   DSPARK_VERIFY_TOKEN: speculative sampling (Leviathan, Kalman, Matias, ICML 2023,
 *     Algorithm 1): draft token t is kept while uniforms[b, t] <= min(1, p_t(x_t) / q_t(x_t));
 *     the first rejected step is replaced by a draw from the normalised max(p_t - q_t, 0).
 *   DSPARK_VERIFY_BLOCK: block verification (Sun et al., "Block Verification Accelerates
 *     Speculative Decoding", ICLR 2025, Algorithm 2): weights w_0 = 1,
 *     w_t = min(w_{t-1} p_{t-1}(x_{t-1}) / q_{t-1}(x_{t-1}), 1); h_t = R_t / (R_t + 1 - w_t)
 *     with R_t = sum_x max(w_t p_t(x) - q_t(x), 0) for t < T, h_T = w_T; the kept length is
 *     the largest t with uniforms[b, t - 1] <= h_t (0 if none), and the next token is drawn
 *     from max(w_tau p_tau - q_tau, 0).
 * With every draft token kept, the next token is drawn from p_T. q_t = softmax(draft row t /
 * temperature[b]) and p_t = softmax(target row t / temperature[b]). The next token is the
 * inverse-CDF draw with u = uniforms[b, T]: the first vocabulary index whose running mass
 * exceeds u times the distribution's total (a total of 0, reachable only through rounding,
 * falls back to p_tau).
 *   draft_logits  [bs, T, V] bf16 bits (dspark_walk_sample / dspark_walk_topk output)
 *   draft_tokens  [bs, T] int32
 *   target_logits [bs, T + 1, V] fp32: row t scores position t of the block, row T the one after
 *   temperature   [bs] fp32, finite and > 0 (the draft's and the target's)
 *   uniforms      [bs, T + 1] fp32 in (0, 1): the caller's random draws
 *   accepted      [bs] int32 out: kept length tau in 0..T
 *   out_tokens    [bs, T + 1] int32 out: the kept draft tokens, the next token, then -1
 *   accept_prob   [bs, T] fp32 out or NULL: min(1, p_t/q_t) (token) or h_{t+1} (block)
 *   workspace of dspark_verify_workspace_bytes(bs, T, V) bytes, zeroed once (left zeroed; it may
 *     be the walk's workspace if large enough for both)
 * Preconditions (not checked): every row holds a finite entry and no NaN or +inf; tokens lie in
 * [0, V) (others are read as 0 and recorded as DSPARK_ERR_INVALID_ARG in the workspace's error
 * word). Same envelope as the walks: bs <= 64, T <= 16, V <= 270336.
 */
enum dspark_verify_mode { DSPARK_VERIFY_TOKEN = 0, DSPARK_VERIFY_BLOCK = 1 };

size_t dspark_verify_workspace_bytes(int64_t bs, int64_t T, int64_t V);

int dspark_verify(const uint16_t* draft_logits, const int32_t* draft_tokens,
                  const float* target_logits, const float* temperature, const float* uniforms,
                  int64_t bs, int64_t T, int64_t V, int mode, int32_t* accepted,
                  int32_t* out_tokens, float* accept_prob, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Error word of a walk workspace: synchronises `stream`, returns DSPARK_OK or the error the
 * last walk recorded, and clears it. Diagnostic call, not for hot loops.
 *   DSPARK_ERR_TIMEOUT: a grid-wide wait ran past its time bound (10 ms by default): the walk's
 *       workgroups were not all resident at once, e.g. other work held compute units. The tokens
 *       of that call are invalid, and the workspace must be zeroed again before the next call
 *       (a workgroup that arrived late may have left keys in it). Callers that share the GPU
 *       with other work should check this after their walks.
 *   DSPARK_ERR_INVALID_ARG: a start token was outside [0, V) (it was replaced by 0).
 */
int dspark_workspace_status(void* workspace, void* stream);

/*
 * Test hook: out[i] = the Philox noise word the sampler uses for vocabulary entry v0 + i at
 * draft position `position` of a request with this seed (see dspark_walk_sample), i < n.
 */
int dspark_philox_words(uint64_t seed, uint64_t position, int64_t v0, int64_t n, uint32_t* out,
                        void* stream);

/*
 * Test hooks (process-wide, not thread-safe):
 *   DSPARK_DEBUG_MAX_WORKGROUPS: cap the dense walk's grid (0 = one per compute unit);
 *   DSPARK_DEBUG_SPIN_LIMIT: bound of each grid-wide wait (and of the one-launch top-k walk's
 *       waits for its rows), in ticks of the 100 MHz device clock, before DSPARK_ERR_TIMEOUT is
 *       recorded (0 = the default, 10 ms; at most 2^32 - 1);
 *   DSPARK_DEBUG_WAIT_UNSET_FLAG: non-zero makes those waits also wait for a workspace flag
 *       that nothing sets, so each runs into its time bound (for the timeout tests);
 *   DSPARK_DEBUG_FORCE_PATH: 0 chooses by batch size; DSPARK_PATH_DOT4 / DSPARK_PATH_MFMA force
 *       that kernel for every batch size, DSPARK_PATH_MFMA1 for one request whose slices fit it
 *       (all compute the same results);
 *   DSPARK_DEBUG_STAMPS: a device address (8-byte aligned) of 256 x 210 uint64 words, or 0.
 *       When set, dense walks with bf16 W1 run an instrumented build of the same kernel that
 *       stores the 100 MHz device clock per workgroup: [0] start, [1] W2 resident, then per step
 *       t at 2 + 5t: W1 codes ready, slice argmax done, own slot stored, reductions done,
 *       result words seen; the multi-request MFMA kernel also, per step t and 16-request tile
 *       r, at 82 + 2 (4t + r): the tile's base logits landed, the tile done. Top-k walks with bf16 W1 (k <= 512, V % 4 == 0) use words
 *       row * 8 + (0 start, 1 first bound, 2 row scanned, 3 k-th key, 4 done) for each
 *       (request, step) row of the candidate select, and 8192 + request * 40 + (0 start, then
 *       per step t: 1 + 2t W1 codes ready, 2 + 2t token known) for the walk. For profiling only;
 *   DSPARK_DEBUG_KERNEL_TIMING: n in 1..4096 launches every later walk and verification kernel
 *       on the current device with hipExtLaunchKernel and one of a ring of n HIP event pairs,
 *       which the dispatch records at the kernel's start and end (read them with
 *       dspark_kernel_times); 0 frees the ring. For benchmarks; not around graph capture;
 *   DSPARK_DEBUG_MFMA_WAVES: 0 = the library's choice; 4 or 8 forces the waves per workgroup of
 *       the multi-request MFMA kernel for slices of at most 624 rows (the same results);
 *   DSPARK_DEBUG_TOPK_SPLIT: non-zero runs top-k walks in two launches also where one would
 *       serve (the same results).
 */
enum dspark_debug_key {
    DSPARK_DEBUG_MAX_WORKGROUPS = 1,
    DSPARK_DEBUG_SPIN_LIMIT = 2,
    DSPARK_DEBUG_WAIT_UNSET_FLAG = 3,
    DSPARK_DEBUG_STAMPS = 4,
    DSPARK_DEBUG_FORCE_PATH = 5,
    DSPARK_DEBUG_KERNEL_TIMING = 6,
    DSPARK_DEBUG_MFMA_WAVES = 7,
    DSPARK_DEBUG_TOPK_SPLIT = 8
};
int dspark_debug_set(int key, int64_t value);

/* Durations in microseconds of the kernels launched while DSPARK_DEBUG_KERNEL_TIMING was on,
 * since it was switched on or last read: at most the ring size and `max` of the most recent,
 * oldest first, into `us`; their number into *count. Blocks until those kernels have finished.
 * Returns DSPARK_ERR_INVALID_ARG for null pointers or max < 0, DSPARK_ERR_LAUNCH if an event
 * query fails; with timing off, *count = 0. */
int dspark_kernel_times(float* us, int max, int* count);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
