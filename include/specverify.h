/*
 * specverify.h -- C ABI of libspecverify: batched verification of drafted
 * tokens in speculative decoding, and D-cut verification-depth allocation,
 * on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (titles as printed):
 *   [Stack]    aimodeling.com, "Tencent Hunyuan Turns Speculative Decoding
 *              Into a Full Open-Source Stack"
 *   [Remio]    remio.ai, "Tencent rilascia AngelSpec in open source, sfidando
 *              lo speculative decoding universale"
 *   [Hamidun]  news.hamidun.com, "Tencent открыл AngelSpec - фреймворк для
 *              ускорения инференса LLM через speculative decoding"
 *   [AIbase]   test-news.aibase.com news item 30001 (AngelSpec release)
 *
 * Problem statement these calls follow: B requests, each with K drafted
 * tokens over a vocabulary of V; the target model has produced logits for
 * every drafted position plus one more ([B, K+1, V]); the target verifies
 * the whole block in one pass by rejection sampling and commits the
 * accepted prefix plus a bonus token ([Stack], section "What problem does
 * it solve"; [Hamidun], section "Qu'est-ce que le speculative decoding").
 * The pages print no accept rule; the calls implement the standard
 * speculative-sampling construction (Leviathan et al. 2023; Chen et al.
 * 2023), the textbook method with the lossless property the pages state.
 *
 * Conventions shared by every call
 *   Pointers.  Every array argument is a DEVICE pointer on the current HIP
 *     device.  Logit arrays must be 16-byte aligned.  Layouts are contiguous
 *     row-major with the vocabulary fastest: target row (b, k) starts at
 *     element (b*(K+1) + k)*V, draft row (b, k) at (b*K + k)*V.
 *   Ownership.  The caller owns every buffer, including the workspace; the
 *     library allocates no device memory and keeps no state between calls.
 *   Execution.  Calls are asynchronous and ordered on `stream`; a call that
 *     returns SV_OK has only enqueued work.  Calls that share a workspace must
 *     be ordered (the same stream, or synchronised): their kernels keep
 *     partial results there.
 *   Workspace.  At least spec_verify_workspace_size(B, K, V) bytes,
 *     256-byte aligned, contents arbitrary: each call writes every part of
 *     it that it later reads, so one workspace can serve calls of any shape
 *     that fits it.  It holds per-call scratch (row partials, sampler
 *     partials, per-request records) and nothing that outlives the call.
 *   Errors.  Arguments the host can check (null pointers, sizes, dtype,
 *     alignment, workspace size, budget) are rejected with a status before
 *     anything is enqueued.  Bad DATA is found on the device and reported per
 *     request as num_accepted[b] = -1 with out_tokens[b, :] = -1: a depth
 *     outside [0, K], a temperature that is neither 0 nor a finite number
 *     above 0 (so NaN, negatives and infinities), a drafted token outside
 *     [0, V), a uniform outside [0, 1), or a row that is read and holds a NaN
 *     or +inf, or only -inf.  -inf logits (masked tokens) are allowed
 *     otherwise.  No C++ exception crosses this interface.
 *   Check mode.  With the environment variable SPECVERIFY_CHECK=1 the verify
 *     calls and dcut_allocate wait for their own work and return
 *     SV_ERR_BAD_INPUT when a request reported bad data (num_accepted[b] or
 *     depth_out[b] = -1; spec_verify_last_error names the first such
 *     request).  A debugging aid: it synchronises the stream, so it is not
 *     for graph capture.
 *   Decomposition override.  SPECVERIFY_CHUNK=n (n > 0) makes the row
 *     statistics pass split every logit row into n chunks (at most one per
 *     4 KiB batch and 256 per row) instead of the count it picks from the
 *     grid.  A test and tuning aid: greedy outputs, dcut depths and sampled
 *     tokens do not depend on it; sampled p/q and the confidence move by
 *     rounding only.
 *   Limits.  1 <= B <= 4096, 0 <= K <= 1024, 1 <= V <= 2000000.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned logits   */
    SV_ERR_UNSUPPORTED = 2,   /* size beyond the limits above                 */
    SV_ERR_WORKSPACE = 3,     /* workspace missing, too small or misaligned   */
    SV_ERR_BUDGET = 4,        /* D-cut budget smaller than the batch          */
    SV_ERR_BAD_INPUT = 5,     /* check mode: a request reported bad data      */
    SV_ERR_HIP = 6            /* a HIP launch or query failed                 */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Version of this interface (incremented on any signature change). */
int32_t spec_verify_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char *spec_verify_status_string(sv_status s);

/* Detail of the last SV_ERR_HIP returned on the calling thread (the HIP
 * error name and the launch that failed), or of a device limit behind an
 * SV_ERR_UNSUPPORTED; "" when the last call on this thread that reached the
 * device succeeded.  Thread-local storage. */
const char *spec_verify_last_error(void);

/* Bytes of workspace spec_verify_greedy, spec_verify_sample,
 * spec_draft_confidence and the calls built on them need for a batch of this
 * shape; 0 for sizes the library rejects. */
size_t spec_verify_workspace_size(int32_t B, int32_t K, int32_t V);

/* Per-kernel timing for benchmarks (instrumentation; changes no result).
 * spec_verify_timing_begin(n) creates 4n HIP events on the current device and
 * arms them for the calling thread: each of its next n calls of
 * spec_verify_greedy, spec_verify_sample or spec_draft_confidence records
 * four of them on its own stream -- before the row-statistics kernel, after
 * it, after the finish kernel and after the draw kernel.
 * spec_verify_timing_end(ms, n) waits for the first n armed calls' events,
 * writes ms[3i + s] = milliseconds of stage s of call i (0 row statistics,
 * 1 finish: merge, accept scan and sampler sums, 2 draw; a stage a call
 * does not launch reads about 0) and releases all events.  n may not exceed
 * the number of calls made since timing_begin (SV_ERR_INVALID_ARG). */
sv_status spec_verify_timing_begin(int32_t n);
sv_status spec_verify_timing_end(float *ms, int32_t n);

/* Read ceiling for benchmarks (instrumentation; computes nothing of the
 * method): one kernel that reads `bytes` bytes of `buf` once, with the load
 * width and cache policy of the row-statistics kernel, the practical
 * bandwidth ceiling that kernel's rate is compared with.  buf: device
 * pointer, 16-byte aligned, bytes a positive multiple of 16; sink: one
 * device uint32 the kernel may write (a fold of the data, kept so the loads
 * are not removed).  Asynchronous on `stream`. */
sv_status spec_verify_read_ceiling(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Greedy (T = 0) verification.
 * For request b with depth d = depth[b] (or K when depth is NULL): drafted
 * token k is accepted iff it equals the argmax of target row (b, k) (values
 * compared as numbers, -0.0 == +0.0, lowest index wins ties); the accepted
 * length n_b counts the drafted tokens accepted before the first mismatch
 * ([Remio], section "Come AngelSpec rende DFly più selettivo"); the emitted
 * token is the argmax of target row (b, n_b): the correction when n_b < d,
 * the bonus token when n_b = d ([Stack], section "What problem does it
 * solve").  Acceptance at T = 0 is what [Hamidun]'s list of numbers reports.
 *   target_logits  [B, K+1, V] of dt          (read: rows 0..d of each request)
 *   draft_tokens   [B, K] int32               (read: 0..d-1)
 *   depth          [B] int32 or NULL
 *   out_tokens     [B, K+1] int32  out: x_0..x_{n-1}, emitted token, then -1
 *   num_accepted   [B] int32       out: n_b, or -1 for bad data */
sv_status spec_verify_greedy(const void *target_logits, sv_dtype dt,
                             const int32_t *draft_tokens, const int32_t *depth,
                             int32_t B, int32_t K, int32_t V,
                             int32_t *out_tokens, int32_t *num_accepted,
                             void *workspace, size_t ws_bytes, hipStream_t stream);

/* Sampled verification by rejection sampling, per-request temperature.
 * For request b with depth d and temperature T = temperature[b]:
 *   T == 0: the greedy rule of spec_verify_greedy.
 *   T  > 0: with p_k = softmax(z_{b,k} / T) and q_k = softmax(y_{b,k} / T)
 *     (T applies to target and draft rows alike), drafted token x = x_{b,k}
 *     is accepted iff u_accept[b,k] < min(1, p_k(x) / q_k(x)) (ratio 1 when
 *     q_k(x) = 0 < p_k(x), 0 when both are 0); n_b = first rejected k, or d.
 *     n_b < d: the emitted token is drawn from max(0, p_n - q_n) (normalised;
 *       p_n itself if that has no mass) by the inverse CDF at u_sample[b];
 *     n_b = d: the bonus token is drawn from p_d the same way.
 *   The inverse CDF takes the first token, in index order, whose inclusive
 *   prefix of the distribution exceeds u_sample[b] times its total.
 *   This keeps the output distributed as the target's ([Hamidun], section
 *   "Qu'est-ce que le speculative decoding"; [Remio], section "Cosa non
 *   dimostrano i numeri di AngelSpec").
 *   draft_logits  [B, K, V] of dt (read: rows 0..d-1 of requests with T > 0)
 *   temperature   [B] float: 0 (greedy rule) or any finite T > 0 (fp32
 *     denormals included)
 *   u_accept      [B, K] float in [0, 1);  u_sample [B] float in [0, 1)
 *   p_draft, q_draft  [B, K] float or NULL  out: p_k(x_k), q_k(x_k) for every
 *     k < d of requests with T > 0; 0 elsewhere.
 *   Other arguments as in spec_verify_greedy.  Target row (b, d) of a request
 *   with T > 0 is read only when nothing is rejected. */
sv_status spec_verify_sample(const void *target_logits, const void *draft_logits,
                             sv_dtype dt, const int32_t *draft_tokens,
                             const int32_t *depth, const float *temperature,
                             const float *u_accept, const float *u_sample,
                             int32_t B, int32_t K, int32_t V,
                             int32_t *out_tokens, int32_t *num_accepted,
                             float *p_draft, float *q_draft,
                             void *workspace, size_t ws_bytes, hipStream_t stream);

/* Packed (CSR) layout of the two verify calls.  D-cut gives every request
 * its own verification depth ([Stack], section "What problem does it
 * solve", inference layer; [Remio], section "Come AngelSpec rende DFly più
 * selettivo"), so a serving engine holds logits only for the positions it
 * verifies: request b's drafted positions are o_b .. o_{b+1} - 1 of one flat
 * array, o = draft_offsets, and its depth is d_b = o_{b+1} - o_b.  Same
 * rules, outputs and kernels as spec_verify_greedy / spec_verify_sample
 * with depth[b] = d_b; only the addresses differ:
 *   target_logits  [n_draft_rows + B, V]: target row k of request b at
 *                  o_b + b + k, k = 0..d_b (d_b + 1 rows per request)
 *   draft_logits   [n_draft_rows, V]: draft row k of request b at o_b + k
 *   draft_tokens, u_accept, p_draft, q_draft  [n_draft_rows]: slot o_b + k
 *   out_tokens     [n_draft_rows + B] int32: slot o_b + b + k, k = 0..d_b
 *   draft_offsets  [B + 1] int32 device array (read on the device)
 *   temperature, u_sample, num_accepted  [B] as in the padded calls
 *   K_max          the largest depth accepted (sizes the workspace:
 *                  spec_verify_workspace_size(B, K_max, V)); a request with
 *                  d_b > K_max is bad data
 *   n_draft_rows   positions the packed arrays hold, 0 <= n <= 2^30
 * Offsets.  They must form a CSR array: 0 <= o_0 <= o_1 <= ... <= o_B <=
 *   n_draft_rows (o_0 need not be 0).  If they do not, no request's rows or
 *   slots are defined: every num_accepted[b] is -1 and nothing else is
 *   written.  Otherwise bad data is reported per request as in the padded
 *   calls, with -1 in the request's own d_b + 1 output slots.
 * Pointers.  draft_tokens, draft_logits and u_accept may be NULL when
 *   n_draft_rows is 0.  The packed calls do not take draft statistics
 *   (spec_verify_sample_reuse) or windows (the early-exit calls). */
sv_status spec_verify_greedy_packed(const void *target_logits, sv_dtype dt,
                                    const int32_t *draft_tokens,
                                    const int32_t *draft_offsets,
                                    int32_t B, int32_t K_max,
                                    int32_t n_draft_rows, int32_t V,
                                    int32_t *out_tokens, int32_t *num_accepted,
                                    void *workspace, size_t ws_bytes,
                                    hipStream_t stream);

sv_status spec_verify_sample_packed(const void *target_logits,
                                    const void *draft_logits, sv_dtype dt,
                                    const int32_t *draft_tokens,
                                    const int32_t *draft_offsets,
                                    const float *temperature,
                                    const float *u_accept,
                                    const float *u_sample,
                                    int32_t B, int32_t K_max,
                                    int32_t n_draft_rows, int32_t V,
                                    int32_t *out_tokens, int32_t *num_accepted,
                                    float *p_draft, float *q_draft,
                                    void *workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* Allocation-free variant of spec_verify_sample, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, rules, outputs and
 * kernels as spec_verify_sample, without the workspace: the library's own
 * static device scratch array (8 MiB = 8388608 bytes, one per GPU, held
 * until the process ends) serves as the workspace.
 * The call allocates nothing and frees nothing.
 *   Limits.  Shapes whose workspace (spec_verify_workspace_size) exceeds the
 *     array are rejected with SV_ERR_UNSUPPORTED before anything is enqueued
 *     (spec_verify_last_error gives the sizes); B=64, K=16 fits up to
 *     V=152064 in fp32 or bf16.
 *   Concurrency.  Every call on a GPU uses that GPU's one array: calls that
 *     may overlap on one GPU (different streams, different threads) race and
 *     must be serialised by the caller.  Nothing in the array needs clearing
 *     between calls.
 *   Errors.  As spec_verify_sample; SV_ERR_HIP if the array's device address
 *     cannot be obtained.  SPECVERIFY_CHECK does not apply (it would copy to
 *     the host and wait). */
sv_status spec_verify_sample_noalloc(const void *target_logits, const void *draft_logits,
                                     sv_dtype dt, const int32_t *draft_tokens,
                                     const int32_t *depth, const float *temperature,
                                     const float *u_accept, const float *u_sample,
                                     int32_t B, int32_t K, int32_t V,
                                     int32_t *out_tokens, int32_t *num_accepted,
                                     float *p_draft, float *q_draft, hipStream_t stream);

/* Early-exit verification: the rules of spec_verify_greedy and
 * spec_verify_sample, with positions examined in order.  The accepted
 * length counts the drafted tokens approved before the first discrepancy
 * ([Remio], section "Come AngelSpec rende DFly più selettivo"), so no row
 * after a request's first rejection can change its output; these calls do
 * not read them.  The library verifies the positions in windows, one launch
 * sequence per window, back to back on the stream: window w reads positions
 * [window_ends[w-1], window_ends[w]) (window_ends[-1] = 0) of the requests
 * that accepted every earlier position, and the rows a request reads end
 * with the window in which it stops.  The host never waits.
 * Results: on data with no bad values, out_tokens and num_accepted equal
 * those of the one-pass call on the same arguments (the accept decisions
 * take the same arithmetic; row statistics may round differently where the
 * windows change how rows are split into chunks).  Bad data is reported as
 * by the one-pass call, but only at positions up to and including the first
 * rejection, and for the rows and uniforms a draw reads: later positions are
 * not read.  p_draft / q_draft hold p_k(x_k), q_k(x_k) of sampled requests
 * at positions k <= min(n_b, d-1) and 0 elsewhere.
 *   window_ends  HOST array of n_windows ints, read during the call:
 *                strictly increasing, window_ends[0] >= 1, some entry >= K;
 *                entries after the first one >= K are ignored
 *                (SV_ERR_INVALID_ARG otherwise).  Fixed windows of W
 *                positions are W, 2W, ...; fewer windows cost less fixed
 *                latency, a short first window reads less when many
 *                requests reject early.
 *   Other arguments as in spec_verify_greedy / spec_verify_sample.
 *   Timing instrumentation (spec_verify_timing_begin) does not record these
 *   calls. */
sv_status spec_verify_greedy_early_exit(const void *target_logits, sv_dtype dt,
                                        const int32_t *draft_tokens, const int32_t *depth,
                                        int32_t B, int32_t K, int32_t V,
                                        const int32_t *window_ends, int32_t n_windows,
                                        int32_t *out_tokens, int32_t *num_accepted,
                                        void *workspace, size_t ws_bytes, hipStream_t stream);
sv_status spec_verify_sample_early_exit(const void *target_logits, const void *draft_logits,
                                        sv_dtype dt, const int32_t *draft_tokens,
                                        const int32_t *depth, const float *temperature,
                                        const float *u_accept, const float *u_sample,
                                        int32_t B, int32_t K, int32_t V,
                                        const int32_t *window_ends, int32_t n_windows,
                                        int32_t *out_tokens, int32_t *num_accepted,
                                        float *p_draft, float *q_draft,
                                        void *workspace, size_t ws_bytes, hipStream_t stream);

/* Window ends for the early-exit calls from per-position acceptance rates
 * (host computation; nothing is enqueued).  With live(p) = alpha[0] * ... *
 * alpha[p-1] (live(0) = 1) the probability that a request still verifies
 * position p, the plan minimises the expected cost
 *     sum over its windows [lo, hi) of  window_cost + live(lo) * (hi - lo)
 * over every list of ends, exactly (dynamic programming over the window
 * starts, O(K^2)); among plans of equal cost the one with the longer
 * window at each start wins.  The unit of cost is the time to stream one
 * drafted position's rows for the whole batch, and window_cost is a window's
 * fixed latency in that unit (on MI355X, about 13 us per window against
 * about 5 us per position of a batch of 64 sampled requests at V = 128000
 * in bf16: about 2.5).  alpha is what spec_accept_stats_update measures:
 * per-position acceptance ([Hamidun], section "Comment fonctionne la voie
 * MTP", reports these rates).
 *   alpha       [K] double in [0, 1] or NaN (host), may be NULL when K = 0;
 *     NaN, a position no request reached, counts as 0
 *   window_cost finite, >= 0
 *   ends        [max(K, 1)] int32 (host, out): the window ends, ready for
 *               spec_verify_*_early_exit; n_windows (out): how many
 *   Errors: SV_ERR_INVALID_ARG for a NULL output, K outside [0, 1024], an
 *   alpha outside [0, 1] (other than NaN) or a bad window_cost. */
sv_status spec_early_exit_plan(const double *alpha, int32_t K, double window_cost, int32_t *ends,
                               int32_t *n_windows);

/* Draft confidence: conf[b,k] = max_v softmax(y_{b,k})_v at T = 1, the
 * per-position confidence whose running product is the prefix confidence
 * that drives D-cut ([Stack], section "What problem does it solve",
 * inference layer; [AIbase]).  Rows k >= max_depth[b] (NULL => K) are not
 * read and get 0; a bad row (NaN, +inf, all -inf) gets NaN; a max_depth
 * outside [0, K] gives NaN for the whole request.
 *   draft_logits [B, K, V] of dt;  conf [B, K] float (out). */
sv_status spec_draft_confidence(const void *draft_logits, sv_dtype dt,
                                const int32_t *max_depth,
                                int32_t B, int32_t K, int32_t V, float *conf,
                                void *workspace, size_t ws_bytes, hipStream_t stream);

/* Draft-row statistics, for reuse by spec_verify_sample_reuse.  Per draft
 * row (b, k) and temperature T: max = the row's largest logit, sum = the sum
 * over the row of 2^((v - max) * c) with c = (float)(log2(e) / T), so that
 * softmax(y / T)_v = 2^((v - max) * c) / sum; temp = the bits of the fp32 T
 * they were taken at (1.0 from spec_draft_confidence_stats; the request's
 * temperature from spec_draft_confidence_stats_t).  A row the confidence pass
 * did not read (k >= max_depth[b]) or could not use (NaN, +inf, all -inf)
 * gets NaN in max and sum.  16 bytes, 16-byte aligned. */
typedef struct {
    float max;
    int32_t temp;
    double sum;
} sv_row_stat;

/* spec_draft_confidence that also returns every read draft row's
 * statistics.  The prefix confidence that drives D-cut is computed from the
 * draft rows before the target verifies them ([Stack], section "What
 * problem does it solve", inference layer); at T = 1 those rows' softmax
 * statistics are exactly the q_k normalisers the accept test needs, so a
 * later spec_verify_sample_reuse need not read the draft rows again except
 * the one it draws from.
 *   conf         [B, K] float (out) or NULL
 *   draft_stats  [B, K] sv_row_stat (out)
 *   Other arguments as in spec_draft_confidence. */
sv_status spec_draft_confidence_stats(const void *draft_logits, sv_dtype dt,
                                      const int32_t *max_depth,
                                      int32_t B, int32_t K, int32_t V, float *conf,
                                      void *draft_stats,
                                      void *workspace, size_t ws_bytes, hipStream_t stream);

/* spec_draft_confidence_stats with the statistics of request b's rows taken
 * at its own temperature: temperature[b] when that is a finite T > 0 (and
 * not 1), at T = 1 otherwise (T = 0, the greedy rule, reads no draft
 * statistics).  The confidence stays the T = 1 value D-cut ranks by; a row
 * at another temperature gets both from one read (two sums, sharing the
 * row's max).  So a later spec_verify_sample_reuse skips the draft rows of
 * every sampled request, whatever its temperature.
 *   temperature  [B] float (device), the verify call's temperatures
 *   Other arguments as in spec_draft_confidence_stats. */
sv_status spec_draft_confidence_stats_t(const void *draft_logits, sv_dtype dt,
                                        const int32_t *max_depth,
                                        const float *temperature,
                                        int32_t B, int32_t K, int32_t V, float *conf,
                                        void *draft_stats,
                                        void *workspace, size_t ws_bytes, hipStream_t stream);

/* spec_verify_sample with the draft rows' statistics given: for a sampled
 * request whose statistics were taken at its temperature (draft_stats[b, 0]
 * .temp holds the bits of temperature[b]) the draft rows 0..d-1 are not
 * streamed; their (max, sum) come from draft_stats[b, 0..d-1] (as written by
 * spec_draft_confidence_stats or spec_draft_confidence_stats_t on the same
 * draft logits) and the draft logit at each drafted token is read singly.
 * Other requests are verified exactly as by spec_verify_sample.  The rule
 * and every output are those of spec_verify_sample; a NaN statistic (a row
 * the confidence pass did not read, depth[b] > its max_depth[b]) or a later
 * row's record taken at another temperature makes the request bad
 * (num_accepted = -1).  The draft row a residual draw needs is still read.
 *   draft_stats  [B, K] sv_row_stat (read: the first record of every
 *                request, rows 0..d-1 of the requests that reuse them)
 *   Other arguments as in spec_verify_sample. */
sv_status spec_verify_sample_reuse(const void *target_logits, const void *draft_logits,
                                   sv_dtype dt, const int32_t *draft_tokens,
                                   const int32_t *depth, const float *temperature,
                                   const float *u_accept, const float *u_sample,
                                   const void *draft_stats,
                                   int32_t B, int32_t K, int32_t V,
                                   int32_t *out_tokens, int32_t *num_accepted,
                                   float *p_draft, float *q_draft,
                                   void *workspace, size_t ws_bytes, hipStream_t stream);

/* Cost-aware D-cut: the pages describe D-cut as weighing the expected value
 * of keeping more drafted positions against a profiled runtime cost and
 * steering verification toward high-confidence prefixes under a shared
 * budget ([Remio], section "Come AngelSpec rende DFly più selettivo").
 * Each request bids one depth, and a cost budget is spent on the best bids
 * (all arithmetic in double, in the order written):
 *   cost(d)  the latency table (table_depth[i], table_cost[i]) read as a
 *            function of depth: linear between neighbouring points,
 *            table_cost[0] before the first point and table_cost[n-1] from
 *            the last one on; at a table depth, that point's own cost;
 *   request b with K_b = max_depth[b] (NULL => K) in [1, K] bids the depth d
 *            in [1, K_b] with the largest value (P(d) * d) / cost(d), where
 *            P(d) is the product of s(conf[b, 0..d-1]) in order (s as in
 *            dcut_allocate); the smallest such d on ties;
 *   the budget is offered to the bids by value descending, then b
 *   ascending: a bid is granted iff the costs granted so far plus its own
 *   stay <= max_verify; a bid that does not fit is passed over (a later,
 *   cheaper one may still fit).
 *   depth_out[b] = the granted depth, 0 when not granted (or K_b = 0), -1
 *   when K_b is outside [0, K].
 *   conf         [B, K] float (device)
 *   table_depth, table_cost  HOST arrays of table_n (1..32) doubles: depths
 *                strictly increasing, costs finite and > 0 (copied into the
 *                launch; the call keeps no reference)
 *   max_verify   finite, >= 0
 *   B <= 4096 and 8 (K + 1) + 10 P + 2 B <= 60 KiB of LDS, P the power of two
 *   at or above B (SV_ERR_UNSUPPORTED). */
sv_status dcut_allocate_cost(const float *conf, const int32_t *max_depth,
                             int32_t B, int32_t K,
                             const double *table_depth, const double *table_cost,
                             int32_t table_n, double max_verify,
                             int32_t *depth_out, hipStream_t stream);

/* Acceptance statistics across calls: adds one verification call's outcome
 * into counters [2K + 4] of uint64 (device memory the caller zeroes once and
 * keeps).  A serving system has to watch acceptance length ([Remio],
 * section "Cosa non dimostrano i numeri di AngelSpec"), and per-position
 * acceptance is what [Hamidun] reports (section "Comment fonctionne la voie
 * MTP").  For request b with num_accepted n >= 0 and window
 * d = depth[b] (NULL => K), over positions k < min(d, K):
 *   counters[k]     += 1 if position k was tested (n >= k)      (reached)
 *   counters[K + k] += 1 if it was accepted (n > k)            (accepted)
 * and counters[2K] += 1 (requests), counters[2K + 2] += n,
 * counters[2K + 3] += n + 1 (tokens committed, the correction or bonus
 * included); a request with n < 0 adds 1 to counters[2K + 1] (bad) only.
 * alpha_k = accepted / reached, mean accepted = counters[2K+2] / requests,
 * tau = counters[2K+3] / requests.  Inputs are the num_accepted and depth of
 * a spec_verify_* call; stream-ordered after it on the same stream.
 *   counters  [2K + 4] uint64, 8-byte aligned (read-modify-write, atomic) */
sv_status spec_accept_stats_update(const int32_t *num_accepted, const int32_t *depth,
                                   int32_t B, int32_t K, unsigned long long *counters,
                                   hipStream_t stream);

/* Summary of the acceptance counters (host memory: the caller copies the
 * [2K + 4] counters from the device first).  For each position k,
 * alpha[k] = accepted[k] / reached[k] (NaN where no request reached k);
 * *mean_accepted = sum n / requests and *tau = sum (n + 1) / requests, the
 * mean accepted length counted with the bonus token as [Hamidun] reports it
 * (section "Comment fonctionne la voie MTP"); NaN when no request was
 * counted.  Divisions in double.  SV_ERR_INVALID_ARG for a null pointer or
 * K outside [0, 1024]. */
sv_status spec_accept_stats_summary(const unsigned long long *counters, int32_t K, double *alpha,
                                    double *mean_accepted, double *tau);

/* D-cut verification-depth allocation: verification compute is a shared
 * batch-level budget that is moved toward the requests whose drafted
 * prefixes are most likely to be accepted ([Stack], section "What problem
 * does it solve", inference layer; [Remio], section "Come AngelSpec rende
 * DFly più selettivo"), built as a global top-k of prefix confidence:
 *   s(c) = 0 for NaN or c <= 0, 1 for c > 1, c otherwise;
 *   c_{b,0} = s(conf[b,0]); c_{b,k} = float(c_{b,k-1} * s(conf[b,k]))
 *   (float products, sequential in k).  Each request with K_b = max_depth[b]
 *   (NULL => K) in [0, K] first gets min(1, K_b); the remaining budget goes
 *   to the entries (b, k), 1 <= k < K_b, by c descending and then flat index
 *   b*K + k ascending; depth_out[b] = its floor + its entries taken.  A
 *   request with K_b outside [0, K] gets -1 and takes nothing.  The result is
 *   a prefix per request, sum(depth_out) = min(budget, sum of valid K_b).
 *   conf [B, K] float, max_depth [B] int32 or NULL, depth_out [B] int32.
 *   Limits: B*K <= 32768 (the 4*B*K bytes of keys are held in one
 *   workgroup's LDS; a device that gives a workgroup less LDS than that
 *   returns SV_ERR_UNSUPPORTED, with the reason in spec_verify_last_error).
 *   budget < B -> SV_ERR_BUDGET. */
sv_status dcut_allocate(const float *conf, const int32_t *max_depth,
                        int32_t B, int32_t K, int32_t budget, int32_t *depth_out,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
