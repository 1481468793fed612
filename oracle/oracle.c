/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for batched
 * speculative-decoding verification and D-cut depth allocation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library; the two are independent implementations of the same
 * definitions so that one can check the other.
 *
 * Pages cited (titles as printed):
 *   [Stack]    aimodeling.com, "Tencent Hunyuan Turns Speculative Decoding
 *              Into a Full Open-Source Stack"
 *   [Remio]    remio.ai, "Tencent rilascia AngelSpec in open source, sfidando
 *              lo speculative decoding universale"
 *   [Hamidun]  news.hamidun.com, "Tencent открыл AngelSpec - фреймворк для
 *              ускорения инференса LLM через speculative decoding"
 *   [AIbase]   test-news.aibase.com news item 30001 (AngelSpec release)
 *   [DeepDive] happyrock.cloud, "Tencent AngelSpec Speculative Decoding
 *              Framework Deep Dive: MTP + Block Diffusion Dual-Draft Strategy
 *              and D-cut High-Concurrency Throughput Optimization"
 *
 * The pages state the properties of the verification step (one target pass
 * over the whole drafted block, rejection sampling, lossless, accepted prefix
 * plus a bonus token, acceptance reported at T=0) but print no accept rule.
 * The rule below is the standard speculative-sampling construction
 * (Leviathan, Kalman & Matias 2023; Chen et al. 2023), which is the textbook
 * method with exactly those properties.
 *
 * Arithmetic: every floating-point quantity is a C double; exp() is libm's;
 * sums run sequentially in index order.  Build with -ffp-contract=off and no
 * fast-math so the order written here is the order executed.  The D-cut
 * prefix confidence is deliberately float (see oracle_dcut_allocate).
 *
 * Every function returns 0 on success.  Bad per-request data is reported in
 * the outputs (num_accepted = -1), never by aborting.
 *
 * Parity pins: every function below is pinned by a CPU test against closed
 * forms, brute force, exact enumeration or a library routine; none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Row check results. */
#define ROW_OK 0
#define ROW_HAS_NAN 1
#define ROW_ALL_NEG_INF 2

/* Widen one stored logit to double, exactly (bf16 is the upper half of an
 * IEEE binary32 word). */
static double logit_at(const void *base, int dtype, int64_t i)
{
    if (dtype == ORC_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

static const void *row_ptr(const void *base, int dtype, int64_t row, int64_t V)
{
    size_t esize = (dtype == ORC_BF16) ? 2 : 4;
    return (const char *)base + (size_t)row * (size_t)V * esize;
}

/* A row the method reads must hold only finite values and -inf (a masked
 * token), with at least one finite value.  NaN or +inf makes the softmax
 * undefined (inf - inf); an all -inf row has no distribution.  The same rule
 * is applied to greedy rows so that one contract covers both modes. */
static int row_check(const void *row, int dtype, int64_t V)
{
    int any = 0;
    for (int64_t v = 0; v < V; ++v) {
        double z = logit_at(row, dtype, v);
        if (isnan(z) || (isinf(z) && z > 0)) return ROW_HAS_NAN;
        if (!isinf(z)) any = 1;
    }
    return any ? ROW_OK : ROW_ALL_NEG_INF;
}

/* Lowest index holding the largest value; values compare as numbers, so
 * -0.0 ties +0.0.  Ties go to the lowest index (the greedy T=0 rule whose
 * acceptance [Hamidun] reports in its list of numbers). */
int64_t oracle_argmax(const void *row, int dtype, int64_t V)
{
    int64_t best = 0;
    double bv = logit_at(row, dtype, 0);
    for (int64_t v = 1; v < V; ++v) {
        double z = logit_at(row, dtype, v);
        if (z > bv) { bv = z; best = v; }
    }
    return best;
}

/* Softmax at temperature T > 0:  P_v = exp((z_v - M)/T) / S with
 * M = max_v z_v and S = sum_v exp((z_v - M)/T), summed in index order.
 * Writes P into p (may be NULL) and M, S into *M_out, *S_out.
 * Returns ROW_OK or the row-check code. */
int oracle_softmax(const void *row, int dtype, int64_t V, double T,
                   double *p, double *M_out, double *S_out)
{
    int rc = row_check(row, dtype, V);
    if (rc != ROW_OK) return rc;
    double M = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double z = logit_at(row, dtype, v);
        if (z > M) M = z;
    }
    double S = 0.0;
    for (int64_t v = 0; v < V; ++v)
        S += exp((logit_at(row, dtype, v) - M) / T);
    if (p)
        for (int64_t v = 0; v < V; ++v)
            p[v] = exp((logit_at(row, dtype, v) - M) / T) / S;
    if (M_out) *M_out = M;
    if (S_out) *S_out = S;
    return ROW_OK;
}

/* Probability of one token under softmax(row / T). */
static double prob_of(const void *row, int dtype, int64_t V, double T,
                      int64_t x, int *rc)
{
    double M, S;
    *rc = oracle_softmax(row, dtype, V, T, NULL, &M, &S);
    if (*rc != ROW_OK) return NAN;
    return exp((logit_at(row, dtype, x) - M) / T) / S;
}

/* Inverse-CDF draw: the first t whose inclusive prefix sum of r exceeds
 * u * R, R = sum(r), both in index order.  If rounding leaves no such t,
 * the last t with r_t > 0.  Returns -1 when r has no positive mass. */
int64_t oracle_inverse_cdf(const double *r, int64_t V, double u)
{
    double R = 0.0;
    for (int64_t v = 0; v < V; ++v) R += r[v];
    double target = u * R;
    double acc = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        acc += r[v];
        if (acc > target) return v;
    }
    for (int64_t v = V - 1; v >= 0; --v)
        if (r[v] > 0.0) return v;
    return -1;
}

/* Distribution the correction token is drawn from after a rejection at a
 * position with target row trow and draft row drow:
 *     r_v = max(0, P(trow)_v - P(drow)_v)
 * (un-normalised; the draw normalises by R = sum r).  When drow is NULL
 * this is the bonus distribution r = P(trow).  When every r_v is zero
 * (possible only through rounding, since a rejection needs P(x) < Q(x)),
 * r falls back to P(trow), which keeps the output a sample of the target.
 * Returns ROW_OK, a row-check code, or 3 if the fallback was taken. */
int oracle_residual(const void *trow, const void *drow, int dtype, int64_t V,
                    double T, double *r)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = drow ? (double *)malloc(sizeof(double) * (size_t)V) : NULL;
    int rc = oracle_softmax(trow, dtype, V, T, p, NULL, NULL);
    if (rc == ROW_OK && drow) rc = oracle_softmax(drow, dtype, V, T, q, NULL, NULL);
    if (rc != ROW_OK) { free(p); free(q); return rc; }
    if (!drow) {
        memcpy(r, p, sizeof(double) * (size_t)V);
        free(p);
        return ROW_OK;
    }
    double R = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        double d = p[v] - q[v];
        r[v] = d > 0.0 ? d : 0.0;
        R += r[v];
    }
    int fell_back = 0;
    if (R == 0.0) {
        memcpy(r, p, sizeof(double) * (size_t)V);
        fell_back = 1;
    }
    free(p);
    free(q);
    return fell_back ? 3 : ROW_OK;
}

static void mark_bad(int32_t *out_row, int32_t K, int32_t *num)
{
    for (int32_t k = 0; k <= K; ++k) out_row[k] = -1;
    *num = -1;
}

/* Greedy verification of one request over target rows 0..d (T = 0):
 * accept drafted token k iff it equals the target argmax of row k; the
 * accepted length n is the count before the first mismatch ([Remio],
 * section "Come AngelSpec rende DFly più selettivo"); the emitted token is
 * the argmax of row n, which is the correction token when n < d and the
 * bonus token when n = d ([Stack], section "What problem does it solve").
 * Returns 1 if the request's data is bad. */
static int greedy_one(const void *target, int dtype, const int32_t *tok,
                      int32_t K, int64_t V, int64_t b, int32_t d,
                      int32_t *out_row, int32_t *num)
{
    for (int32_t k = 0; k < d; ++k)
        if (tok[k] < 0 || (int64_t)tok[k] >= V) return 1;
    for (int32_t k = 0; k <= d; ++k)
        if (row_check(row_ptr(target, dtype, b * (K + 1) + k, V), dtype, V) != ROW_OK)
            return 1;
    int32_t n = d;
    for (int32_t k = 0; k < d; ++k) {
        int64_t g = oracle_argmax(row_ptr(target, dtype, b * (K + 1) + k, V), dtype, V);
        if ((int64_t)tok[k] != g) { n = k; break; }
    }
    int64_t emit = oracle_argmax(row_ptr(target, dtype, b * (K + 1) + n, V), dtype, V);
    for (int32_t k = 0; k <= K; ++k) out_row[k] = -1;
    for (int32_t k = 0; k < n; ++k) out_row[k] = tok[k];
    out_row[n] = (int32_t)emit;
    *num = n;
    return 0;
}

/* Greedy (T = 0) verification of a batch.
 * target [B, K+1, V], tokens [B, K], depth [B] or NULL (=> K),
 * out_tokens [B, K+1], num_accepted [B].  A request with depth outside
 * [0, K], a drafted token outside [0, V) or a NaN / all -inf target row in
 * its window gets num_accepted = -1 and out_tokens = -1. */
int oracle_verify_greedy(const void *target, int dtype, const int32_t *tokens,
                         const int32_t *depth, int32_t B, int32_t K, int64_t V,
                         int32_t *out_tokens, int32_t *num_accepted)
{
    for (int64_t b = 0; b < B; ++b) {
        int32_t *out_row = out_tokens + b * (K + 1);
        int32_t d = depth ? depth[b] : K;
        if (d < 0 || d > K ||
            greedy_one(target, dtype, tokens + b * K, K, V, b, d, out_row,
                       num_accepted + b))
            mark_bad(out_row, K, num_accepted + b);
    }
    return 0;
}

static int bad_uniform(float u) { return !(u >= 0.0f && u < 1.0f); }

/* Temperatures the contract accepts: 0 (the greedy rule, the limit of
 * softmax(z/T) as T falls to 0) or any finite T > 0, for which softmax(z/T)
 * is defined for every row of finite and -inf logits.  NaN is no number;
 * a negative T would reverse the ranking of the tokens; T = +inf would make
 * (z - M)/T the undefined -inf/inf at a masked token.  Those are bad data. */
static int bad_temperature(float T) { return !(T == 0.0f || (T > 0.0f && isfinite(T))); }

/* Sampled verification (rejection sampling) of a batch.
 *
 * For each request b with depth d and temperature T:
 *   T == 0: the greedy rule above on target rows 0..d.
 *   T  > 0: for k = 0..d-1 with x = tokens[b,k]
 *             a = P(z_{b,k})_x,  c = P(y_{b,k})_x      (softmax at T)
 *             ratio = min(1, a/c) if c > 0; 1 if c == 0 < a; 0 if both 0
 *             accept iff (double)u_accept[b,k] < ratio (strict)
 *           n = first rejected k, or d if none.
 *           n <  d: draw from r = max(0, P(z_{b,n}) - P(y_{b,n}))
 *           n == d: draw the bonus token from r = P(z_{b,d})
 *           with the inverse CDF at u_sample[b].
 * This is one pass over the drafted block by rejection sampling that keeps
 * the target's output distribution ([Stack], section "What problem does it
 * solve"; [Hamidun], section "Qu'est-ce que le speculative decoding";
 * [Remio], section "Cosa non dimostrano i numeri di AngelSpec").
 *
 * p_draft / q_draft [B, K] (may be NULL) receive (float)a and (float)c for
 * every k < d of sampled requests, 0 elsewhere.  ratio_out [B, K] (may be
 * NULL) receives the ratio, NaN where none is computed.
 *
 * Bad data (depth outside [0,K], T not 0 and not a finite T > 0, token outside [0,V), a
 * uniform outside [0,1), NaN or all -inf in a row that is read) gives
 * num_accepted = -1 and out_tokens = -1 for that request.  The rows read
 * are target and draft rows 0..d-1, plus target row d only when nothing
 * is rejected. */
int oracle_verify_sample(const void *target, const void *draft, int dtype,
                         const int32_t *tokens, const int32_t *depth,
                         const float *temperature, const float *u_accept,
                         const float *u_sample, int32_t B, int32_t K, int64_t V,
                         int32_t *out_tokens, int32_t *num_accepted,
                         float *p_draft, float *q_draft, double *ratio_out)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    for (int64_t b = 0; b < B; ++b) {
        int32_t *out_row = out_tokens + b * (K + 1);
        const int32_t *tok = tokens + b * K;
        int32_t d = depth ? depth[b] : K;
        double T = temperature ? (double)temperature[b] : 0.0;
        for (int32_t k = 0; k < K; ++k) {
            if (p_draft) p_draft[b * K + k] = 0.0f;
            if (q_draft) q_draft[b * K + k] = 0.0f;
            if (ratio_out) ratio_out[b * K + k] = NAN;
        }
        if (d < 0 || d > K || bad_temperature(temperature ? temperature[b] : 0.0f)) {
            mark_bad(out_row, K, num_accepted + b);
            continue;
        }
        if (T == 0.0) {
            if (greedy_one(target, dtype, tok, K, V, b, d, out_row, num_accepted + b))
                mark_bad(out_row, K, num_accepted + b);
            continue;
        }
        int bad = bad_uniform(u_sample[b]);
        for (int32_t k = 0; k < d && !bad; ++k)
            bad = tok[k] < 0 || (int64_t)tok[k] >= V || bad_uniform(u_accept[b * K + k]);
        int32_t n = d;
        for (int32_t k = 0; k < d && !bad; ++k) {
            int rc1, rc2;
            const void *zr = row_ptr(target, dtype, b * (K + 1) + k, V);
            const void *yr = row_ptr(draft, dtype, b * K + k, V);
            double a = prob_of(zr, dtype, V, T, tok[k], &rc1);
            double c = prob_of(yr, dtype, V, T, tok[k], &rc2);
            if (rc1 != ROW_OK || rc2 != ROW_OK) { bad = 1; break; }
            double ratio;
            if (c > 0.0) ratio = (a / c < 1.0) ? a / c : 1.0;
            else ratio = (a > 0.0) ? 1.0 : 0.0;
            if (p_draft) p_draft[b * K + k] = (float)a;
            if (q_draft) q_draft[b * K + k] = (float)c;
            if (ratio_out) ratio_out[b * K + k] = ratio;
            /* Every row in the window is read (one pass over the block), so
             * the scan continues past the first rejection for the outputs
             * above, but n keeps the first one. */
            if (n == d && !((double)u_accept[b * K + k] < ratio)) n = k;
        }
        if (!bad) {
            int rc;
            if (n < d)
                rc = oracle_residual(row_ptr(target, dtype, b * (K + 1) + n, V),
                                     row_ptr(draft, dtype, b * K + n, V),
                                     dtype, V, T, r);
            else
                rc = oracle_residual(row_ptr(target, dtype, b * (K + 1) + d, V),
                                     NULL, dtype, V, T, r);
            if (rc == ROW_HAS_NAN || rc == ROW_ALL_NEG_INF) bad = 1;
        }
        if (bad) {
            mark_bad(out_row, K, num_accepted + b);
            for (int32_t k = 0; k < K; ++k) {
                if (p_draft) p_draft[b * K + k] = 0.0f;
                if (q_draft) q_draft[b * K + k] = 0.0f;
                if (ratio_out) ratio_out[b * K + k] = NAN;
            }
            continue;
        }
        int64_t t = oracle_inverse_cdf(r, V, (double)u_sample[b]);
        for (int32_t k = 0; k <= K; ++k) out_row[k] = -1;
        for (int32_t k = 0; k < n; ++k) out_row[k] = tok[k];
        out_row[n] = (int32_t)t;
        num_accepted[b] = n;
    }
    free(r);
    return 0;
}

/* Early-exit verification of a batch: the same accept rules (the greedy
 * rule at T = 0, rejection sampling at T > 0), but positions are examined in
 * order and the first rejection ends the request.  The accepted length
 * counts the drafted tokens approved before the first discrepancy ([Remio],
 * section "Come AngelSpec rende DFly più selettivo"), so nothing after that
 * position can change the committed prefix or the emitted token; this
 * reading reads nothing after it.
 *
 * For request b with depth d and temperature T (temperature NULL: all 0):
 *   position k = 0, 1, ... < d reads tokens[b,k], target row k and, at
 *   T > 0, u_accept[b,k] and draft row k.  Bad data at position k (a token
 *   outside [0,V), a uniform outside [0,1), NaN, +inf or all -inf in a row
 *   read there) makes the request bad; a rejection at k ends the scan with
 *   n = k.  If no position rejects, n = d and the bonus row d is read.
 *   The emitted token is chosen as in oracle_verify_greedy (argmax of target
 *   row n) or oracle_verify_sample (inverse CDF of the residual or bonus
 *   distribution at u_sample[b], which is read only then).
 * Bad data after the stopping position is never read and so never reported.
 * On inputs with no bad data the outputs equal oracle_verify_sample's
 * out_tokens and num_accepted.
 *
 * p_draft / q_draft [B,K] (may be NULL) receive (float)a and (float)c for
 * the positions read, k <= min(n, d-1), of sampled requests; 0 elsewhere and
 * everywhere for bad or greedy requests. */
int oracle_verify_early_exit(const void *target, const void *draft, int dtype,
                             const int32_t *tokens, const int32_t *depth,
                             const float *temperature, const float *u_accept,
                             const float *u_sample, int32_t B, int32_t K, int64_t V,
                             int32_t *out_tokens, int32_t *num_accepted,
                             float *p_draft, float *q_draft)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    for (int64_t b = 0; b < B; ++b) {
        int32_t *out_row = out_tokens + b * (K + 1);
        const int32_t *tok = tokens + b * K;
        int32_t d = depth ? depth[b] : K;
        float Tf = temperature ? temperature[b] : 0.0f;
        double T = (double)Tf;
        for (int32_t k = 0; k < K; ++k) {
            if (p_draft) p_draft[b * K + k] = 0.0f;
            if (q_draft) q_draft[b * K + k] = 0.0f;
        }
        int bad = d < 0 || d > K || bad_temperature(Tf);
        int32_t n = d;
        int64_t emit = -1;
        if (!bad && T == 0.0) {
            for (int32_t k = 0; k < d; ++k) {
                const void *zr = row_ptr(target, dtype, b * (K + 1) + k, V);
                if (tok[k] < 0 || (int64_t)tok[k] >= V || row_check(zr, dtype, V) != ROW_OK) { bad = 1; break; }
                int64_t g = oracle_argmax(zr, dtype, V);
                if ((int64_t)tok[k] != g) { n = k; emit = g; break; }
            }
            if (!bad && n == d) {
                const void *zr = row_ptr(target, dtype, b * (K + 1) + d, V);
                if (row_check(zr, dtype, V) != ROW_OK) bad = 1;
                else emit = oracle_argmax(zr, dtype, V);
            }
        } else if (!bad) {
            for (int32_t k = 0; k < d; ++k) {
                const int32_t x = tok[k];
                if (x < 0 || (int64_t)x >= V || bad_uniform(u_accept[b * K + k])) { bad = 1; break; }
                int rc1, rc2;
                double a = prob_of(row_ptr(target, dtype, b * (K + 1) + k, V), dtype, V, T, x, &rc1);
                double c = prob_of(row_ptr(draft, dtype, b * K + k, V), dtype, V, T, x, &rc2);
                if (rc1 != ROW_OK || rc2 != ROW_OK) { bad = 1; break; }
                double ratio;
                if (c > 0.0) ratio = (a / c < 1.0) ? a / c : 1.0;
                else ratio = (a > 0.0) ? 1.0 : 0.0;
                if (p_draft) p_draft[b * K + k] = (float)a;
                if (q_draft) q_draft[b * K + k] = (float)c;
                if (!((double)u_accept[b * K + k] < ratio)) { n = k; break; }
            }
            if (!bad && bad_uniform(u_sample[b])) bad = 1;
            if (!bad) {
                int rc;
                if (n < d)
                    rc = oracle_residual(row_ptr(target, dtype, b * (K + 1) + n, V),
                                         row_ptr(draft, dtype, b * K + n, V), dtype, V, T, r);
                else
                    rc = oracle_residual(row_ptr(target, dtype, b * (K + 1) + d, V),
                                         NULL, dtype, V, T, r);
                if (rc == ROW_HAS_NAN || rc == ROW_ALL_NEG_INF) bad = 1;
                else emit = oracle_inverse_cdf(r, V, (double)u_sample[b]);
            }
        }
        if (bad) {
            mark_bad(out_row, K, num_accepted + b);
            for (int32_t k = 0; k < K; ++k) {
                if (p_draft) p_draft[b * K + k] = 0.0f;
                if (q_draft) q_draft[b * K + k] = 0.0f;
            }
            continue;
        }
        for (int32_t k = 0; k <= K; ++k) out_row[k] = -1;
        for (int32_t k = 0; k < n; ++k) out_row[k] = tok[k];
        out_row[n] = (int32_t)emit;
        num_accepted[b] = n;
    }
    free(r);
    return 0;
}

/* Draft confidence: the largest softmax probability of each draft row at
 * T = 1, which equals 1/S with S = sum_v exp(y_v - M).  Rows k >= K_b
 * (max_depth[b], NULL => K) are not read and get 0; a bad row gets NaN.
 * This is the per-position confidence whose running product is the
 * "prefix confidence" that drives D-cut ([Stack], section "What problem
 * does it solve", inference layer; [AIbase]). */
int oracle_draft_confidence(const void *draft, int dtype, const int32_t *max_depth,
                            int32_t B, int32_t K, int64_t V, float *conf)
{
    for (int64_t b = 0; b < B; ++b) {
        int32_t Kb = max_depth ? max_depth[b] : K;
        for (int32_t k = 0; k < K; ++k) {
            float *o = conf + b * K + k;
            if (k >= Kb) { *o = 0.0f; continue; }
            double S;
            int rc = oracle_softmax(row_ptr(draft, dtype, b * K + k, V), dtype, V,
                                    1.0, NULL, NULL, &S);
            *o = (rc == ROW_OK) ? (float)(1.0 / S) : NAN;
        }
    }
    return 0;
}

/* Confidence sanitisation shared by definition (not by code) with the
 * device allocator: NaN and negatives count as 0, values above 1 as 1. */
static float sanitize_conf(float c)
{
    if (!(c > 0.0f)) return 0.0f;   /* NaN, -0, negatives */
    if (c > 1.0f) return 1.0f;
    return c;
}

typedef struct { float c; int64_t flat; int32_t b; } dcut_entry;

static int dcut_cmp(const void *pa, const void *pb)
{
    const dcut_entry *a = (const dcut_entry *)pa, *b = (const dcut_entry *)pb;
    if (a->c > b->c) return -1;
    if (a->c < b->c) return 1;
    return (a->flat < b->flat) ? -1 : (a->flat > b->flat);
}

/* D-cut verification-depth allocation as a global top-k of prefix
 * confidence.  The pages describe D-cut as treating verification compute as
 * a shared batch-level budget that is moved toward high-confidence prefixes
 * ([Stack], section "What problem does it solve"; [Remio], section "Come
 * AngelSpec rende DFly più selettivo"); the global top-k is the reading
 * built here.
 *
 *   c_{b,0} = s(conf_{b,0}),  c_{b,k} = float(c_{b,k-1} * s(conf_{b,k}))
 *   (s = sanitisation above; products in float, sequential in k).
 *   Each valid request (K_b in [0,K]) first gets min(1, K_b).  The remaining
 *   budget goes to the entries (b,k), 1 <= k < K_b, in order of c
 *   descending, then flat index b*K+k ascending.  d_b = floor + taken.
 *   Requests with K_b outside [0,K] get -1 and take nothing.
 * Returns 1 for B < 1 or K < 0, 4 if budget < B. */
int oracle_dcut_allocate(const float *conf, const int32_t *max_depth, int32_t B,
                         int32_t K, int32_t budget, int32_t *depth_out)
{
    if (B < 1 || K < 0) return 1;
    if (budget < B) return 4;
    dcut_entry *e = (dcut_entry *)malloc(sizeof(dcut_entry) * ((size_t)B * (size_t)K + 1));
    int64_t ne = 0, floors = 0;
    for (int64_t b = 0; b < B; ++b) {
        int32_t Kb = max_depth ? max_depth[b] : K;
        if (Kb < 0 || Kb > K) { depth_out[b] = -1; continue; }
        depth_out[b] = Kb > 0 ? 1 : 0;
        floors += depth_out[b];
        float c = 0.0f;
        for (int32_t k = 0; k < Kb; ++k) {
            float s = sanitize_conf(conf[b * K + k]);
            c = (k == 0) ? s : c * s;
            if (k >= 1) { e[ne].c = c; e[ne].flat = b * K + k; e[ne].b = (int32_t)b; ++ne; }
        }
    }
    qsort(e, (size_t)ne, sizeof(dcut_entry), dcut_cmp);
    int64_t take = (int64_t)budget - floors;
    if (take > ne) take = ne;
    for (int64_t i = 0; i < take; ++i) depth_out[e[i].b] += 1;
    free(e);
    return 0;
}

/* Acceptance statistics of one verification call, added into counters
 * [2K + 4] (the monitoring of acceptance length the pages ask of a serving
 * system, [Remio] section "Cosa non dimostrano i numeri di AngelSpec"; the
 * per-position acceptance [Hamidun] reports, section "Comment fonctionne la
 * voie MTP").  The definition, one request at a time:
 *   a request with num_accepted n < 0 is bad: counters[2K + 1] += 1;
 *   otherwise, with window d = depth[b] (NULL: K):
 *     for every position k < d that was tested (all drafts before it were
 *     accepted, n >= k): counters[k] += 1 (reached);
 *     if it was also accepted (n > k): counters[K + k] += 1 (accepted);
 *     counters[2K] += 1 (requests), counters[2K + 2] += n,
 *     counters[2K + 3] += n + 1 (tokens committed: accepted prefix plus the
 *     correction or bonus token).
 * Returns 1 for B < 1 or K < 0. */
int oracle_accept_stats(const int32_t *num_accepted, const int32_t *depth, int32_t B, int32_t K,
                        uint64_t *counters)
{
    if (B < 1 || K < 0) return 1;
    for (int64_t b = 0; b < B; ++b) {
        int32_t n = num_accepted[b];
        if (n < 0) {
            counters[2 * K + 1] += 1;
            continue;
        }
        int32_t d = depth ? depth[b] : K;
        for (int32_t k = 0; k < d && k < K; ++k) {
            if (n >= k) counters[k] += 1;
            if (n > k) counters[K + k] += 1;
        }
        counters[2 * K] += 1;
        counters[2 * K + 2] += (uint64_t)n;
        counters[2 * K + 3] += (uint64_t)n + 1;
    }
    return 0;
}

/* Cost-aware D-cut.  [Remio] (section "Come AngelSpec rende DFly più
 * selettivo") has D-cut weigh the expected value of more drafted positions
 * against a profiled runtime cost, and [DeepDive] sketches a scheduler that
 * scores each request's depth by benefit per unit of cost and then spends a
 * verification budget on the best scores.  The rule built here:
 *
 *   cost(d): the latency table (tdepth[i], tcost[i]), tdepth strictly
 *     increasing, read as a function of depth that is linear between
 *     neighbouring table points and constant before the first point and
 *     after the last.  At a table depth it is that point's own cost.
 *   value of request b at depth d: V_b(d) = (P_b(d) * d) / cost(d), where
 *     P_b(d) = s(conf[b,0]) * ... * s(conf[b,d-1]) multiplied in order in
 *     double (s as in oracle_dcut_allocate).
 *   request b (K_b = max_depth[b], NULL => K, in [1, K]) bids the depth in
 *     [1, K_b] with the largest value, the smallest such depth on ties.
 *   The budget max_verify is then offered to the bids one at a time, in
 *     order of value (highest first, lower request index on ties).  A bid
 *     whose cost fits in what is left (spent + cost <= max_verify, spent
 *     summed in offer order) is granted its depth; one that does not fit
 *     gets 0 and the offer moves on, so a later, cheaper bid may still fit.
 *   depth_out[b] = the granted depth, 0 (not granted, or K_b = 0), or -1
 *     (K_b outside [0, K]).
 * Returns 1 for B < 1, K < 0 or n < 1. */
double oracle_dcut_cost(const double *tdepth, const double *tcost, int32_t n, double d)
{
    int32_t above = 0;                 /* table points at or below d */
    while (above < n && tdepth[above] <= d) ++above;
    if (above == 0) return tcost[0];
    if (above == n) return tcost[n - 1];
    /* tdepth[above - 1] <= d < tdepth[above] */
    double w = (d - tdepth[above - 1]) / (tdepth[above] - tdepth[above - 1]);
    return tcost[above - 1] + w * (tcost[above] - tcost[above - 1]);
}

int oracle_dcut_allocate_cost(const float *conf, const int32_t *max_depth, int32_t B, int32_t K,
                              const double *tdepth, const double *tcost, int32_t n, double max_verify,
                              int32_t *depth_out)
{
    if (B < 1 || K < 0 || n < 1) return 1;
    double *value = (double *)malloc(sizeof(double) * (size_t)B);
    int32_t *bid = (int32_t *)malloc(sizeof(int32_t) * (size_t)B);
    char *open_bid = (char *)calloc((size_t)B, 1);
    for (int64_t b = 0; b < B; ++b) {
        int32_t Kb = max_depth ? max_depth[b] : K;
        depth_out[b] = (Kb < 0 || Kb > K) ? -1 : 0;
        if (Kb < 1 || Kb > K) continue;
        double P = 1.0;
        for (int32_t d = 1; d <= Kb; ++d) {
            P = P * (double)sanitize_conf(conf[b * K + d - 1]);
            double v = (P * (double)d) / oracle_dcut_cost(tdepth, tcost, n, (double)d);
            if (d == 1 || v > value[b]) { value[b] = v; bid[b] = d; }
        }
        open_bid[b] = 1;
    }
    double spent = 0.0;
    for (;;) {
        int64_t best = -1;             /* highest open bid, lowest index on ties */
        for (int64_t b = 0; b < B; ++b)
            if (open_bid[b] && (best < 0 || value[b] > value[best])) best = b;
        if (best < 0) break;
        open_bid[best] = 0;
        double c = oracle_dcut_cost(tdepth, tcost, n, (double)bid[best]);
        if (spent + c <= max_verify) {
            spent = spent + c;
            depth_out[best] = bid[best];
        }
    }
    free(value);
    free(bid);
    free(open_bid);
    return 0;
}
