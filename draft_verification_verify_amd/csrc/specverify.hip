// libspecverify: batched verification of drafted tokens (speculative
// decoding) and D-cut verification-depth allocation, written for AMD Instinct
// MI355X (gfx950, CDNA4, wave64).
//
// Pages cited (titles as printed):
//   [Stack]  aimodeling.com, "Tencent Hunyuan Turns Speculative Decoding Into
//            a Full Open-Source Stack"
//   [Remio]  remio.ai, "Tencent rilascia AngelSpec in open source, sfidando lo
//            speculative decoding universale"
//   [Hamidun] news.hamidun.com, "Tencent открыл AngelSpec - фреймворк для
//            ускорения инференса LLM через speculative decoding"
//
// The target verifies every drafted token of every request in one pass over
// its logits and commits the accepted prefix plus one token drawn by
// rejection sampling ([Stack], section "What problem does it solve";
// [Hamidun], section "Qu'est-ce que le speculative decoding"); the accept
// rule is the standard speculative-sampling construction (Leviathan et al.
// 2023; Chen et al. 2023).
//
// Structure of one verification call (all kernels on the caller's stream):
//  1. row_stats_kernel -- persistent grid; every workgroup plans the batch
//     itself from depth[] and temperature[] (no host round trip), then walks
//     (row, chunk) tasks.  A task streams one chunk of one logit row from HBM
//     with 16-byte loads and reduces it to (max, lowest argmax) or to
//     (max, sum of exp) in fp32 with a double accumulator.  The last chunk of
//     a row to finish (device-scope atomic) merges the chunk partials; the
//     last row of a request to finish runs that request's accept test and
//     first-rejection scan (one wave, lanes over positions).
//  2. sampler_sums_kernel -- per (request, chunk) of the one row pair a
//     sampled request draws from: fp64 softmax normalisers of that pair.
//  3. sampler_draw_kernel -- per (request, chunk): fp64 residual
//     max(0, p - q) (or p for the bonus) chunk totals; the last chunk of a
//     request to finish locates u*R among the chunk totals and scans that
//     chunk for the token.
// Greedy calls run only step 1.  The draft-confidence call runs step 1 in a
// third mode.  dcut_allocate is one workgroup: fp32 running products and an
// LDS radix select.
//
// Nothing on this path is a dense contraction, so there is no MFMA here: the
// row pass is bound by HBM bandwidth, the sampler by fp64 VALU throughput.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "specverify.h"

namespace {

constexpr int WG = 256;           // threads per workgroup
constexpr int NWAVE = WG / 64;    // wave64
constexpr int UMAX = 8;           // 16-byte loads per thread per row task
constexpr int US = 4;             // 16-byte loads per thread per sampler task
constexpr int CPR_CAP = 256;      // chunks per row, at most
constexpr int B_MAX = 4096;
constexpr int K_MAX = 1024;
constexpr int V_MAX = 2000000;
constexpr int DCUT_MAX = 32768;   // B*K for dcut_allocate
constexpr int DCUT_WG = 1024;

enum : int { MODE_GREEDY = 0, MODE_SAMPLE = 1, MODE_CONF = 2 };
enum : int { KIND_GREEDY = 0, KIND_SAMPLED = 1, KIND_CONF = 2, KIND_BAD = 3 };
enum : int { SREQ_NONE = 0, SREQ_RESID = 1, SREQ_BONUS = 2 };

constexpr double LOG2E = 1.4426950408889634;

// Partial or merged statistics of (part of) a row.  Argmax rows use (m, idx);
// log-sum-exp rows use (m, s) with s = sum exp2((v - m) * log2e / T).  A row
// that is unusable (NaN, +inf, nothing but -inf) has m = NaN.
struct alignas(16) Stat {
    float m;
    int32_t idx;
    double s;
};

struct alignas(16) ReqDesc {
    int32_t state;   // SREQ_*
    int32_t n;       // accepted length = row the sampler reads
    int32_t pad;
    float T;
};

struct alignas(16) S1Part {
    float mz, my;
    int32_t bad, pad;
    double sz, sy;
};

struct alignas(16) S2Part {
    double r, p;
};

struct Ws {
    uint32_t *row_cnt;   // [R_max]
    uint32_t *req_cnt;   // [B]
    Stat *part;          // [R_max * cpr_max]
    Stat *rows;          // [R_max]
    ReqDesc *req;        // [B]
    S1Part *s1;          // [B * cs_max]
    uint32_t *s1cnt;     // [B]
    S1Part *s1tot;       // [B]
    S2Part *s2;          // [B * cs_max]
    uint32_t *s2cnt;     // [B]
};

struct Layout {
    size_t off[10];
    size_t total;
    int64_t r_max;
    int cpr_max;
    int cs_max;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Vectors of 16 bytes that can cover a row of V elements starting at any
// element offset within a vector (elements per vector epv).
__host__ __device__ inline int64_t nvec_max(int V, int epv) { return ceil_div((int64_t)V + epv - 1, epv); }

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool make_layout(int B, int K, int V, Layout &L)
{
    if (B < 1 || B > B_MAX || K < 0 || K > K_MAX || V < 1 || V > V_MAX) return false;
    const int64_t nv = nvec_max(V, 4);   // fp32 is the worst case
    L.r_max = (int64_t)B * (2 * K + 1);
    L.cpr_max = (int)std::min<int64_t>(CPR_CAP, ceil_div(nv, WG));
    L.cs_max = (int)ceil_div(nv, (int64_t)WG * US);
    const size_t sz[10] = {
        sizeof(uint32_t) * (size_t)L.r_max,
        sizeof(uint32_t) * (size_t)B,
        sizeof(Stat) * (size_t)L.r_max * (size_t)L.cpr_max,
        sizeof(Stat) * (size_t)L.r_max,
        sizeof(ReqDesc) * (size_t)B,
        sizeof(S1Part) * (size_t)B * (size_t)L.cs_max,
        sizeof(uint32_t) * (size_t)B,
        sizeof(S1Part) * (size_t)B,
        sizeof(S2Part) * (size_t)B * (size_t)L.cs_max,
        sizeof(uint32_t) * (size_t)B,
    };
    size_t o = 0;
    for (int i = 0; i < 10; ++i) {
        L.off[i] = o;
        o += align256(sz[i]);
    }
    L.total = o;
    return true;
}

Ws carve(void *base, const Layout &L)
{
    char *p = (char *)base;
    Ws w;
    w.row_cnt = (uint32_t *)(p + L.off[0]);
    w.req_cnt = (uint32_t *)(p + L.off[1]);
    w.part = (Stat *)(p + L.off[2]);
    w.rows = (Stat *)(p + L.off[3]);
    w.req = (ReqDesc *)(p + L.off[4]);
    w.s1 = (S1Part *)(p + L.off[5]);
    w.s1cnt = (uint32_t *)(p + L.off[6]);
    w.s1tot = (S1Part *)(p + L.off[7]);
    w.s2 = (S2Part *)(p + L.off[8]);
    w.s2cnt = (uint32_t *)(p + L.off[9]);
    return w;
}

struct Params {
    const void *target;
    const void *draft;
    const int32_t *tokens;
    const int32_t *depth;
    const float *temperature;
    const float *u_accept;
    const float *u_sample;
    const int32_t *max_depth;
    int32_t *out_tokens;
    int32_t *num_accepted;
    float *p_draft;
    float *q_draft;
    float *conf;
    int32_t B, K, V;
    int32_t bf16;      // logits dtype: 1 bf16, 0 fp32
    int32_t mode;
    int32_t cpr_max;
    int32_t cs;        // sampler chunks per row (this call's dtype)
    Ws ws;
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element e of a 16-byte vector, as fp32 (exact widening for bf16).
template <bool BF16>
__device__ __forceinline__ void unpack(const uint4 &v, float *f)
{
    if constexpr (BF16) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
}

template <bool BF16>
__device__ __forceinline__ float load_logit(const void *base, int64_t i)
{
    if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t *)base)[i] << 16);
    else return ((const float *)base)[i];
}

__device__ __forceinline__ float load_logit_dt(const void *base, bool bf16, int64_t i)
{
    return bf16 ? load_logit<true>(base, i) : load_logit<false>(base, i);
}

// Device-scope release/acquire around the cross-workgroup hand-offs.  The
// eight XCDs have separate L2s, so a partial written by one workgroup is made
// visible to a workgroup on another XCD only through agent-scope fences.
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t atomic_inc_agent(uint32_t *p)
{
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_zero_agent(uint32_t *p)
{
    __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ int wave_or(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, 64);
    return v;
}

// (value desc, index asc) argmax merge; NaN values are carried by a flag.
__device__ __forceinline__ void argmax_merge(float &m, int &i, float m2, int i2)
{
    if (m2 > m || (m2 == m && i2 < i)) { m = m2; i = i2; }
}

__device__ __forceinline__ void wave_argmax(float &m, int &i)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o, 64);
        int i2 = __shfl_xor(i, o, 64);
        argmax_merge(m, i, m2, i2);
    }
}

// Workgroup reductions through LDS (all threads must call; result in all).
struct RedSmem {
    float f[NWAVE];
    int i[NWAVE];
    double d[NWAVE];
    int flag;
};

__device__ float wg_max(float v, RedSmem &sm)
{
    v = wave_max(v);
    __syncthreads();
    if (lane_id() == 0) sm.f[wave_id()] = v;
    __syncthreads();
    float r = sm.f[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) r = fmaxf(r, sm.f[w]);
    return r;
}

__device__ double wg_sum(double v, RedSmem &sm)
{
    v = wave_sum(v);
    __syncthreads();
    if (lane_id() == 0) sm.d[wave_id()] = v;
    __syncthreads();
    double r = sm.d[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) r += sm.d[w];
    return r;
}

__device__ int wg_or(int v, RedSmem &sm)
{
    v = wave_or(v);
    __syncthreads();
    if (lane_id() == 0) sm.i[wave_id()] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) r |= sm.i[w];
    return r;
}

__device__ void wg_argmax(float &m, int &i, RedSmem &sm)
{
    wave_argmax(m, i);
    __syncthreads();
    if (lane_id() == 0) { sm.f[wave_id()] = m; sm.i[wave_id()] = i; }
    __syncthreads();
    m = sm.f[0];
    i = sm.i[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) argmax_merge(m, i, sm.f[w], sm.i[w]);
}

// ---------------------------------------------------------------------------
// Batch plan: rows each request contributes to the row pass.
//   greedy request (greedy call, or T == 0): target rows 0..d
//   sampled request (T > 0): target rows 0..d-1, then draft rows 0..d-1
//   confidence call: draft rows 0..K_b-1
// A request whose depth or temperature is invalid contributes no rows.
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool temp_ok(float T)
{
    return T == 0.0f || (T >= 1e-6f && T <= 1e6f);   // excludes NaN, < 0, inf
}

struct Plan {
    int *row_off;   // [B + 1] in LDS
    int *info;      // [B] in LDS: d | kind << 16
    float *T;       // [B] in LDS
};

__device__ void make_plan(const Params &P, Plan pl, int *scan_tmp)
{
    const int B = P.B, K = P.K;
    const int per = (int)ceil_div(B, WG);
    const int b0 = threadIdx.x * per;
    int local = 0;
    for (int j = 0; j < per; ++j) {
        int b = b0 + j;
        if (b >= B) break;
        int d, kind, rows;
        float T = 0.0f;
        if (P.mode == MODE_CONF) {
            d = P.max_depth ? P.max_depth[b] : K;
            bool ok = d >= 0 && d <= K;
            kind = ok ? KIND_CONF : KIND_BAD;
            rows = ok ? d : 0;
        } else {
            d = P.depth ? P.depth[b] : K;
            T = (P.mode == MODE_SAMPLE) ? P.temperature[b] : 0.0f;
            bool ok = d >= 0 && d <= K && temp_ok(T);
            kind = !ok ? KIND_BAD : (T > 0.0f ? KIND_SAMPLED : KIND_GREEDY);
            rows = !ok ? 0 : (kind == KIND_SAMPLED ? 2 * d : d + 1);
        }
        if (kind == KIND_BAD) d = 0;
        pl.info[b] = d | (kind << 16);
        pl.T[b] = T;
        pl.row_off[b] = rows;    // count for now
        local += rows;
    }
    // exclusive scan of the per-thread totals
    int v = local;
    int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    if (lane == 63) scan_tmp[wave_id()] = v;
    __syncthreads();
    int wave_base = 0;
    for (int w = 0; w < wave_id(); ++w) wave_base += scan_tmp[w];
    int run = wave_base + v - local;
    for (int j = 0; j < per; ++j) {
        int b = b0 + j;
        if (b >= B) break;
        int c = pl.row_off[b];
        pl.row_off[b] = run;
        run += c;
    }
    if (threadIdx.x == WG - 1) pl.row_off[B] = run;
    __syncthreads();
}

// request containing global active row r (row_off is non-decreasing)
__device__ __forceinline__ int find_request(const int *row_off, int B, int r)
{
    int lo = 0, hi = B;   // row_off[lo] <= r < row_off[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (row_off[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Row-pass chunk reductions.  A chunk of a row is the 16-byte vectors
// [vbeg, vbeg + U*WG) of the row's vector grid; thread t reads vectors
// vbeg + j*WG + t, j < U, so each wave load is one contiguous 1 KiB.  The
// vector grid starts at the row's first element rounded down to 16 bytes;
// `head` elements of the first vector belong to the previous row and are
// masked, as are elements past the row end.
// ---------------------------------------------------------------------------

template <bool BF16>
struct RowView {
    static constexpr int EPV = BF16 ? 8 : 4;
    const uint4 *vec;   // 16-byte aligned start of the vector grid
    int head;           // elements of vector 0 before the row start
    int64_t nvec;       // vectors covering the row
    int V;

    __device__ RowView(const void *row_start, int V_) : V(V_)
    {
        uintptr_t a = (uintptr_t)row_start;
        uintptr_t a0 = a & ~uintptr_t(15);
        vec = (const uint4 *)a0;
        head = (int)((a - a0) / (BF16 ? 2 : 4));
        nvec = ceil_div((int64_t)head + V, EPV);
    }
    // element index (within the row) of element e of vector vi
    __device__ __forceinline__ int64_t elem(int64_t vi, int e) const { return vi * EPV + e - head; }
    __device__ __forceinline__ bool edge(int64_t vi) const
    {
        return vi * EPV < head || (vi + 1) * EPV - head > V;
    }
};

// Greedy row chunk: largest value and its lowest index; NaN flagged.
template <bool BF16>
__device__ void chunk_argmax(const RowView<BF16> &rv, int64_t vbeg, int U, float &best, int &bidx, int &nanf)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const uint32_t NEG = BF16 ? 0xff80ff80u : 0xff800000u;
    uint4 raw[UMAX];
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        int64_t vi = vbeg + (int64_t)j * WG + threadIdx.x;
        if (j < U && vi < rv.nvec) raw[j] = rv.vec[vi];
        else raw[j] = make_uint4(NEG, NEG, NEG, NEG);
    }
    best = -INFINITY;
    int bj = -1;
    uint4 bvec = make_uint4(NEG, NEG, NEG, NEG);
    int un = 0;
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        int64_t vi = vbeg + (int64_t)j * WG + threadIdx.x;
        float f[EPV];
        unpack<BF16>(raw[j], f);
        if (rv.edge(vi)) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                int64_t x = rv.elem(vi, e);
                if (x < 0 || x >= rv.V) f[e] = -INFINITY;
            }
        }
#pragma unroll
        for (int e = 0; e < EPV; e += 2) un |= __builtin_isunordered(f[e], f[e + 1]);
        float m = f[0];
#pragma unroll
        for (int e = 1; e < EPV; ++e) m = fmaxf(m, f[e]);
        if (m > best) { best = m; bj = j; bvec = raw[j]; }
    }
    nanf = un;
    bidx = 0x7fffffff;
    if (bj >= 0) {
        int64_t vi = vbeg + (int64_t)bj * WG + threadIdx.x;
        float f[EPV];
        unpack<BF16>(bvec, f);
        int found = -1;
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e) {
            int64_t x = rv.elem(vi, e);
            if (x >= 0 && x < rv.V && f[e] == best) found = e;
        }
        if (found >= 0) bidx = (int)rv.elem(vi, found);
    }
}

// Sampled / confidence row chunk: thread max m and s = sum exp2((v-m)*c),
// with c = log2(e)/T rounded to fp32 (c32).  The per-element exponent is one
// FMA, v*c32 - fl(m*c32); its constant offset fl(m*c32) - m*c32 is exact
// (FMA residual) and is removed from the sum in double.  Terms are summed in
// fp32 per vector (a short tree) and the vector sums in double.
template <bool BF16>
__device__ void chunk_lse(const RowView<BF16> &rv, int64_t vbeg, int U, float c32, float &m_out, double &s_out)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const uint32_t NEG = BF16 ? 0xff80ff80u : 0xff800000u;
    uint4 raw[UMAX];
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        int64_t vi = vbeg + (int64_t)j * WG + threadIdx.x;
        if (j < U && vi < rv.nvec) raw[j] = rv.vec[vi];
        else raw[j] = make_uint4(NEG, NEG, NEG, NEG);
    }
    float f[UMAX][EPV];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        int64_t vi = vbeg + (int64_t)j * WG + threadIdx.x;
        unpack<BF16>(raw[j], f[j]);
        if (rv.edge(vi)) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                int64_t x = rv.elem(vi, e);
                if (x < 0 || x >= rv.V) f[j][e] = -INFINITY;
            }
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) m = fmaxf(m, f[j][e]);
    }
    m_out = m;
    if (m == -INFINITY) {   // nothing but -inf / masked in this thread
        // a NaN still has to poison the sum
        int un = 0;
#pragma unroll
        for (int j = 0; j < UMAX; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) un |= (f[j][e] != f[j][e]);
        s_out = un ? (double)NAN : 0.0;
        return;
    }
    const float mc = m * c32;
    const float delta = __builtin_fmaf(m, c32, -mc);   // exact: m*c32 - fl(m*c32)
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        float t[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) t[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[j][e], c32, -mc));
#pragma unroll
        for (int w = EPV / 2; w > 0; w >>= 1)
#pragma unroll
            for (int e = 0; e < w; ++e) t[e] += t[e + w];
        s += (double)t[0];
    }
    // the exponents above are (v - m)*c32 + delta; take delta back out
    s_out = s * exp2(-(double)delta);
}

// Merge (m_i, s_i) pairs of log-sum-exp partials into (M, S); s_i is relative
// to m_i with exponent scale c.  Unusable partials (NaN) poison S.
__device__ __forceinline__ double lse_rescale(float m_i, double s_i, float M, double cd)
{
    if (m_i == -INFINITY) return (s_i != s_i) ? s_i : 0.0;
    return s_i * exp2(((double)m_i - (double)M) * cd);
}

// ---------------------------------------------------------------------------
// Per-request accept test and first-rejection scan (one wave, lanes over the
// drafted positions).
// ---------------------------------------------------------------------------

__device__ void mark_bad_request(const Params &P, int b)
{
    const int K = P.K;
    for (int k = lane_id(); k <= K; k += 64) P.out_tokens[(int64_t)b * (K + 1) + k] = -1;
    if (P.mode == MODE_SAMPLE) {
        for (int k = lane_id(); k < K; k += 64) {
            if (P.p_draft) P.p_draft[(int64_t)b * K + k] = 0.0f;
            if (P.q_draft) P.q_draft[(int64_t)b * K + k] = 0.0f;
        }
    }
    if (lane_id() == 0) P.num_accepted[b] = -1;
}

// Unusable row statistics: NaN or +inf present (m = NaN or +inf), nothing
// but -inf (m = -inf), or a normaliser that is not a positive finite number.
__device__ __forceinline__ bool stat_bad(const Stat &s, bool lse)
{
    if (!(s.m == s.m) || s.m == INFINITY || s.m == -INFINITY) return true;
    if (lse) return !(s.s > 0.0) || s.s == (double)INFINITY;
    return false;
}

__device__ __forceinline__ bool unif_ok(float u) { return u >= 0.0f && u < 1.0f; }

// One full wave.  rowbase = first active row of request b in the plan.
__device__ void scan_request(const Params &P, int b, int d, int kind, float T, int rowbase)
{
    const int K = P.K;
    const int lane = lane_id();
    const int64_t ob = (int64_t)b * (K + 1);
    const int64_t tb = (int64_t)b * K;
    ReqDesc desc = {SREQ_NONE, 0, 0, T};

    if (kind == KIND_BAD) {
        mark_bad_request(P, b);
        if (P.mode == MODE_SAMPLE && lane == 0) P.ws.req[b] = desc;
        return;
    }
    const Stat *rows = P.ws.rows + rowbase;

    if (kind == KIND_GREEDY) {
        // accept k iff x_k == argmax of target row k; emit argmax of row n
        int n = d;
        int bad = 0;
        for (int k0 = 0; k0 <= d; k0 += 64) {
            const int k = k0 + lane;
            bool mism = false;
            if (k <= d) {
                const Stat s = rows[k];
                bad |= stat_bad(s, false);
                if (k < d) {
                    const int x = P.tokens[tb + k];
                    bad |= (x < 0 || x >= P.V);
                    mism = (x != s.idx);
                }
            }
            const uint64_t mm = __ballot(mism);
            if (mm && n == d) n = k0 + __builtin_ctzll(mm);
        }
        bad = wave_or(bad);
        if (bad) {
            mark_bad_request(P, b);
        } else {
            const int emit = rows[n].idx;
            for (int k = lane; k <= K; k += 64)
                P.out_tokens[ob + k] = (k < n) ? P.tokens[tb + k] : (k == n ? emit : -1);
            if (P.mode == MODE_SAMPLE) {
                for (int k = lane; k < K; k += 64) {
                    if (P.p_draft) P.p_draft[tb + k] = 0.0f;
                    if (P.q_draft) P.q_draft[tb + k] = 0.0f;
                }
            }
            if (lane == 0) P.num_accepted[b] = n;
        }
        if (P.mode == MODE_SAMPLE && lane == 0) P.ws.req[b] = desc;
        return;
    }

    // Sampled request (T > 0): target rows 0..d-1, then draft rows 0..d-1.
    // accept k iff u_k < min(1, p_k(x)/q_k(x)), evaluated in double from the
    // row statistics and the two logits at x.
    int bad = unif_ok(P.u_sample[b]) ? 0 : 1;
    int n = d;
    const double Td = (double)T;
    const int64_t V = P.V;
    for (int k0 = 0; k0 < d; k0 += 64) {
        const int k = k0 + lane;
        const bool active = k < d;
        bool rej = false;
        if (active) {
            const int x = P.tokens[tb + k];
            const float ua = P.u_accept[tb + k];
            const Stat st = rows[k], sd = rows[d + k];
            const bool lb = (x < 0 || x >= P.V) || !unif_ok(ua) || stat_bad(st, true) || stat_bad(sd, true);
            double a = 0.0, c = 0.0;
            if (!lb) {
                const float zx = load_logit_dt(P.target, P.bf16, ((int64_t)b * (K + 1) + k) * V + x);
                const float yx = load_logit_dt(P.draft, P.bf16, (tb + k) * V + x);
                a = exp(((double)zx - (double)st.m) / Td) / st.s;
                c = exp(((double)yx - (double)sd.m) / Td) / sd.s;
                const double ratio = (c > 0.0) ? fmin(1.0, a / c) : (a > 0.0 ? 1.0 : 0.0);
                rej = !((double)ua < ratio);
            }
            bad |= lb;
            if (P.p_draft) P.p_draft[tb + k] = (float)a;
            if (P.q_draft) P.q_draft[tb + k] = (float)c;
        }
        const uint64_t rm = __ballot(active && rej);
        if (rm && n == d) n = k0 + __builtin_ctzll(rm);
    }
    bad = wave_or(bad);
    if (bad) {
        mark_bad_request(P, b);
        if (lane == 0) P.ws.req[b] = desc;
        return;
    }
    for (int k = d + lane; k < K; k += 64) {
        if (P.p_draft) P.p_draft[tb + k] = 0.0f;
        if (P.q_draft) P.q_draft[tb + k] = 0.0f;
    }
    // the emitted token at position n is written by the sampler
    for (int k = lane; k <= K; k += 64) P.out_tokens[ob + k] = (k < n) ? P.tokens[tb + k] : -1;
    if (lane == 0) {
        P.num_accepted[b] = n;
        desc.state = (n == d) ? SREQ_BONUS : SREQ_RESID;
        desc.n = n;
        P.ws.req[b] = desc;
    }
}

// ---------------------------------------------------------------------------
// Row pass
// ---------------------------------------------------------------------------

template <bool BF16>
__device__ void row_task(const Params &P, const Plan &pl, RedSmem &sm, int r, int c, int cpr, int U)
{
    const int B = P.B, K = P.K, V = P.V;
    const int b = find_request(pl.row_off, B, r);
    const int local = r - pl.row_off[b];
    const int info = pl.info[b];
    const int d = info & 0xffff, kind = info >> 16;
    const float T = pl.T[b];

    bool is_draft, lse;
    int k;
    if (kind == KIND_GREEDY) { is_draft = false; k = local; lse = false; }
    else if (kind == KIND_SAMPLED) { is_draft = local >= d; k = is_draft ? local - d : local; lse = true; }
    else { is_draft = true; k = local; lse = true; }   // KIND_CONF
    const int64_t row = is_draft ? ((int64_t)b * K + k) : ((int64_t)b * (K + 1) + k);
    const char *row_start = (const char *)(is_draft ? P.draft : P.target) + row * (int64_t)V * (BF16 ? 2 : 4);
    const RowView<BF16> rv(row_start, V);
    const int64_t vbeg = (int64_t)c * U * WG;

    const double cd = LOG2E / (double)(kind == KIND_CONF ? 1.0f : T);
    Stat st;
    if (!lse) {
        float best;
        int bidx, nanf;
        chunk_argmax<BF16>(rv, vbeg, U, best, bidx, nanf);
        nanf = wg_or(nanf, sm);
        wg_argmax(best, bidx, sm);
        st.m = nanf ? NAN : best;
        st.idx = bidx;
        st.s = 0.0;
    } else {
        float m;
        double s;
        chunk_lse<BF16>(rv, vbeg, U, (float)cd, m, s);
        const float M = wg_max(m, sm);
        const double S = wg_sum(lse_rescale(m, s, M, cd), sm);
        st.m = M;
        st.idx = 0;
        st.s = S;
    }

    __shared__ int sh_last;
    if (cpr > 1) {
        if (threadIdx.x == 0) {
            P.ws.part[(int64_t)r * P.cpr_max + c] = st;
            fence_release();
            const uint32_t old = atomic_inc_agent(&P.ws.row_cnt[r]);
            sh_last = (old == (uint32_t)(cpr - 1));
        }
        __syncthreads();
        const int last = sh_last;
        __syncthreads();
        if (!last) return;
        if (wave_id() != 0) return;
        // merge the chunk partials of row r (wave 0)
        fence_acquire();
        const Stat *pp = P.ws.part + (int64_t)r * P.cpr_max;
        if (!lse) {
            float m = -INFINITY;
            int i = 0x7fffffff, nanf = 0;
            for (int j = lane_id(); j < cpr; j += 64) {
                const Stat s = pp[j];
                if (!(s.m == s.m)) nanf = 1;
                else argmax_merge(m, i, s.m, s.idx);
            }
            wave_argmax(m, i);
            nanf = wave_or(nanf);
            st.m = nanf ? NAN : m;
            st.idx = i;
            st.s = 0.0;
        } else {
            float M = -INFINITY;
            for (int j = lane_id(); j < cpr; j += 64) M = fmaxf(M, pp[j].m);
            M = wave_max(M);
            double S = 0.0;
            for (int j = lane_id(); j < cpr; j += 64) S += lse_rescale(pp[j].m, pp[j].s, M, cd);
            st.m = M;
            st.idx = 0;
            st.s = wave_sum(S);
        }
        if (lane_id() == 0) {
            P.ws.rows[r] = st;
            store_zero_agent(&P.ws.row_cnt[r]);
        }
    } else {
        if (wave_id() != 0) return;
        if (lane_id() == 0) P.ws.rows[r] = st;
    }

    // Row r is complete (wave 0 only from here on).
    if (kind == KIND_CONF) {
        if (lane_id() == 0)
            P.conf[(int64_t)b * K + k] = stat_bad(st, true) ? NAN : (float)(1.0 / st.s);
        return;
    }
    const int nrows = pl.row_off[b + 1] - pl.row_off[b];
    int lastreq = 0;
    if (lane_id() == 0) {
        fence_release();
        const uint32_t old = atomic_inc_agent(&P.ws.req_cnt[b]);
        lastreq = (old == (uint32_t)(nrows - 1));
    }
    lastreq = __shfl(lastreq, 0, 64);
    if (!lastreq) return;
    fence_acquire();
    if (lane_id() == 0) store_zero_agent(&P.ws.req_cnt[b]);
    scan_request(P, b, d, kind, T, pl.row_off[b]);
}

template <bool BF16>
__global__ __launch_bounds__(WG) void row_stats_kernel(Params P)
{
    extern __shared__ int plan_smem[];
    __shared__ RedSmem sm;
    __shared__ int scan_tmp[NWAVE];
    Plan pl;
    pl.row_off = plan_smem;
    pl.info = plan_smem + P.B + 1;
    pl.T = (float *)(plan_smem + 2 * P.B + 1);
    make_plan(P, pl, scan_tmp);

    const int B = P.B, K = P.K;
    const int R = pl.row_off[B];

    // Requests with no rows in the pass (bad plan, sampled with depth 0,
    // confidence with K_b = 0) and confidence entries beyond K_b are
    // finished here by workgroup 0.
    if (blockIdx.x == 0 && wave_id() == 0) {
        for (int b = 0; b < B; ++b) {
            const int info = pl.info[b];
            const int d = info & 0xffff, kind = info >> 16;
            if (P.mode == MODE_CONF) {
                for (int k = lane_id(); k < K; k += 64)
                    if (kind == KIND_BAD || k >= d) P.conf[(int64_t)b * K + k] = (kind == KIND_BAD) ? NAN : 0.0f;
            } else if (pl.row_off[b + 1] == pl.row_off[b]) {
                scan_request(P, b, d, kind, pl.T[b], pl.row_off[b]);
            }
        }
    }

    // Chunking: 16-byte loads per thread U in {8,4,2,1}; smaller when the
    // batch has too few rows to give every workgroup two tasks.
    constexpr int EPV = BF16 ? 8 : 4;
    const int64_t nv = nvec_max(P.V, EPV);
    const int u_lo = (int)ceil_div(nv, (int64_t)WG * CPR_CAP);
    int U = UMAX;
    while (U > 1 && U > u_lo && (int64_t)R * ceil_div(nv, (int64_t)WG * U) < 2 * (int64_t)gridDim.x) U >>= 1;
    if (U < u_lo) U = u_lo;
    const int cpr = (int)ceil_div(nv, (int64_t)WG * U);
    const int64_t ntask = (int64_t)R * cpr;
    for (int64_t t = blockIdx.x; t < ntask; t += gridDim.x) {
        const int r = (int)(t / cpr);
        const int c = (int)(t - (int64_t)r * cpr);
        row_task<BF16>(P, pl, sm, r, c, cpr, U);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Sampler.  A sampled request draws one token from one row pair: after a
// rejection at n, r = max(0, p_n - q_n); without one, r = p_d.  Both kernels
// split that row pair into chunks of US*WG vectors, one workgroup each, and
// work in fp64 throughout (terms, sums, prefix scan): the draw compares u*R
// against prefix sums over V terms, and fp32 terms would move the result
// for about one draw in a thousand.
// ---------------------------------------------------------------------------

template <bool BF16>
__device__ __forceinline__ void load_sampler_chunk(const RowView<BF16> &rv, int64_t vbeg, float (&f)[US][RowView<BF16>::EPV], int &flag)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const uint32_t NEG = BF16 ? 0xff80ff80u : 0xff800000u;
#pragma unroll
    for (int j = 0; j < US; ++j) {
        const int64_t vi = vbeg + (int64_t)j * WG + threadIdx.x;
        const uint4 raw = (vi < rv.nvec) ? rv.vec[vi] : make_uint4(NEG, NEG, NEG, NEG);
        unpack<BF16>(raw, f[j]);
        if (rv.edge(vi)) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int64_t x = rv.elem(vi, e);
                if (x < 0 || x >= rv.V) f[j][e] = -INFINITY;
            }
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) flag |= (!(f[j][e] == f[j][e]) || f[j][e] == INFINITY);
    }
}

template <bool BF16>
__global__ __launch_bounds__(WG) void sampler_sums_kernel(Params P)
{
    constexpr int EPV = RowView<BF16>::EPV;
    __shared__ RedSmem sm;
    __shared__ int sh_last;
    const int b = blockIdx.y, c = blockIdx.x;
    const ReqDesc desc = P.ws.req[b];
    if (desc.state == SREQ_NONE) return;
    const bool resid = desc.state == SREQ_RESID;
    const int K = P.K, V = P.V;
    const int64_t esz = BF16 ? 2 : 4;
    const double invT = 1.0 / (double)desc.T;
    const RowView<BF16> rz((const char *)P.target + ((int64_t)b * (K + 1) + desc.n) * V * esz, V);
    const int64_t vbeg = (int64_t)c * US * WG;

    int flag = 0;
    float f[US][EPV];
    load_sampler_chunk<BF16>(rz, vbeg, f, flag);
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < US; ++j)
#pragma unroll
        for (int e = 0; e < EPV; ++e) m = fmaxf(m, f[j][e]);
    const float mz = wg_max(m, sm);
    double s = 0.0;
    if (mz != -INFINITY && mz != INFINITY) {
#pragma unroll
        for (int j = 0; j < US; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) s += exp(((double)f[j][e] - (double)mz) * invT);
    }
    const double sz = wg_sum(s, sm);
    float my = 0.0f;
    double sy = 0.0;
    if (resid) {
        const RowView<BF16> ry((const char *)P.draft + ((int64_t)b * K + desc.n) * V * esz, V);
        int fy = 0;
        load_sampler_chunk<BF16>(ry, vbeg, f, fy);
        m = -INFINITY;
#pragma unroll
        for (int j = 0; j < US; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) m = fmaxf(m, f[j][e]);
        my = wg_max(m, sm);
        s = 0.0;
        if (my != -INFINITY && my != INFINITY) {
#pragma unroll
            for (int j = 0; j < US; ++j)
#pragma unroll
                for (int e = 0; e < EPV; ++e) s += exp(((double)f[j][e] - (double)my) * invT);
        }
        sy = wg_sum(s, sm);
    }
    flag = wg_or(flag, sm);

    if (threadIdx.x == 0) {
        S1Part part = {mz, my, flag, 0, sz, sy};
        P.ws.s1[(int64_t)b * P.cs + c] = part;
        fence_release();
        const uint32_t old = atomic_inc_agent(&P.ws.s1cnt[b]);
        sh_last = (old == (uint32_t)(P.cs - 1));
    }
    __syncthreads();
    if (!sh_last || wave_id() != 0) return;
    fence_acquire();
    const S1Part *pp = P.ws.s1 + (int64_t)b * P.cs;
    float Mz = -INFINITY, My = -INFINITY;
    int bad = 0;
    for (int j = lane_id(); j < P.cs; j += 64) {
        const S1Part q = pp[j];
        Mz = fmaxf(Mz, q.mz);
        My = fmaxf(My, q.my);
        bad |= q.bad;
    }
    Mz = wave_max(Mz);
    My = wave_max(My);
    double Sz = 0.0, Sy = 0.0;
    for (int j = lane_id(); j < P.cs; j += 64) {
        const S1Part q = pp[j];
        if (q.mz != -INFINITY) Sz += q.sz * exp(((double)q.mz - (double)Mz) * invT);
        if (resid && q.my != -INFINITY) Sy += q.sy * exp(((double)q.my - (double)My) * invT);
    }
    Sz = wave_sum(Sz);
    Sy = wave_sum(Sy);
    bad = wave_or(bad);
    // only the bonus row is new to this call; residual rows were checked in
    // the row pass, so `bad` can only come from target row d
    bad |= (Mz == -INFINITY || Mz == INFINITY || !(Sz > 0.0));
    if (resid) bad |= (My == -INFINITY || My == INFINITY || !(Sy > 0.0));
    if (lane_id() == 0) {
        S1Part tot = {Mz, My, bad, 0, Sz, Sy};
        P.ws.s1tot[b] = tot;
        store_zero_agent(&P.ws.s1cnt[b]);
    }
    if (bad) mark_bad_request(P, b);
}

// Exclusive scan of one double per thread over the workgroup, in thread order.
__device__ double wg_excl_scan(double v, double *sm4, double &total)
{
    const int lane = lane_id();
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == 63) sm4[wave_id()] = incl;
    __syncthreads();
    double wb = 0.0, tot = 0.0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
        if (w < wave_id()) wb += sm4[w];
        tot += sm4[w];
    }
    total = tot;
    return wb + excl;
}

// Sampler terms of one chunk, in fp64.  which: 0 = residual max(0, p - q),
// 1 = target distribution p.  Values are written per (slot j, element e).
template <bool BF16>
__device__ void sampler_terms(const Params &P, int b, const ReqDesc &desc, const S1Part &tot, int64_t vbeg,
                              int which, double (&val)[US][RowView<BF16>::EPV])
{
    constexpr int EPV = RowView<BF16>::EPV;
    const int K = P.K, V = P.V;
    const int64_t esz = BF16 ? 2 : 4;
    const double invT = 1.0 / (double)desc.T;
    const double invSz = 1.0 / tot.sz;
    int flag = 0;
    float f[US][EPV];
    const RowView<BF16> rz((const char *)P.target + ((int64_t)b * (K + 1) + desc.n) * V * esz, V);
    load_sampler_chunk<BF16>(rz, vbeg, f, flag);
#pragma unroll
    for (int j = 0; j < US; ++j)
#pragma unroll
        for (int e = 0; e < EPV; ++e) val[j][e] = exp(((double)f[j][e] - (double)tot.mz) * invT) * invSz;
    if (which == 0) {
        const double invSy = 1.0 / tot.sy;
        const RowView<BF16> ry((const char *)P.draft + ((int64_t)b * K + desc.n) * V * esz, V);
        load_sampler_chunk<BF16>(ry, vbeg, f, flag);
#pragma unroll
        for (int j = 0; j < US; ++j)
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const double q = exp(((double)f[j][e] - (double)tot.my) * invT) * invSy;
                const double dlt = val[j][e] - q;
                val[j][e] = dlt > 0.0 ? dlt : 0.0;
            }
    }
}

template <bool BF16>
__global__ __launch_bounds__(WG) void sampler_draw_kernel(Params P)
{
    constexpr int EPV = RowView<BF16>::EPV;
    constexpr int CS_LDS = 512;
    __shared__ double sm4[NWAVE];
    __shared__ int sh_last;
    __shared__ S2Part parts[CS_LDS];
    __shared__ double sh_base, sh_target;
    __shared__ int sh_c, sh_which, sh_over;
    __shared__ RedSmem sm;
    const int b = blockIdx.y, c = blockIdx.x;
    const ReqDesc desc = P.ws.req[b];
    if (desc.state == SREQ_NONE) return;
    const S1Part tot = P.ws.s1tot[b];
    if (tot.bad) return;
    const bool resid = desc.state == SREQ_RESID;
    const int64_t vbeg_own = (int64_t)c * US * WG;

    // chunk totals of r (and of p, for the all-zero-residual fallback)
    double val[US][EPV];
    double total_r = 0.0, total_p = 0.0;
    {
        sampler_terms<BF16>(P, b, desc, tot, vbeg_own, resid ? 0 : 1, val);
        double carry = 0.0;
#pragma unroll
        for (int j = 0; j < US; ++j) {
            double vs = 0.0;
#pragma unroll
            for (int e = 0; e < EPV; ++e) vs += val[j][e];
            double t;
            (void)wg_excl_scan(vs, sm4, t);
            carry += t;
        }
        total_r = carry;
    }
    if (resid) {
        sampler_terms<BF16>(P, b, desc, tot, vbeg_own, 1, val);
        double carry = 0.0;
#pragma unroll
        for (int j = 0; j < US; ++j) {
            double vs = 0.0;
#pragma unroll
            for (int e = 0; e < EPV; ++e) vs += val[j][e];
            double t;
            (void)wg_excl_scan(vs, sm4, t);
            carry += t;
        }
        total_p = carry;
    }
    if (threadIdx.x == 0) {
        S2Part part = {total_r, total_p};
        P.ws.s2[(int64_t)b * P.cs + c] = part;
        fence_release();
        const uint32_t old = atomic_inc_agent(&P.ws.s2cnt[b]);
        sh_last = (old == (uint32_t)(P.cs - 1));
    }
    __syncthreads();
    if (!sh_last) return;
    fence_acquire();

    // Last chunk of request b: locate u*R among the chunk totals.
    for (int j = threadIdx.x; j < P.cs; j += WG) parts[j] = P.ws.s2[(int64_t)b * P.cs + j];
    __syncthreads();
    if (threadIdx.x == 0) {
        double R = 0.0;
        for (int j = 0; j < P.cs; ++j) R += parts[j].r;
        int which = resid ? 0 : 1;
        if (resid && R == 0.0) {   // no residual mass: fall back to p
            which = 1;
            R = 0.0;
            for (int j = 0; j < P.cs; ++j) R += parts[j].p;
        }
        const double target = (double)P.u_sample[b] * R;
        double cum = 0.0, base = 0.0;
        int cstar = -1, lastpos = -1;
        for (int j = 0; j < P.cs; ++j) {
            const double t = which == 0 ? parts[j].r : parts[j].p;
            if (t > 0.0) lastpos = j;
            const double nc = cum + t;
            if (cstar < 0 && nc > target) { cstar = j; base = cum; }
            cum = nc;
        }
        sh_over = cstar < 0;
        sh_c = cstar < 0 ? lastpos : cstar;
        sh_base = base;
        sh_target = target;
        sh_which = which;
    }
    __syncthreads();
    const int cs = sh_c;
    if (cs < 0) {   // no chunk holds positive mass (unreachable for valid statistics)
        if (threadIdx.x < 64) mark_bad_request(P, b);
        if (threadIdx.x == 0) store_zero_agent(&P.ws.s2cnt[b]);
        return;
    }
    const double base = sh_base, target = sh_target;
    const int which = sh_which;
    const bool over = sh_over;
    const int64_t vbeg = (int64_t)cs * US * WG;

    // Rescan chunk cs: first positive-mass element whose prefix exceeds
    // u*R; the chunk's last positive-mass element if none does.
    sampler_terms<BF16>(P, b, desc, tot, vbeg, which, val);
    const RowView<BF16> rz((const char *)P.target + ((int64_t)b * (P.K + 1) + desc.n) * P.V * (BF16 ? 2 : 4), P.V);
    int first = 0x7fffffff, lastp = -1;
    double carry = 0.0;
#pragma unroll
    for (int j = 0; j < US; ++j) {
        double vs = 0.0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) vs += val[j][e];
        double t;
        const double ex = wg_excl_scan(vs, sm4, t);
        const double slot0 = carry + ex;
        const int64_t vi = vbeg + (int64_t)j * WG + threadIdx.x;
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            part += val[j][e];
            const int64_t x = rz.elem(vi, e);
            if (val[j][e] > 0.0 && x >= 0 && x < P.V) {
                if (x > lastp) lastp = (int)x;
                if (first == 0x7fffffff && base + (slot0 + part) > target) first = (int)x;
            }
        }
        carry += t;
    }
    // workgroup min of `first`, max of `lastp`
    float dummy = 0.0f;
    int fi = first;
    {
        // min via argmax merge on negated index
        float m = (fi == 0x7fffffff) ? -INFINITY : 0.0f;
        int i = fi;
        (void)dummy;
        wg_argmax(m, i, sm);
        fi = (m == -INFINITY) ? 0x7fffffff : i;
    }
    int lp;
    {
        float m = (lastp < 0) ? -INFINITY : 0.0f;
        int i = (lastp < 0) ? 0x7fffffff : (0x7fffffff - lastp);
        wg_argmax(m, i, sm);
        lp = (m == -INFINITY) ? -1 : (0x7fffffff - i);
    }
    if (threadIdx.x == 0) {
        const int tok = (!over && fi != 0x7fffffff) ? fi : lp;
        P.out_tokens[(int64_t)b * (P.K + 1) + desc.n] = tok;
        store_zero_agent(&P.ws.s2cnt[b]);
    }
}

// ---------------------------------------------------------------------------
// D-cut allocation: one workgroup of 1024 threads; keys in LDS.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float sanitize_conf(float c)
{
    if (!(c > 0.0f)) return 0.0f;
    return c > 1.0f ? 1.0f : c;
}

__device__ int block_sum_int(int v, int *sm32)
{
    v = __reduce_add_sync(0xffffffffffffffffull, v);
    __syncthreads();
    if (lane_id() == 0) sm32[wave_id()] = v;
    __syncthreads();
    int t = 0;
    for (int w = 0; w < DCUT_WG / 64; ++w) t += sm32[w];
    __syncthreads();
    return t;
}

__device__ int block_excl_scan_int(int v, int *sm32)
{
    const int lane = lane_id();
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) sm32[wave_id()] = incl;
    __syncthreads();
    int wb = 0;
    for (int w = 0; w < wave_id(); ++w) wb += sm32[w];
    __syncthreads();
    return wb + incl - v;
}

__global__ __launch_bounds__(DCUT_WG) void dcut_kernel(const float *conf, const int32_t *max_depth, int B, int K,
                                                      int budget, int32_t *depth_out)
{
    extern __shared__ uint32_t keys[];   // [B*K]: 0 = not a candidate, else float bits of c + 1
    __shared__ int hist[256];
    __shared__ int sm32[DCUT_WG / 64];
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_kr;
    const int per = (int)ceil_div(B, DCUT_WG);
    const int b0 = threadIdx.x * per;
    int floors = 0, cands = 0;
    for (int j = 0; j < per; ++j) {
        const int b = b0 + j;
        if (b >= B) break;
        const int Kb = max_depth ? max_depth[b] : K;
        const bool valid = Kb >= 0 && Kb <= K;
        float c = 0.0f;
        for (int k = 0; k < K; ++k) {
            uint32_t key = 0;
            if (valid && k < Kb) {
                const float s = sanitize_conf(conf[(int64_t)b * K + k]);
                c = (k == 0) ? s : c * s;
                if (k >= 1) key = __float_as_uint(c) + 1u;
            }
            keys[(int64_t)b * K + k] = key;
        }
        if (valid) {
            floors += Kb > 0 ? 1 : 0;
            cands += Kb > 1 ? Kb - 1 : 0;
        }
    }
    floors = block_sum_int(floors, sm32);
    cands = block_sum_int(cands, sm32);
    int take = budget - floors;
    if (take > cands) take = cands;
    if (take < 0) take = 0;

    // radix select of the take-th largest key, 8 bits at a time
    uint32_t prefix = 0;
    int kr = take;
    if (take > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = threadIdx.x; i < 256; i += DCUT_WG) hist[i] = 0;
            __syncthreads();
            const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
            for (int j = 0; j < per * K; ++j) {
                const int64_t fi = (int64_t)b0 * K + j;
                if (fi >= (int64_t)B * K) break;
                const uint32_t key = keys[fi];
                if (key != 0 && (key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 255u], 1);
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                int acc = 0, digit = 0;
                for (int bin = 255; bin >= 0; --bin) {
                    if (acc + hist[bin] >= kr) { digit = bin; break; }
                    acc += hist[bin];
                }
                sh_kr = kr - acc;
                sh_prefix = prefix | ((uint32_t)digit << shift);
            }
            __syncthreads();
            prefix = sh_prefix;
            kr = sh_kr;
            __syncthreads();
        }
    }
    // entries above the threshold are taken; ties at the threshold go in
    // flat-index order (threads own contiguous flat ranges)
    const uint32_t thr = (take > 0) ? prefix : 0xffffffffu;
    int eq = 0;
    for (int j = 0; j < per * K; ++j) {
        const int64_t fi = (int64_t)b0 * K + j;
        if (fi >= (int64_t)B * K) break;
        eq += (keys[fi] == thr && take > 0);
    }
    int rank = block_excl_scan_int(eq, sm32);
    for (int j = 0; j < per; ++j) {
        const int b = b0 + j;
        if (b >= B) break;
        const int Kb = max_depth ? max_depth[b] : K;
        const bool valid = Kb >= 0 && Kb <= K;
        int dep = valid ? (Kb > 0 ? 1 : 0) : -1;
        for (int k = 0; k < K; ++k) {
            const uint32_t key = keys[(int64_t)b * K + k];
            if (key == 0 || take == 0) continue;
            if (key > thr) ++dep;
            else if (key == thr) {
                if (rank < kr) ++dep;
                ++rank;
            }
        }
        depth_out[b] = dep;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

constexpr int MAX_DEVICES = 64;
std::atomic<int> g_cu_count[MAX_DEVICES];

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of the persistent row pass per compute unit.
int g_row_wgs_per_cu = 8;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

sv_status check_shape(int32_t B, int32_t K, int32_t V)
{
    if (B < 1 || K < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (B > B_MAX || K > K_MAX || V > V_MAX) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

sv_status check_ws(void *ws, size_t ws_bytes, const Layout &L)
{
    if (!ws || ws_bytes < L.total || ((uintptr_t)ws & 255u) != 0) return SV_ERR_WORKSPACE;
    return SV_OK;
}

sv_status launch_rows(Params &P, hipStream_t stream)
{
    const int64_t nv = nvec_max(P.V, P.bf16 ? 8 : 4);
    const int64_t rows_max = (P.mode == MODE_SAMPLE) ? (int64_t)P.B * (2 * P.K + 1)
                           : (P.mode == MODE_GREEDY) ? (int64_t)P.B * (P.K + 1) : (int64_t)P.B * P.K;
    int64_t grid = (int64_t)cu_count() * g_row_wgs_per_cu;
    grid = std::min<int64_t>(grid, std::max<int64_t>(1, rows_max * ceil_div(nv, WG)));
    const size_t lds = sizeof(int) * (size_t)(3 * P.B + 1);
    if (P.bf16) hipLaunchKernelGGL(row_stats_kernel<true>, dim3((unsigned)grid), dim3(WG), lds, stream, P);
    else hipLaunchKernelGGL(row_stats_kernel<false>, dim3((unsigned)grid), dim3(WG), lds, stream, P);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status launch_sampler(Params &P, hipStream_t stream)
{
    dim3 grid((unsigned)P.cs, (unsigned)P.B);
    if (P.bf16) {
        hipLaunchKernelGGL(sampler_sums_kernel<true>, grid, dim3(WG), 0, stream, P);
        hipLaunchKernelGGL(sampler_draw_kernel<true>, grid, dim3(WG), 0, stream, P);
    } else {
        hipLaunchKernelGGL(sampler_sums_kernel<false>, grid, dim3(WG), 0, stream, P);
        hipLaunchKernelGGL(sampler_draw_kernel<false>, grid, dim3(WG), 0, stream, P);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

Params base_params(int32_t B, int32_t K, int32_t V, sv_dtype dt, int mode, const Layout &L, void *ws)
{
    Params P;
    memset(&P, 0, sizeof P);
    P.B = B;
    P.K = K;
    P.V = V;
    P.bf16 = dt == SV_BF16;
    P.mode = mode;
    P.cpr_max = L.cpr_max;
    P.cs = (int)ceil_div(nvec_max(V, P.bf16 ? 8 : 4), (int64_t)WG * US);
    P.ws = carve(ws, L);
    return P;
}

}  // namespace

extern "C" {

int32_t spec_verify_abi_version(void) { return 1; }

const char *spec_verify_status_string(sv_status s)
{
    switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_BUDGET: return "SV_ERR_BUDGET";
    case SV_ERR_BAD_INPUT: return "SV_ERR_BAD_INPUT";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    }
    return "SV_ERR_UNKNOWN";
}

size_t spec_verify_workspace_size(int32_t B, int32_t K, int32_t V)
{
    Layout L;
    return make_layout(B, K, V, L) ? L.total : 0;
}

sv_status spec_verify_greedy(const void *target_logits, sv_dtype dt, const int32_t *draft_tokens,
                             const int32_t *depth, int32_t B, int32_t K, int32_t V, int32_t *out_tokens,
                             int32_t *num_accepted, void *workspace, size_t ws_bytes, hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!target_logits || !out_tokens || !num_accepted || (K > 0 && !draft_tokens)) return SV_ERR_INVALID_ARG;
    if (!aligned16(target_logits)) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K, V, dt, MODE_GREEDY, L, workspace);
    P.target = target_logits;
    P.tokens = draft_tokens;
    P.depth = depth;
    P.out_tokens = out_tokens;
    P.num_accepted = num_accepted;
    return launch_rows(P, stream);
}

sv_status spec_verify_sample(const void *target_logits, const void *draft_logits, sv_dtype dt,
                             const int32_t *draft_tokens, const int32_t *depth, const float *temperature,
                             const float *u_accept, const float *u_sample, int32_t B, int32_t K, int32_t V,
                             int32_t *out_tokens, int32_t *num_accepted, float *p_draft, float *q_draft,
                             void *workspace, size_t ws_bytes, hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!target_logits || !temperature || !u_sample || !out_tokens || !num_accepted) return SV_ERR_INVALID_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
    if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits))) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K, V, dt, MODE_SAMPLE, L, workspace);
    P.target = target_logits;
    P.draft = draft_logits;
    P.tokens = draft_tokens;
    P.depth = depth;
    P.temperature = temperature;
    P.u_accept = u_accept;
    P.u_sample = u_sample;
    P.out_tokens = out_tokens;
    P.num_accepted = num_accepted;
    P.p_draft = p_draft;
    P.q_draft = q_draft;
    if ((st = launch_rows(P, stream)) != SV_OK) return st;
    return launch_sampler(P, stream);
}

sv_status spec_draft_confidence(const void *draft_logits, sv_dtype dt, const int32_t *max_depth, int32_t B,
                                int32_t K, int32_t V, float *conf, void *workspace, size_t ws_bytes,
                                hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (K == 0) return SV_OK;
    if (!draft_logits || !conf) return SV_ERR_INVALID_ARG;
    if (!aligned16(draft_logits)) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K, V, dt, MODE_CONF, L, workspace);
    P.draft = draft_logits;
    P.max_depth = max_depth;
    P.conf = conf;
    return launch_rows(P, stream);
}

sv_status dcut_allocate(const float *conf, const int32_t *max_depth, int32_t B, int32_t K, int32_t budget,
                        int32_t *depth_out, hipStream_t stream)
{
    if (B < 1 || K < 0) return SV_ERR_INVALID_ARG;
    if ((int64_t)B * K > DCUT_MAX || B > B_MAX || K > K_MAX) return SV_ERR_UNSUPPORTED;
    if (!depth_out || (K > 0 && !conf)) return SV_ERR_INVALID_ARG;
    if (budget < B) return SV_ERR_BUDGET;
    const size_t lds = sizeof(uint32_t) * (size_t)std::max<int64_t>(1, (int64_t)B * K);
    static std::atomic<int> attr_set{0};
    if (!attr_set.load()) {
        if (hipFuncSetAttribute((const void *)dcut_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)(sizeof(uint32_t) * DCUT_MAX)) != hipSuccess)
            return SV_ERR_HIP;
        attr_set.store(1);
    }
    hipLaunchKernelGGL(dcut_kernel, dim3(1), dim3(DCUT_WG), lds, stream, conf, max_depth, B, K, budget, depth_out);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
