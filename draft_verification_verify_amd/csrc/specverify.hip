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
// One verification call is three kernels on the caller's stream:
//  A. row_pass_kernel -- the HBM stream.  A persistent grid of independent
//     waves; every workgroup plans the batch itself from depth[] and
//     temperature[] (no host round trip).  A wave task is one chunk of one
//     logit row, read with 16-byte nontemporal loads, double-buffered across
//     batches and across consecutive tasks, and reduced to (max, lowest
//     argmax) for greedy rows or (max, sum of exp) for sampled rows.  Each
//     task stores its partial with plain stores: no atomics, no waits.
//  B. finish_kernel -- workgroups (c, b) for request b.  Every workgroup of
//     a request merges the request's chunk partials per row and runs the
//     accept test and first-rejection scan itself (a short chain, so none
//     waits on another); workgroup 0 writes the outputs and a draw record.
//     For a request that draws a token, each wave then sums one 2048-logit
//     unit of the drawn row pair in fp64: the row normalisers and the
//     unit's residual max(0, p - q) mass (or, for a bonus draw, the unit's
//     maximum and sum of p).
//  C. draw_kernel -- one workgroup per drawing request: combines the unit
//     sums, locates u*R among the unit masses and rescans that unit in
//     token order.
// The kernel boundaries order all data between phases: no kernel of a call
// uses atomics, fences or flags to hand data to another workgroup.
// dcut_allocate is one workgroup: fp32 running products and an LDS radix
// select.  Nothing here is a dense contraction, so there is no MFMA: A is
// bound by HBM bandwidth, B by fp64 arithmetic on one row pair per request,
// C by latency.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>
#include <vector>

#include "specverify.h"

namespace {

constexpr int WG = 256;           // threads per workgroup
constexpr int NWAVE = WG / 64;    // wave64
constexpr int UW = 4;             // 16-byte loads per lane per row-pass batch
constexpr int WVEC = UW * 64;     // vectors per wave batch
constexpr int UNIT_E = 2048;      // logits of a row in one sampler unit (one wave)
constexpr int SE = 16;            // logits per lane per step of a unit
constexpr int SUB = UNIT_E / (64 * SE);   // steps per unit
constexpr int UNITS_MAX = 1024;   // sampler units per row, at most
constexpr int CPR_CAP = 256;      // chunks per row, at most
constexpr int B_MAX = 4096;
constexpr int K_MAX = 1024;
constexpr int V_MAX = 2000000;
constexpr int DCUT_MAX = 32768;   // B*K for dcut_allocate (keys held in LDS)
constexpr int DCUT_WG = 1024;
constexpr int EXP2_TAB = 512;     // table entries of the fp64 exp2
constexpr int SLOT_MAX = 4;       // dispatch slots of the row pass told apart
constexpr uint32_t ROUND_SHIFT = 5;   // row pass: rotation of the task order per round
// Task-count slope across dispatch slots, measured on MI355X on the dense
// B=64, K=16, V=128000 bf16 batch (greedy and sampled).  Per-slot task counts
// round to whole tasks, so nearby slopes can give the same schedule or
// jump: for the greedy batch 0.3 and 0.45 ran 1.3 and 2 us slower than 0.35.
constexpr float ROW_SKEW_GREEDY = 0.35f;
constexpr float ROW_SKEW_LSE = 0.3f;

enum : int { MODE_GREEDY = 0, MODE_SAMPLE = 1, MODE_CONF = 2 };
// KIND_SAMPLED_R: a sampled request at T = 1 whose draft-row statistics come
// from a confidence pass (the row pass reads its target rows only).
// KIND_DONE: early-exit calls, a request that ended in an earlier window.
// KIND_CONF2: a confidence row whose statistics are also wanted at the
// request's own temperature T != 1 (two sums over one read of the row).
enum : int { KIND_GREEDY = 0, KIND_SAMPLED = 1, KIND_CONF = 2, KIND_BAD = 3, KIND_SAMPLED_R = 4, KIND_DONE = 5,
             KIND_CONF2 = 6 };
// outcome of a request's accept scan; SREQ_CONT (early-exit calls): every
// position of the window accepted and the depth lies beyond it; SREQ_DONE:
// nothing to do in this window
enum : int { SREQ_BAD = 0, SREQ_GREEDY = 1, SREQ_RESID = 2, SREQ_BONUS = 3, SREQ_CONT = 4, SREQ_DONE = 5 };

constexpr double LOG2E = 1.4426950408889634;
constexpr double LN2 = 0.6931471805599453;

// Partial or merged statistics of (part of) a row.  Argmax rows use (m, idx);
// log-sum-exp rows use (m, s) with s = sum exp2((v - m) * c32).  A row that
// is unusable (NaN, +inf, nothing but -inf) has m = NaN or infinite.
struct alignas(16) Stat {
    float m;
    int32_t idx;
    double s;
};

// The C ABI's sv_row_stat is this record.
static_assert(sizeof(Stat) == sizeof(sv_row_stat) && alignof(Stat) == 16, "row statistics record");
static_assert(offsetof(Stat, m) == offsetof(sv_row_stat, max) && offsetof(Stat, s) == offsetof(sv_row_stat, sum),
              "row statistics fields");

struct ReqDesc {
    int32_t state;   // SREQ_*
    int32_t n;       // accepted length (the row pair a draw reads)
    int32_t emit;    // greedy: the emitted token
    float T;
};

// One sampler chunk's fp64 sums over the drawn row pair, all in units of
// 2^((v - max) * log2(e)/T):
//   residual draw: d = sum over {P > rho_hat Q} of (P - rho_hat Q), bq = sum of
//   Q over the same set, sz = sum P, sy = sum Q (P, Q: target and draft terms
//   relative to their row maxima, rho_hat an estimate of sz/sy);
//   bonus draw: m = the chunk's maximum, sz = sum of P relative to m.
struct alignas(16) ChunkPart {
    double d, bq, sz, sy;
    float m;
    int32_t bad;
    int32_t pad[2];
};

// What the draw kernel needs to know of a request (written by the finish
// kernel): the scan's outcome and the drawn row pair's statistics.
struct alignas(16) DrawRec {
    int32_t state, n;
    float T, mz;
    float my;
    int32_t tb;       // first target row (and output slot) of the request
    double rho_hat;
    int32_t db;       // first draft row (and drafted-token slot) of the request
    int32_t nout;     // output slots of the request
    int32_t pad[2];
};

struct Ws {
    int32_t *meta;       // [4]: chunks per row and batches per chunk of the row pass;
                         // then one Stat of scratch (the row pass's placeholder stores)
    Stat *part;          // [B * (2K + 1) * cpr_max] row-pass chunk partials: row j of
                         // request b in slot row b * (2K + 1) + j, chunk c in column c
    ChunkPart *cp;       // [B * cs_max] sampler chunk sums
    DrawRec *rec;        // [B]
    int32_t *alive;      // [2 * B] early-exit calls: request still verifying, per window parity
};

struct Layout {
    size_t off[5];
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
    L.cpr_max = (int)std::min<int64_t>(CPR_CAP, ceil_div(nv, WVEC));
    L.cs_max = (int)std::max(ceil_div(nv, (int64_t)UNIT_E / 4), ceil_div(nvec_max(V, 8), (int64_t)UNIT_E / 8));
    if (L.cs_max > UNITS_MAX) return false;
    const size_t sz[5] = {
        sizeof(int32_t) * 4 + sizeof(Stat),
        sizeof(Stat) * (size_t)L.r_max * (size_t)L.cpr_max,
        sizeof(ChunkPart) * (size_t)B * (size_t)L.cs_max,
        sizeof(DrawRec) * (size_t)B,
        sizeof(int32_t) * 2 * (size_t)B,
    };
    size_t o = 0;
    for (int i = 0; i < 5; ++i) {
        L.off[i] = o;
        o += align256(sz[i]);
    }
    L.total = o;
    return true;
}

Ws carve(void *base, const Layout &L, int B)
{
    char *p = (char *)base;
    Ws w;
    w.meta = (int32_t *)(p + L.off[0]);
    w.part = (Stat *)(p + L.off[1]);
    w.cp = (ChunkPart *)(p + L.off[2]);
    w.rec = (DrawRec *)(p + L.off[3]);
    w.alive = (int32_t *)(p + L.off[4]);
    (void)B;
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
    const Stat *dstats_in;   // sampled calls: draft-row statistics [B, K] from a confidence pass, or NULL
    Stat *dstats_out;        // confidence calls: draft-row statistics out [B, K], or NULL
    const float *conf_temp;  // confidence calls: temperature [B] of the statistics, or NULL (all at T = 1)
    // Packed (CSR) layout, or NULL for the padded one: request b's drafted
    // positions are offs[b] .. offs[b + 1] - 1 of n_rows; K is then the
    // largest depth the call accepts.
    const int32_t *offs;
    int32_t n_rows;
    int32_t B, K, V;
    int32_t bf16;      // logits dtype: 1 bf16, 0 fp32
    int32_t mode;
    int32_t cpr_max;
    int32_t cs;        // sampler units per row (this call's dtype)
    int32_t usplit;    // waves per sampler unit (1, 2 or 4)
    int32_t aligned;   // V * element size is a multiple of 16: every row starts 16-byte aligned
    int32_t row_cus;   // compute units the row-pass grid is spread over
    float row_skew;    // row pass: task-count slope across dispatch slots
    int32_t chunks;    // row pass: chunks per row forced by SPECVERIFY_CHUNK (0: chosen from the grid)
    // Early-exit calls: this launch verifies positions [win_lo, win_hi) of
    // the requests still verifying (alive_in, read when win_lo > 0) and
    // records in alive_out which of them continue into the next window.
    int32_t ee;
    int32_t ee_last;   // the call's last window: its finish kernel sums every drawn row pair
    int32_t win_lo, win_hi;
    const int32_t *alive_in;
    int32_t *alive_out;
    Ws ws;
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The elements of a 16-byte vector as fp32 (exact widening for bf16).
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

// Pointers into device memory in the global address space: loads through
// them compile to global_load (a generic pointer, e.g. one taken out of a
// struct kernel argument, would compile to flat_load).
typedef const __attribute__((address_space(1))) uint4 *gvec_t;

// Plain 16-byte load (the sampler re-reads rows the row pass streamed).
__device__ __forceinline__ uint4 ld_plain(gvec_t p)
{
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v w = *(const __attribute__((address_space(1))) u4v *)p;
    return make_uint4(w.x, w.y, w.z, w.w);
}

// Streaming 16-byte load (nontemporal: the row pass reads each logit once).
__device__ __forceinline__ uint4 ld_stream(gvec_t p)
{
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v w = __builtin_nontemporal_load((const __attribute__((address_space(1))) u4v *)p);
    return make_uint4(w.x, w.y, w.z, w.w);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Butterfly partner exchanges without the LDS crossbar.  Level L pairs every
// lane with one lane of the other half of its aligned group of 2^(L+1)
// lanes: L0 lane^1 and L1 lane^2 (DPP quad permutes), L2 the mirror lane
// within 8 and L3 within 16 (DPP row mirrors), L4 lane^16 and L5 lane^32
// (gfx950 permlane swaps).  After levels 0..L every lane of a group holds the
// group's combination (each pair combines the same two values).
template <int L>
__device__ __forceinline__ uint32_t xchg(uint32_t v)
{
    if constexpr (L == 0) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
    else if constexpr (L == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
    else if constexpr (L == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
    else if constexpr (L == 3) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
    else if constexpr (L == 4) {
        const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & 16) ? q[0] : q[1];
    } else {
        const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? q[0] : q[1];
    }
}
template <int L> __device__ __forceinline__ float xchg_f(float v) { return __uint_as_float(xchg<L>(__float_as_uint(v))); }
template <int L> __device__ __forceinline__ int xchg_i(int v) { return (int)xchg<L>((uint32_t)v); }
template <int L>
__device__ __forceinline__ double xchg_d(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t r = (uint64_t)xchg<L>((uint32_t)u) | ((uint64_t)xchg<L>((uint32_t)(u >> 32)) << 32);
    return __longlong_as_double((long long)r);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, xchg_f<0>(v));
    v = fmaxf(v, xchg_f<1>(v));
    v = fmaxf(v, xchg_f<2>(v));
    v = fmaxf(v, xchg_f<3>(v));
    v = fmaxf(v, xchg_f<4>(v));
    return fmaxf(v, xchg_f<5>(v));
}

__device__ __forceinline__ double wave_sum(double v)
{
    v += xchg_d<0>(v);
    v += xchg_d<1>(v);
    v += xchg_d<2>(v);
    v += xchg_d<3>(v);
    v += xchg_d<4>(v);
    return v + xchg_d<5>(v);
}

__device__ __forceinline__ int wave_sum_i(int v)
{
    v += xchg_i<0>(v);
    v += xchg_i<1>(v);
    v += xchg_i<2>(v);
    v += xchg_i<3>(v);
    v += xchg_i<4>(v);
    return v + xchg_i<5>(v);
}

__device__ __forceinline__ int wave_or(int v)
{
    v |= xchg_i<0>(v);
    v |= xchg_i<1>(v);
    v |= xchg_i<2>(v);
    v |= xchg_i<3>(v);
    v |= xchg_i<4>(v);
    return v | xchg_i<5>(v);
}

// (value desc, index asc) argmax merge.
__device__ __forceinline__ void argmax_merge(float &m, int &i, float m2, int i2)
{
    if (m2 > m || (m2 == m && i2 < i)) { m = m2; i = i2; }
}

template <int L>
__device__ __forceinline__ void argmax_level(float &m, int &i)
{
    const float m2 = xchg_f<L>(m);
    const int i2 = xchg_i<L>(i);
    argmax_merge(m, i, m2, i2);
}

__device__ __forceinline__ void wave_argmax(float &m, int &i)
{
    argmax_level<0>(m, i);
    argmax_level<1>(m, i);
    argmax_level<2>(m, i);
    argmax_level<3>(m, i);
    argmax_level<4>(m, i);
    argmax_level<5>(m, i);
}

// Inclusive scans over the wave in lane order with DPP: shifts right by 1, 2,
// 4, 8 inside each 16-lane row (lanes without a source read 0), then each
// row's total carried forward by the row broadcasts of lane 15 (into rows 1
// and 3) and lane 31 (into rows 2 and 3).
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, BC);
}
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ double dpp_d(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint64_t r = (uint64_t)dpp_u<CTRL, ROWS, BC>((uint32_t)u) |
                       ((uint64_t)dpp_u<CTRL, ROWS, BC>((uint32_t)(u >> 32)) << 32);
    return __longlong_as_double((long long)r);
}

__device__ __forceinline__ double wave_incl_scan(double v)
{
    v += dpp_d<0x111, 0xF, true>(v);
    v += dpp_d<0x112, 0xF, true>(v);
    v += dpp_d<0x114, 0xF, true>(v);
    v += dpp_d<0x118, 0xF, true>(v);
    v += dpp_d<0x142, 0xA, false>(v);
    v += dpp_d<0x143, 0xC, false>(v);
    return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v)
{
    v += (int)dpp_u<0x111, 0xF, true>((uint32_t)v);
    v += (int)dpp_u<0x112, 0xF, true>((uint32_t)v);
    v += (int)dpp_u<0x114, 0xF, true>((uint32_t)v);
    v += (int)dpp_u<0x118, 0xF, true>((uint32_t)v);
    v += (int)dpp_u<0x142, 0xA, false>((uint32_t)v);
    v += (int)dpp_u<0x143, 0xC, false>((uint32_t)v);
    return v;
}

// value of the previous lane (0 in lane 0): DPP wave shift right by one
__device__ __forceinline__ double wave_shr1(double v) { return dpp_d<0x138, 0xF, true>(v); }

// Workgroup reductions through LDS (all threads must call; result in all).
struct RedSmem {
    float f[NWAVE];
    int i[NWAVE];
    double d[NWAVE];
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

// Exclusive scan of one double per thread over the workgroup, in thread order.
__device__ double wg_excl_scan(double v, double *sm4, double &total)
{
    const int lane = lane_id();
    const double incl = wave_incl_scan(v);
    const double excl = wave_shr1(incl);
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

// fp64 2^(s/512) for s <= 0, within 6e-11 relative, not correctly rounded.
// The sampler's sums compare a uniform with a residual CDF to within 1e-6
// of the residual's mass R; a per-term relative error e moves that CDF by at
// most about 2e/R (R as a fraction of the row's mass), so 6e-11 holds the
// band for every R above 1e-4, and a rejection whose residual holds less
// than that happens with probability below 1e-4.  s = k + r with
// k = round(s) taken from the low word of s + 1.5*2^52, |r| <= 1/2;
// 2^(k/512) = 2^(k >> 9) * T[k & 511] with T[j] = 2^(j/512) tabulated in LDS
// at kernel start, and 2^(r/512) = e^x, |x| <= ln2/1024, by its Taylor
// polynomial of degree 2 (truncation x^3/6 < 5.2e-11).  Taking the argument pre-scaled by 512
// lets callers fold the scale into their own constants.  s is clamped at
// -2000*512, so -inf (a masked logit) and anything below 2^-2000 give exactly
// 0 through ldexp's underflow; a NaN argument also gives 0 (rows holding NaN
// are flagged separately wherever they are read).
// Entry j = q + 64 i of the table is 2^(q/512) * 2^(i/8): one exp2 per lane
// and eight products, each entry within about 2 ulp.
__device__ constexpr double EXP2_EIGHTHS[8] = {   // 2^(i/8), correctly rounded
    0x1.0000000000000p+0, 0x1.172b83c7d517bp+0, 0x1.306fe0a31b715p+0, 0x1.4bfdad5362a27p+0,
    0x1.6a09e667f3bcdp+0, 0x1.8ace5422aa0dbp+0, 0x1.ae89f995ad3adp+0, 0x1.d5818dcfba487p+0};

static_assert(EXP2_TAB == 64 * 8, "the table is 64 lanes times 8 eighths");

// One wave writes the whole table.
__device__ __forceinline__ void fill_exp2_table(double *tab)
{
    const int q = lane_id();
    const double e = exp2((double)q / EXP2_TAB);
#pragma unroll
    for (int i = 0; i < 8; ++i) tab[q + 64 * i] = e * EXP2_EIGHTHS[i];
}

__device__ void init_exp2_table(double *tab)
{
    if (wave_id() == 0) fill_exp2_table(tab);
    __syncthreads();
}

__device__ __forceinline__ double exp2_512(double s, const double *tab)
{
    constexpr double SHIFT = 6755399441055744.0;   // 1.5 * 2^52
    constexpr double D1 = LN2 / EXP2_TAB, D2 = D1 * D1 / 2.0;
    s = __builtin_fmax(s, -2000.0 * EXP2_TAB);
    const double kb = s + SHIFT;
    const int k = (int)(uint32_t)(uint64_t)__double_as_longlong(kb);
    const double r = s - (kb - SHIFT);
    double p = fma(r, D2, D1);
    p = fma(r, p, 1.0);
    return ldexp(tab[k & (EXP2_TAB - 1)] * p, k >> 9);
}

// fp64 2^x for x <= 0 (see exp2_512).
__device__ __forceinline__ double exp2_tab(double x, const double *tab) { return exp2_512(x * EXP2_TAB, tab); }

// ---------------------------------------------------------------------------
// Batch plan: rows each request contributes to the row pass.
//   greedy request (greedy call, or T == 0): target rows 0..d
//   sampled request (T > 0): target rows 0..d-1, then draft rows 0..d-1
//   confidence call: draft rows 0..K_b-1
// A request whose depth or temperature is invalid contributes no rows.
// Early-exit calls verify the positions [lo, hi) of a window, lo = win_lo
// and hi = min(win_hi, d), of the requests still verifying: a greedy
// request reads target rows lo..hi-1, plus its bonus row d when the window
// reaches the depth (win_hi >= d); a sampled request reads target rows and
// then draft rows lo..hi-1.  Row indices within the request are relative to
// lo, and d below is then the window's position count hi - lo.
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool temp_ok(float T)
{
    return T == 0.0f || (T > 0.0f && T <= 3.40282347e38f);   // excludes NaN, < 0, inf
}

// A readable word no kernel writes: the address an unused optional
// argument's load goes to.
__device__ int32_t k_stand_in = 0;

// Where request b's rows and slots start.  Padded layout: target row k and
// output slot k at b(K + 1) + k; draft row k, drafted token k, accept
// uniform k and p/q slot k at bK + k; K + 1 output slots.  Packed layout
// (positions o0 = offs[b] .. o1 - 1 = offs[b + 1] - 1): target row and output
// slot k at o0 + b + k, the others at o0 + k; o1 - o0 + 1 output slots (none
// when the offsets are unusable).
struct ReqBase {
    int64_t tb, db;
    int nout;
};

struct ReqPlan {
    int d, kind, rows;
    float T;
    int lo;      // first position of the window (0 outside early-exit calls)
    bool fin;    // the window reaches the depth: the request ends in it
    bool pair_ok;   // packed layout: 0 <= offs[b] <= offs[b + 1] <= n_rows
    ReqBase rb;
};

// The per-request arguments a plan reads.  Every load is issued, and
// unconditionally: an argument the call does not use is read from a valid
// stand-in address and its value discarded.  (Loads issued under branches
// were each waited for at the branch's join, one after another.)  Kept
// apart from the arithmetic so a caller can issue these loads ahead of its
// others and wait for them alone: waits on vector loads retire in issue
// order.
struct PlanArgs {
    int dv;      // depth (or max_depth) of request b
    float tv;    // temperature
    int rtv;     // the first given draft record's temperature bits
    float ctv;   // confidence call: the statistics temperature
    int av;      // early exit: still verifying
    int o0, o1;  // packed layout: the request's offsets
};

template <bool EE>
__device__ __forceinline__ PlanArgs plan_loads(const Params &P, int b)
{
    const int32_t *stand_in = &k_stand_in;
    const int32_t *dp = P.mode == MODE_CONF ? (P.max_depth ? P.max_depth + b : stand_in)
                                            : (P.depth ? P.depth + b : stand_in);
    const float *tp = P.mode == MODE_SAMPLE ? P.temperature + b : (const float *)stand_in;
    const int32_t *ap = (EE && P.win_lo > 0) ? P.alive_in + b : stand_in;
    const int32_t *o0p = P.offs ? P.offs + b : stand_in;
    const int32_t *o1p = P.offs ? P.offs + b + 1 : stand_in;
    // the temperature the given draft statistics were taken at (the first
    // record's temp field), and a confidence call's statistics temperature
    const int32_t *rtp = (P.mode == MODE_SAMPLE && P.dstats_in && P.K > 0)
                             ? (const int32_t *)(P.dstats_in + (int64_t)b * P.K) + 1 : stand_in;
    const float *ctp = (P.mode == MODE_CONF && P.conf_temp) ? P.conf_temp + b : (const float *)stand_in;
    // through the scalar cache where b is wave-uniform (the finish kernel):
    // counted apart from the vector loads issued after these
    typedef const __attribute__((address_space(4))) int32_t *CI;
    PlanArgs a;
    a.dv = *(CI)dp;
    a.tv = __int_as_float(*(CI)tp);
    a.rtv = *(CI)rtp;
    a.ctv = __int_as_float(*(CI)ctp);
    a.av = *(CI)ap;
    a.o0 = *(CI)o0p;
    a.o1 = *(CI)o1p;
    return a;
}

// offs_bad: packed layout, the offsets are not a valid CSR array (some
// request's pair is unusable), which makes every request bad.
template <bool EE>
__device__ __forceinline__ ReqPlan plan_request(const Params &P, int b, bool offs_bad, const PlanArgs &a)
{
    int dv = a.dv;
    const float tv = a.tv;
    const int rtv = a.rtv;
    const float ctv = a.ctv;
    const int av = a.av;
    const int o0 = a.o0, o1 = a.o1;
    const bool have_depth = P.offs || (P.mode == MODE_CONF ? P.max_depth != nullptr : P.depth != nullptr);

    ReqPlan q;
    q.T = 0.0f;
    q.lo = 0;
    q.fin = true;
    q.pair_ok = true;
    if (P.offs) {
        q.pair_ok = 0 <= o0 && o0 <= o1 && o1 <= P.n_rows;
        dv = (q.pair_ok && !offs_bad) ? o1 - o0 : -1;
        q.rb.tb = (int64_t)o0 + b;
        q.rb.db = o0;
        q.rb.nout = (q.pair_ok && !offs_bad) ? o1 - o0 + 1 : 0;
    } else {
        q.rb.tb = (int64_t)b * (P.K + 1);
        q.rb.db = (int64_t)b * P.K;
        q.rb.nout = P.K + 1;
    }
    if (P.mode == MODE_CONF) {
        q.d = have_depth ? dv : P.K;
        const bool ok = q.d >= 0 && q.d <= P.K;
        // statistics at the request's own temperature when one is given and
        // is a finite T > 0 other than 1; at T = 1 otherwise
        const bool dual = P.conf_temp && ctv > 0.0f && ctv <= 3.40282347e38f && ctv != 1.0f;
        q.kind = ok ? (dual ? KIND_CONF2 : KIND_CONF) : KIND_BAD;
        q.T = dual ? ctv : 1.0f;
        q.rows = ok ? q.d : 0;
    } else {
        q.d = have_depth ? dv : P.K;
        q.T = (P.mode == MODE_SAMPLE) ? tv : 0.0f;
        const bool ok = q.d >= 0 && q.d <= P.K && temp_ok(q.T);
        q.kind = !ok ? KIND_BAD : (q.T > 0.0f ? KIND_SAMPLED : KIND_GREEDY);
        // reuse the draft rows' statistics when they were taken at this
        // request's temperature
        if (q.kind == KIND_SAMPLED && P.dstats_in && rtv == __float_as_int(q.T)) q.kind = KIND_SAMPLED_R;
        q.rows = !ok ? 0 : (q.kind == KIND_SAMPLED ? 2 * q.d : q.kind == KIND_SAMPLED_R ? q.d : q.d + 1);
        if constexpr (EE) {
            q.lo = P.win_lo;
            if (q.lo > 0 && !av) {
                q.kind = KIND_DONE;
                q.rows = 0;
            } else if (ok) {
                // a request still verifying at lo > 0 accepted positions
                // 0..lo-1 of a window that ended before its depth: lo < d
                q.fin = P.win_hi >= q.d;
                const int nd = min(P.win_hi, q.d) - q.lo;
                q.rows = q.kind == KIND_SAMPLED ? 2 * nd : nd + (q.fin ? 1 : 0);
                q.d = nd;
            }
        }
    }
    if (q.kind == KIND_BAD || q.kind == KIND_DONE) q.d = 0;
    return q;
}

// Exponent scale of a row's log-sum-exp statistics.  Every exponent of the
// row statistics and of the accept test is (v - M) * c with c = c32 * 2^sh:
// c32 = fl(log2(e)/T), which differs from log2(e)/T by at most 6e-8
// relative, and sh = 0; only when log2(e)/T exceeds 2^100 (T below about
// 1.1e-30, down to the smallest positive fp32 value) is c32 the rounded
// quotient times 2^-64 and sh = 64, so that c32 stays a finite fp32 number
// for every finite T > 0.
struct LseScale {
    float c32;
    int sh;   // 0 or 64
};

constexpr double SCALE_SHIFT_AT = 0x1p100;

__device__ __forceinline__ LseScale scale_of(int kind, float T)
{
    const double c = LOG2E / (double)((kind == KIND_CONF || kind == KIND_CONF2) ? 1.0f : T);
    LseScale sc;
    sc.sh = c > SCALE_SHIFT_AT ? 64 : 0;
    sc.c32 = (float)(sc.sh ? c * 0x1p-64 : c);
    return sc;
}

struct Plan {
    int *row_off;   // [B + 1] in LDS
    int *info;      // [B] in LDS: d | kind << 16
    float *c32;     // [B] in LDS: the request's own-temperature scale (scale_of at its T)
};

// Plan info word: d in bits 0-15, the kind in bits 16-23, and PLAN_SH when
// the request's own-temperature scale carries the 2^64 shift.
constexpr int PLAN_SH = 1 << 24;

// Whole-workgroup plan: row_off = exclusive prefix of per-request rows.
// Returns 1 when the packed layout's offsets are not a valid CSR array
// (then every request is bad and reads no rows), else 0.
template <bool EE>
__device__ int make_plan(const Params &P, Plan pl, int *scan_tmp)
{
    const int B = P.B;
    const int per = (int)ceil_div(B, WG);
    const int b0 = threadIdx.x * per;
    int local = 0, bad_pair = 0;
    for (int j = 0; j < per; ++j) {
        const int b = b0 + j;
        if (b >= B) break;
        const ReqPlan q = plan_request<EE>(P, b, false, plan_loads<EE>(P, b));
        // the scale's division once per request here, not once per task;
        // meaningless (unused) for requests without a temperature
        const LseScale sc = scale_of(KIND_SAMPLED, q.T);
        pl.info[b] = q.d | (q.kind << 16) | (sc.sh ? PLAN_SH : 0);
        pl.c32[b] = sc.c32;
        pl.row_off[b] = q.rows;   // count for now
        local += q.rows;
        bad_pair |= !q.pair_ok;
    }
    int offs_bad = 0;
    if (P.offs && __syncthreads_or(bad_pair)) {
        offs_bad = 1;
        local = 0;
        for (int j = 0; j < per; ++j) {
            const int b = b0 + j;
            if (b >= B) break;
            pl.info[b] = KIND_BAD << 16;
            pl.row_off[b] = 0;
        }
    }
    const int v = wave_incl_scan_i(local);
    const int lane = lane_id();
    if (lane == 63) scan_tmp[wave_id()] = v;
    __syncthreads();
    int wave_base = 0;
    for (int w = 0; w < wave_id(); ++w) wave_base += scan_tmp[w];
    int run = wave_base + v - local;
    for (int j = 0; j < per; ++j) {
        const int b = b0 + j;
        if (b >= B) break;
        const int c = pl.row_off[b];
        pl.row_off[b] = run;
        run += c;
    }
    if (threadIdx.x == WG - 1) pl.row_off[B] = run;
    __syncthreads();
    return offs_bad;
}

// Request containing global active row r, for a wave-uniform r: the b with
// row_off[b] <= r < row_off[b + 1] (row_off non-decreasing, row_off[0] = 0,
// so an empty request is never the answer).  That b is the number of
// j in [1, B - 1] with row_off[j] <= r, and those j form a prefix, so the
// wave counts them with ballots instead of a serial binary search: the lanes
// first test every S-th entry (S = ceil((B - 1) / 64)), which bounds b to S
// consecutive values, then test those.  One LDS read per lane for B <= 65,
// two up to B = 4097, whatever the batch.
__device__ __forceinline__ int find_request(const int *row_off, int B, int r)
{
    const int n = B - 1;
    if (n <= 0) return 0;
    const int lane = lane_id();
    const int S = (n + 63) >> 6;
    const int j1 = 1 + lane * S;
    const bool t1 = j1 <= n && row_off[j1] <= r;
    const int c1 = __builtin_popcountll(__ballot(t1));
    if (S == 1 || c1 == 0) return c1;
    const int base = 1 + (c1 - 1) * S;   // row_off[base] <= r, so b >= base
    const int j2 = base + 1 + lane;
    const bool t2 = lane < S - 1 && j2 <= n && row_off[j2] <= r;
    return base + __builtin_popcountll(__ballot(t2));
}

// Chunking of the row pass: cpr chunks per row of nb batches each, with cpr
// chosen so that every wave gets about `tpw` tasks, but a task covers at
// least two batches where the row has them: a wave sets up its next task
// while its other buffer's batch is in flight, and a run of one-batch tasks
// leaves that set-up exposed between loads (passes over a few hundred rows
// ran about 12 % slower on MI355X).  Calls with log-sum-exp rows take about
// twelve tasks per wave: finer tasks round the per-slot task counts more
// evenly, and the dense B=64, K=16, V=128000 sampled batch ran 1.3 us faster
// at 21 chunks of three batches than at 16 of four.  Greedy calls take about
// eight: their rows cost less per batch, so a task's set-up weighs more, and
// the same batch ran about 0.4 us slower at 32 chunks of two batches than at
// 21 of three (measured on MI355X).
// A positive `forced` (SPECVERIFY_CHUNK, a test and tuning override) asks for
// that many chunks per row instead, within [1, min(batches, 256)].
__device__ __forceinline__ void row_chunking(int R, int V, bool bf16, int64_t nwaves, int tpw, int forced, int &cpr,
                                             int &nb)
{
    const int64_t nv = nvec_max(V, bf16 ? 8 : 4);
    const int nbt = (int)ceil_div(nv, WVEC);
    const int64_t want = ceil_div((int64_t)tpw * nwaves, (int64_t)(R > 0 ? R : 1));
    cpr = (int)std::min<int64_t>(std::max<int64_t>(want, 1),
                                 std::min<int64_t>(std::min(nbt, CPR_CAP), ceil_div(nbt, 2)));
    if (forced > 0) cpr = std::min(forced, std::min(nbt, CPR_CAP));
    nb = (int)ceil_div(nbt, cpr);
    cpr = (int)ceil_div(nbt, nb);
}

// ---------------------------------------------------------------------------
// Row pass (kernel A).  A wave task reads a run of batches of one logit row;
// a batch is UW 16-byte vectors per lane, lane l reading vectors
// vbeg + j*64 + l, so every wave load instruction is one contiguous 1 KiB.
// The vector grid starts at the row's first element rounded down to 16
// bytes; elements before the row start or past its end are masked to -inf.
// ---------------------------------------------------------------------------

template <bool BF16>
struct RowView {
    static constexpr int EPV = BF16 ? 8 : 4;
    gvec_t vec;         // 16-byte aligned start of the vector grid
    int head;           // elements of vector 0 before the row start
    int nvec;           // vectors covering the row
    int V;

    __device__ RowView() {}
    __device__ RowView(const void *row_start, int V_) : V(V_)
    {
        const int off = (int)((uintptr_t)row_start & 15u);
        vec = (gvec_t)((const char *)row_start - off);
        head = off / (BF16 ? 2 : 4);
        nvec = (int)ceil_div((int64_t)head + V, EPV);
    }
    // element index (within the row) of element e of vector vi
    __device__ __forceinline__ int elem(int vi, int e) const { return vi * EPV + e - head; }
    // does vector vi hold elements outside the row?
    __device__ __forceinline__ bool edge(int vi) const { return vi * EPV < head || (vi + 1) * EPV - head > V; }
    // does the batch of vectors [vbeg, vbeg + n) touch a row edge?
    __device__ __forceinline__ bool batch_edge(int vbeg, int n) const
    {
        return vbeg * EPV < head || (vbeg + n) * EPV - head > V;
    }
};

// Issues one batch of loads.  Branch-free: vectors past the row are loaded
// from the row's last vector instead (always a valid address) and their
// elements, whose indices lie past V, are masked when the batch is widened.
// A load under a branch would make the compiler wait for every outstanding
// load at the join, which would defeat the double buffering.
__device__ __forceinline__ void issue_batch(gvec_t vec, int nvec, int vbeg, uint4 (&raw)[UW])
{
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < UW; ++j) raw[j] = ld_stream(vec + min(vbeg + j * 64 + lane, nvec - 1));
}

template <bool BF16, bool EDGE>
__device__ __forceinline__ void widen(const RowView<BF16> &rv, int vi, const uint4 &raw, float (&f)[RowView<BF16>::EPV])
{
    unpack<BF16>(raw, f);
    if (EDGE) {
#pragma unroll
        for (int e = 0; e < RowView<BF16>::EPV; ++e) {
            const int x = rv.elem(vi, e);
            if (x < 0 || x >= rv.V) f[e] = -INFINITY;
        }
    }
}

// Greedy rows: running largest value and its lowest index (lane level); NaN
// is flagged.  A lane visits its elements in index order, so a strict >
// keeps the lowest index of the lane's maximum.
struct ArgmaxLane {
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    int nanf = 0;
};

template <bool BF16, bool EDGE>
__device__ __forceinline__ void argmax_batch(const RowView<BF16> &rv, int vbeg, const uint4 (&raw)[UW], ArgmaxLane &st)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < UW; ++j) {
        const int vi = vbeg + j * 64 + lane;
        float f[EPV];
        widen<BF16, EDGE>(rv, vi, raw[j], f);
#pragma unroll
        for (int e = 0; e < EPV; e += 2) st.nanf |= __builtin_isunordered(f[e], f[e + 1]);
        float m = f[0];
#pragma unroll
        for (int e = 1; e < EPV; ++e) m = fmaxf(m, f[e]);
        if (m > st.best) {
            // first element of this vector equal to its maximum
            int found = EPV - 1;
#pragma unroll
            for (int e = EPV - 2; e >= 0; --e)
                if (f[e] == m) found = e;
            st.best = m;
            st.bidx = rv.elem(vi, found);
        }
    }
}

// The scale as a double, exactly c32 * 2^sh.
__device__ __forceinline__ double scale_d(const LseScale &sc) { return sc.sh ? (double)sc.c32 * 0x1p64 : (double)sc.c32; }

// fp32 exponent d * c for a difference d = v - M <= 0 (rounded twice at
// most; a product past the fp32 range is -inf, whose exp2 is the exact 0).
__device__ __forceinline__ float scaled_exp(float d, const LseScale &sc)
{
    return sc.sh ? (d * 0x1p64f) * sc.c32 : d * sc.c32;
}

// 2^-dl for the residual dl of an fp32 product (|dl| <= 64): the second-order
// series where its truncation (below 2e-16 relative) vanishes in double, the
// fp64 exp2 otherwise.
__device__ __forceinline__ double offset_factor(float dl)
{
    if (__builtin_fabsf(dl) <= 0x1p-16f) {
        const double x = (double)dl * LN2;
        return 1.0 - x + 0.5 * x * x;
    }
    return exp2(-(double)dl);
}

// Sampled / confidence rows: the lane's running max M and
// s = sum 2^((v - M) * c) (scale as above), s kept in double.  Terms are
// summed in fp32 per vector (a short tree) and the vector sums in a second
// short tree.  Two ways to form each term's exponent:
//  * the FMA form (the normal case): one FMA, v*c32 - fl(M*c32).  The
//    offset dl = M*c32 - fl(M*c32) is exact (the FMA residual of the
//    product) and is taken out of every batch sum by the factor 2^-dl
//    (offset_factor), computed when M changes.  It needs sh = 0 and
//    |fl(M*c32)| < 2^31, so that |dl| <= 64 keeps every term inside the fp32
//    range;
//  * the difference form: (v - M) * c, two operations, valid for every
//    finite M and every scale.  A wave takes it for a batch when any of its
//    lanes is outside the FMA form's range (very large |M| / T).
// When a batch raises M, s is rescaled once by 2^((M_old - M_new) * c)
// (fp32 exp2, within 2 ulp).
struct LseLane {
    float M = -INFINITY;
    float mc = 0.0f;      // fl(M*c32)
    double corr = 1.0;    // 2^-dl
    double s = 0.0;
};

template <bool BF16, bool EDGE>
__device__ __forceinline__ void lse_batch(const RowView<BF16> &rv, int vbeg, const uint4 (&raw)[UW],
                                          const LseScale &sc, LseLane &st)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const int lane = lane_id();
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
        float f[EPV];
        widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) bm = fmaxf(bm, f[e]);
    }
    if (bm > st.M) {
        if (st.M != -INFINITY) st.s *= (double)__builtin_amdgcn_exp2f(scaled_exp(st.M - bm, sc));
        st.M = bm;
        st.mc = bm * sc.c32;
        st.corr = offset_factor(__builtin_fmaf(bm, sc.c32, -st.mc));
    }
    if (st.M == -INFINITY) {
        // nothing but -inf / masked so far; a NaN must still poison the sum
        int un = 0;
#pragma unroll
        for (int j = 0; j < UW; ++j) {
            float f[EPV];
            widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
#pragma unroll
            for (int e = 0; e < EPV; e += 2) un |= __builtin_isunordered(f[e], f[e + 1]);
        }
        if (un) st.s = NAN;
        return;
    }
    const bool diff_form = sc.sh != 0 || __ballot(!(__builtin_fabsf(st.mc) < 0x1p31f)) != 0;
    float vs[UW];
    if (!diff_form) {
#pragma unroll
        for (int j = 0; j < UW; ++j) {
            float f[EPV];
            widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
            float t[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) t[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], sc.c32, -st.mc));
#pragma unroll
            for (int w = EPV / 2; w > 0; w >>= 1)
#pragma unroll
                for (int e = 0; e < w; ++e) t[e] += t[e + w];
            vs[j] = t[0];
        }
    } else {
#pragma unroll
        for (int j = 0; j < UW; ++j) {
            float f[EPV];
            widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
            float t[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) t[e] = __builtin_amdgcn_exp2f(scaled_exp(f[e] - st.M, sc));
#pragma unroll
            for (int w = EPV / 2; w > 0; w >>= 1)
#pragma unroll
                for (int e = 0; e < w; ++e) t[e] += t[e + w];
            vs[j] = t[0];
        }
    }
#pragma unroll
    for (int w = UW / 2; w > 0; w >>= 1)
#pragma unroll
        for (int j = 0; j < w; ++j) vs[j] += vs[j + w];
    st.s += diff_form ? (double)vs[0] : (double)vs[0] * st.corr;
}

template <bool BF16, bool LSE, typename State>
__device__ __forceinline__ void process_batch(const RowView<BF16> &rv, int vbeg, const uint4 (&raw)[UW],
                                              const LseScale &sc, State &st)
{
    if constexpr (LSE) {
        if (rv.batch_edge(vbeg, WVEC)) lse_batch<BF16, true>(rv, vbeg, raw, sc, st);
        else lse_batch<BF16, false>(rv, vbeg, raw, sc, st);
    } else {
        if (rv.batch_edge(vbeg, WVEC)) argmax_batch<BF16, true>(rv, vbeg, raw, st);
        else argmax_batch<BF16, false>(rv, vbeg, raw, st);
    }
}


// Two log-sum-exp statistics of the same row over one read: lane states a
// (scale sa, T = 1) and b (scale sb, a request's own temperature) share the
// running max M.  State a takes exactly lse_batch's arithmetic (so the
// confidence is the same bits as the single-statistic pass); state b's terms
// use the difference form, (v - M) * c, valid for every finite M and scale.
// A confidence row whose statistics are also wanted at another temperature.
template <bool BF16, bool EDGE>
__device__ __forceinline__ void lse_batch2(const RowView<BF16> &rv, int vbeg, const uint4 (&raw)[UW],
                                           const LseScale &sa, const LseScale &sb, LseLane &a, LseLane &b)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const int lane = lane_id();
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
        float f[EPV];
        widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) bm = fmaxf(bm, f[e]);
    }
    if (bm > a.M) {
        if (a.M != -INFINITY) {
            a.s *= (double)__builtin_amdgcn_exp2f(scaled_exp(a.M - bm, sa));
            b.s *= (double)__builtin_amdgcn_exp2f(scaled_exp(a.M - bm, sb));
        }
        a.M = b.M = bm;
        a.mc = bm * sa.c32;
        a.corr = offset_factor(__builtin_fmaf(bm, sa.c32, -a.mc));
    }
    if (a.M == -INFINITY) {
        int un = 0;
#pragma unroll
        for (int j = 0; j < UW; ++j) {
            float f[EPV];
            widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
#pragma unroll
            for (int e = 0; e < EPV; e += 2) un |= __builtin_isunordered(f[e], f[e + 1]);
        }
        if (un) a.s = b.s = NAN;
        return;
    }
    const bool diff_a = sa.sh != 0 || __ballot(!(__builtin_fabsf(a.mc) < 0x1p31f)) != 0;
    float va[UW], vb[UW];
    // state a: the single-statistic pass's forms and pairwise tree (same
    // bits); state b: difference-form terms added in order (fewer live
    // registers).  The form of a is wave-uniform: one loop per form.
    auto terms = [&](auto fma_form) {
        constexpr bool FMA = decltype(fma_form)::value;
#pragma unroll
        for (int j = 0; j < UW; ++j) {
            float f[EPV];
            widen<BF16, EDGE>(rv, vbeg + j * 64 + lane, raw[j], f);
            float ta[EPV];
            float sbv = 0.0f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                ta[e] = __builtin_amdgcn_exp2f(FMA ? __builtin_fmaf(f[e], sa.c32, -a.mc) : scaled_exp(f[e] - a.M, sa));
                sbv += __builtin_amdgcn_exp2f(scaled_exp(f[e] - a.M, sb));
            }
#pragma unroll
            for (int w = EPV / 2; w > 0; w >>= 1)
#pragma unroll
                for (int e = 0; e < w; ++e) ta[e] += ta[e + w];
            va[j] = ta[0];
            vb[j] = sbv;
            // one vector's terms at a time: interleaving all UW vectors'
            // temporaries would need more registers than the kernel has
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (diff_a) terms(std::false_type());
    else terms(std::true_type());
#pragma unroll
    for (int w = UW / 2; w > 0; w >>= 1)
#pragma unroll
        for (int j = 0; j < w; ++j) {
            va[j] += va[j + w];
            vb[j] += vb[j + w];
        }
    a.s += diff_a ? (double)va[0] : (double)va[0] * a.corr;
    b.s += (double)vb[0];
}

// One chunk of one row: its row view and the end b1 of the batches
// [c * nb, b1) it covers.  A chunk past the end of a short row (rows whose
// start is not 16-byte aligned cover one vector more) gets one fully masked
// batch, so a chunk is never empty.  All fields are wave-uniform (scalar).
template <bool BF16>
struct Task {
    gvec_t vec;    // row view: vector grid start, head elements, vectors
    int head, nvec;
    int r, c, b1;
    int slot;      // partial slot row: request * (2K + 1) + row within the request
    int k;         // the wave's round of this task
    uint32_t pre;  // first task index of round k
    LseScale sc;   // log-sum-exp scale; c32 = 0 marks a greedy (argmax) row
    float zx;      // sampled rows: the row's logit at the drafted token
    LseScale sc2;  // confidence rows with temperatures: the second statistic's scale
    int slot2;     // confidence rows with temperatures: the second statistic's partial slot row
    __device__ __forceinline__ bool lse() const { return sc.c32 != 0.0f; }
    __device__ __forceinline__ RowView<BF16> view(int V) const
    {
        RowView<BF16> rv;
        rv.vec = vec;
        rv.head = head;
        rv.nvec = nvec;
        rv.V = V;
        return rv;
    }
};

// Wave-uniform loads through the scalar cache (constant address space): they
// are counted apart from the vector loads of the stream, so waiting for one
// never drains the batches in flight.
__device__ __forceinline__ int ld_scalar_i32(const int *p)
{
    return *(const __attribute__((address_space(4))) int *)p;
}
template <bool BF16>
__device__ __forceinline__ float ld_scalar_logit(const void *row, int x)
{
    if constexpr (BF16) {
        // the aligned word holding the element (same page, always readable)
        const uintptr_t a = (uintptr_t)row + 2 * (uintptr_t)x;
        const uint32_t w = (uint32_t)ld_scalar_i32((const int *)(a & ~(uintptr_t)3));
        return __uint_as_float((a & 2) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __int_as_float(ld_scalar_i32((const int *)row + x));
    }
}

// Task (r, c): chunk c of global active row r.  Everything here is
// wave-uniform.
template <bool BF16, bool EE>
__device__ __forceinline__ Task<BF16> make_task(const Params &P, const Plan &pl, int r, int c, int nb)
{
    Task<BF16> k;
    k.r = r;
    k.c = c;
    bool lse;
    const int b = find_request(pl.row_off, P.B, r);
    const int local = r - __builtin_amdgcn_readfirstlane(pl.row_off[b]);
    const int info = __builtin_amdgcn_readfirstlane(pl.info[b]);
    const float cT = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(pl.c32[b])));
    const int d = info & 0xffff, kind = (info >> 16) & 0xff;
    const int shT = (info & PLAN_SH) ? 64 : 0;
    k.slot = b * (2 * P.K + 1) + local;
    bool is_draft;
    int kk;
    if (kind == KIND_GREEDY) { is_draft = false; kk = local; lse = false; }
    else if (kind == KIND_SAMPLED) { is_draft = local >= d; kk = is_draft ? local - d : local; lse = true; }
    else if (kind == KIND_SAMPLED_R) { is_draft = false; kk = local; lse = true; }
    else { is_draft = true; kk = local; lse = true; }   // KIND_CONF, KIND_CONF2
    // KIND_CONF2: the statistics at the request's temperature go to slot row
    // d + local of the request (the confidence's own in row local)
    k.sc2 = k.sc;
    k.slot2 = k.slot + d;
    if (kind == KIND_CONF2) {
        k.sc2.c32 = cT;
        k.sc2.sh = shT;
    }
    if constexpr (EE) kk += P.win_lo;   // the window's first position
    if (lse) {
        // confidence statistics are at T = 1 (scale_of's rule for those kinds)
        const bool conf = kind == KIND_CONF || kind == KIND_CONF2;
        k.sc.c32 = conf ? (float)LOG2E : cT;
        k.sc.sh = conf ? 0 : shT;
    } else {
        k.sc.c32 = 0.0f;
        k.sc.sh = 0;
    }
    // the request's first draft row and first target row
    const int64_t db = P.offs ? (int64_t)ld_scalar_i32(P.offs + b) : (int64_t)b * P.K;
    const int64_t tb = P.offs ? db + b : (int64_t)b * (P.K + 1);
    const int64_t row = is_draft ? db + kk : tb + kk;
    const char *row_start = (const char *)(is_draft ? P.draft : P.target) + row * (int64_t)P.V * (BF16 ? 2 : 4);
    const RowView<BF16> rv(row_start, P.V);
    k.vec = rv.vec;
    k.head = rv.head;
    k.nvec = rv.nvec;
    // The accept test needs this row's logit at the drafted token x; the
    // row's first chunk reads it (the others carry the merge identity, so
    // only one task per row waits on these two loads), and the finish kernel
    // has it from the merged partials.  x outside [0, V) is clamped here and
    // rejected as bad data by the scan.
    k.zx = __int_as_float(0x7fffffff);
    if ((kind == KIND_SAMPLED || kind == KIND_SAMPLED_R) && c == 0) {
        const int x = min(max(ld_scalar_i32(P.tokens + db + kk), 0), P.V - 1);
        k.zx = ld_scalar_logit<BF16>(row_start, x);
    }
    const int nbr = (int)ceil_div(k.nvec, WVEC);
    const int b0 = c * nb;
    k.b1 = std::max(std::min(nbr, b0 + nb), b0 + 1);
    return k;
}

__device__ __forceinline__ Stat finish_task(bool lse, const ArgmaxLane &am, const LseLane &ls, const LseScale &sc)
{
    Stat st;
    if (!lse) {
        const int nanf = wave_or(am.nanf);
        float best = am.best;
        int bidx = am.bidx;
        wave_argmax(best, bidx);
        st.m = nanf ? NAN : best;
        st.idx = bidx;
        st.s = 0.0;
    } else {
        const float M = wave_max(ls.M);
        double sl = 0.0;
        if (ls.M != -INFINITY) sl = ls.s * (double)__builtin_amdgcn_exp2f(scaled_exp(ls.M - M, sc));
        else if (ls.s != ls.s) sl = ls.s;
        st.m = M;
        st.idx = 0;
        st.s = wave_sum(sl);
    }
    return st;
}

// A sampled row's first chunk carries the logit at the drafted token in the
// partial's index; the other chunks carry the merge identity.
template <bool BF16>
__device__ __forceinline__ Stat finish_task(const Task<BF16> &k, const ArgmaxLane &am, const LseLane &ls)
{
    Stat st = finish_task(k.lse(), am, ls, k.sc);
    if (k.lse()) st.idx = __float_as_int(k.zx);
    return st;
}

// Reduces one batch of a task into the running lane state and stores the
// task's partial slot: after the task's last batch the reduced partial
// (plain store; the finish kernel reads it after the kernel boundary),
// before that a placeholder the last store overwrites (same wave, same
// address, so program order holds).  Storing on every batch keeps one store
// per batch on every path, so the compiler's load-wait counts stay exact and
// no wait ever covers a store.  The partial is wave-uniform (butterfly
// reductions), so every lane stores the same 16 bytes: one write.
// DUAL (confidence calls with temperatures; their rows are all log-sum-exp
// rows): every task keeps two statistics, ls at T = 1 and ls2 at scale sc2
// (its request's temperature for KIND_CONF2, else T = 1 again), and stores
// both, the second into slot row slot2 (for a KIND_CONF request a row the
// finish kernel does not read).  One path for every task keeps the
// compiler's wait counts exact, as in the single-statistic kernel.
template <bool BF16, bool DUAL>
__device__ __forceinline__ void consume(const Params &P, const Task<BF16> &k, int i, const uint4 (&raw)[UW],
                                        ArgmaxLane &am, LseLane &ls, LseLane &ls2)
{
    Stat st, st2;
    if constexpr (DUAL) {
        const RowView<BF16> rv = k.view(P.V);
        if (rv.batch_edge(i * WVEC, WVEC)) lse_batch2<BF16, true>(rv, i * WVEC, raw, k.sc, k.sc2, ls, ls2);
        else lse_batch2<BF16, false>(rv, i * WVEC, raw, k.sc, k.sc2, ls, ls2);
    } else if (k.lse()) {
        process_batch<BF16, true>(k.view(P.V), i * WVEC, raw, k.sc, ls);
    } else {
        process_batch<BF16, false>(k.view(P.V), i * WVEC, raw, k.sc, am);
    }
    if (i + 1 >= k.b1) {
        st = finish_task<BF16>(k, am, ls);
        if constexpr (DUAL) st2 = finish_task(true, am, ls2, k.sc2);
        am = ArgmaxLane();
        ls = LseLane();
        if constexpr (DUAL) ls2 = LseLane();
    } else {
        st.m = 0.0f;
        st.idx = 0;
        st.s = 0.0;
        st2 = st;
    }
    if constexpr (DUAL) P.ws.part[(int64_t)k.slot2 * P.cpr_max + k.c] = st2;
    P.ws.part[(int64_t)k.slot * P.cpr_max + k.c] = st;
}

// Four waves per SIMD (128 VGPRs) keep enough 16-byte loads in flight per CU
// to cover HBM latency; the register budget fits without spills.  DUAL: the
// instantiation for confidence calls with temperatures (two sums per row);
// with bf16's eight logits per vector its two sums need more than 128
// registers: at three waves per SIMD it spills least and ran fastest of
// two, three and four (measured on MI355X, B=64, K=16, V=128000).
constexpr int row_waves_per_eu(bool bf16, bool dual) { return bf16 && dual ? 3 : 4; }

template <bool BF16, bool EE, bool DUAL>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(row_waves_per_eu(BF16, DUAL), 8)))
void row_pass_kernel(Params P)
{
    extern __shared__ int plan_smem[];
    __shared__ int scan_tmp[NWAVE];
    Plan pl;
    pl.row_off = plan_smem;
    pl.info = plan_smem + P.B + 1;
    pl.c32 = (float *)(plan_smem + 2 * P.B + 1);
    const int offs_bad = make_plan<EE>(P, pl, scan_tmp);

    const int R = __builtin_amdgcn_readfirstlane(pl.row_off[P.B]);
    const uint32_t nwaves = gridDim.x * NWAVE;
    int cpr, nb;
    row_chunking(R, P.V, BF16, nwaves, P.mode == MODE_GREEDY ? 8 : 12, P.chunks, cpr, nb);
    // The divisions above run on the vector unit; their (uniform) results
    // are moved to scalar registers so everything derived stays scalar.
    cpr = __builtin_amdgcn_readfirstlane(cpr);
    nb = __builtin_amdgcn_readfirstlane(nb);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        P.ws.meta[0] = cpr;
        P.ws.meta[1] = nb;
        P.ws.meta[2] = offs_bad;
    }

    // Static assignment in rounds.  Task t is chunk t % cpr of row t / cpr.
    // Workgroups land on the CUs in blockIdx order, so blockIdx / row_cus is
    // a workgroup's dispatch slot on its CU; waves of earlier slots are older
    // and win more issue cycles, so slot group s gets n_s tasks per wave,
    // n_s = ceil(avg * (1 + skew * ((nslot - 1) / 2 - s))), non-increasing in
    // s.  Round k is run by the slot groups with n_s > k -- a prefix of the
    // waves, of size A_k -- and wave gw's round-k task is
    // pre_k + (gw + ROUND_SHIFT * k) mod A_k, with pre_k the tasks of the
    // earlier rounds (a rotation: each round's tasks go to its waves one to
    // one).  Without the rotation a wave would meet the same chunk position
    // in every round whenever A_k is a multiple of the chunks per row, and
    // chunk positions differ in work: the first chunk of a sampled row also
    // loads the logit at the drafted token, the last is usually short.  All
    // loop state is wave-uniform (scalar).
    const uint32_t ntask = (uint32_t)R * (uint32_t)cpr;
    const uint32_t gw = blockIdx.x * NWAVE + (uint32_t)__builtin_amdgcn_readfirstlane(wave_id());
    if (gw >= ntask) return;
    const int Q = max(P.row_cus, 1);
    const int nslot = min((int)ceil_div(gridDim.x, Q), SLOT_MAX);
    const int myslot = min((int)blockIdx.x / Q, nslot - 1);
    int nt[SLOT_MAX];        // tasks per wave of each slot group
    uint32_t gend[SLOT_MAX]; // end (in waves) of each slot group
    {
        const float avg = (float)ntask / (float)nwaves;
        uint32_t cover = 0;
#pragma unroll
        for (int g = 0; g < SLOT_MAX; ++g) {
            const float w = 1.0f + P.row_skew * (0.5f * (float)(nslot - 1) - (float)g);
            nt[g] = g < nslot ? max(1, (int)(avg * fmaxf(w, 0.0f) + 0.5f)) : 0;
            if (g > 0) nt[g] = min(nt[g], nt[g - 1]);
            gend[g] = g < nslot - 1 ? (uint32_t)((g + 1) * Q) * NWAVE : nwaves;
            const uint32_t gbeg = g == 0 ? 0u : (uint32_t)(g * Q) * NWAVE;
            if (g < nslot) cover += (uint32_t)nt[g] * (gend[g] - gbeg);
        }
        // rounding shortfall: more rounds for the first (fastest) group
        const uint32_t g0 = gend[0];
        if (cover < ntask) nt[0] += (int)ceil_div(ntask - cover, g0);
    }
    int mytasks = 0;
#pragma unroll
    for (int g = 0; g < SLOT_MAX; ++g)
        if (g == myslot) mytasks = nt[g];
    // waves active in round k: the slot groups with nt > k (a prefix)
    auto active = [&](int k) -> uint32_t {
        uint32_t a = 0;
#pragma unroll
        for (int g = 0; g < SLOT_MAX; ++g)
            if (g < nslot && nt[g] > k) a = gend[g];
        return a;
    };
    const int r0 = __builtin_amdgcn_readfirstlane((int)(gw / (uint32_t)cpr));
    const int c0 = (int)gw - r0 * cpr;

    // (kn, in) = the batch after batch i of task k in this wave's stream;
    // false past the stream's end.
    auto next_batch = [&](const Task<BF16> &k, int i, Task<BF16> &kn, int &in) -> bool {
        if (i + 1 < k.b1) {
            kn = k;
            in = i + 1;
            return true;
        }
        const int k1 = k.k + 1;
        if (k1 >= mytasks) return false;
        const uint32_t pre1 = k.pre + active(k.k);
        const uint32_t t = pre1 + (gw + ROUND_SHIFT * (uint32_t)k1) % active(k1);
        if (t >= ntask) return false;
        const int r = __builtin_amdgcn_readfirstlane((int)(t / (uint32_t)cpr));
        const int c = (int)t - r * cpr;
        kn = make_task<BF16, EE>(P, pl, r, c, nb);
        kn.k = k1;
        kn.pre = pre1;
        in = c * nb;
        return true;
    };

    // Steady state: [A, store, B] in flight when A is reduced, [B, store, A]
    // when B is.  Every step issues a batch, a store follows every
    // reduction (or stands in for one), and the loop has one exit, at its
    // bottom, so the compiler's wait counts stay exact: a reduction waits
    // for its own buffer only, never for the other buffer or a store.  Past
    // the stream's end the issue is a dummy: every lane loads the last vector
    // of a row already read (one cached line) and the batch is not reduced.
    Stat *const spare = (Stat *)(P.ws.meta + 4);
    Stat zero;
    zero.m = 0.0f;
    zero.idx = 0;
    zero.s = 0.0;
    uint4 A[UW], Bv[UW];
    Task<BF16> kA = make_task<BF16, EE>(P, pl, r0, c0, nb);
    kA.k = 0;
    kA.pre = 0;
    Task<BF16> kB = kA;
    int iA = c0 * nb, iB = iA;
    // stands in for a reduction's stores (one, or two in the DUAL kernel)
    auto stand_in = [&]() {
        *spare = zero;
        if constexpr (DUAL) *spare = zero;
    };
    bool vB = next_batch(kA, iA, kB, iB);
    issue_batch(kA.vec, kA.nvec, iA * WVEC, A);
    stand_in();
    issue_batch(kB.vec, kB.nvec, vB ? iB * WVEC : kB.nvec, Bv);
    ArgmaxLane am;
    LseLane ls, ls2;
    for (;;) {
        consume<BF16, DUAL>(P, kA, iA, A, am, ls, ls2);
        const bool vA = vB && next_batch(kB, iB, kA, iA);
        issue_batch(kA.vec, kA.nvec, vA ? iA * WVEC : kA.nvec, A);
        if (vB) consume<BF16, DUAL>(P, kB, iB, Bv, am, ls, ls2);
        else stand_in();
        vB = vA && next_batch(kA, iA, kB, iB);
        issue_batch(kB.vec, kB.nvec, vB ? iB * WVEC : kB.nvec, Bv);
        if (!vA) break;
    }
}

// ---------------------------------------------------------------------------
// Accept test and first-rejection scan of one request (one wave, lanes over
// the drafted positions), from the request's merged row statistics.
// ---------------------------------------------------------------------------

// Unusable row statistics: NaN or +inf present (m = NaN or +inf), nothing
// but -inf (m = -inf), or a normaliser that is not a positive finite number.
__device__ __forceinline__ bool stat_bad(const Stat &s, bool lse)
{
    if (!(s.m == s.m) || s.m == INFINITY || s.m == -INFINITY) return true;
    if (lse) return !(s.s > 0.0) || s.s == (double)INFINITY;
    return false;
}

__device__ __forceinline__ bool unif_ok(float u) { return u >= 0.0f && u < 1.0f; }

// rows: target rows 0..d (greedy) or target rows 0..d-1 then draft rows
// 0..d-1 (sampled), in LDS.  For a sampled request pq[k] receives
// (p_k(x_k), q_k(x_k)) for k < d.  Writes nothing to global memory.
// (x0, ua0, us0): lane l's drafted token and accept uniform at position l, and
// the request's draw uniform, loaded by the caller ahead of time.
__device__ ReqDesc scan_request(const Params &P, int b, const ReqPlan &q, const Stat *rows, float2 *pq,
                                const double *tab, int x0, float ua0, float us0)
{
    const int d = q.d;
    const int lane = lane_id();
    const int64_t tb = q.rb.db;
    ReqDesc desc = {SREQ_BAD, 0, -1, q.T};
    if (q.kind == KIND_BAD) return desc;

    if (q.kind == KIND_GREEDY) {
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
                    const int x = k0 == 0 ? x0 : P.tokens[tb + k];
                    bad |= (x < 0 || x >= P.V);
                    mism = (x != s.idx);
                }
            }
            const uint64_t mm = __ballot(mism);
            if (mm && n == d) n = k0 + __builtin_ctzll(mm);
        }
        if (!wave_or(bad)) desc = {SREQ_GREEDY, n, rows[n].idx, q.T};
        return desc;
    }

    // Sampled request (T > 0): accept k iff u_k < min(1, p_k(x)/q_k(x)), in
    // double from the row statistics and the two logits at x, with the same
    // exponent scale as the statistics.
    int bad = unif_ok(us0) ? 0 : 1;
    int n = d;
    const double c2 = scale_d(scale_of(q.kind, q.T));
    for (int k0 = 0; k0 < d; k0 += 64) {
        const int k = k0 + lane;
        const bool active = k < d;
        bool rej = false;
        if (active) {
            const int x = k0 == 0 ? x0 : P.tokens[tb + k];
            const float ua = k0 == 0 ? ua0 : P.u_accept[tb + k];
            const Stat st = rows[k], sd = rows[d + k];
            const bool lb = (x < 0 || x >= P.V) || !unif_ok(ua) || stat_bad(st, true) || stat_bad(sd, true);
            double a = 0.0, c = 0.0;
            if (!lb) {
                // logits at x, carried by the row partials
                const float zx = __int_as_float(st.idx);
                const float yx = __int_as_float(sd.idx);
                a = exp2_tab(((double)zx - (double)st.m) * c2, tab) / st.s;
                c = exp2_tab(((double)yx - (double)sd.m) * c2, tab) / sd.s;
                const double ratio = (c > 0.0) ? fmin(1.0, a / c) : (a > 0.0 ? 1.0 : 0.0);
                rej = !((double)ua < ratio);
            }
            bad |= lb;
            pq[k] = make_float2((float)a, (float)c);
        }
        const uint64_t rm = __ballot(active && rej);
        if (rm && n == d) n = k0 + __builtin_ctzll(rm);
    }
    if (!wave_or(bad)) desc = {n == d ? SREQ_BONUS : SREQ_RESID, n, -1, q.T};
    return desc;
}

// One wave writes request b's outputs: the accepted prefix, the emitted token
// at position n, -1 after it, num_accepted, and (sampled calls) p/q at the
// drafted tokens.  A bad request gets -1 everywhere and zero probabilities
// (in every slot it has: none when its packed offsets are unusable).
__device__ void write_outputs(const Params &P, int b, int d, const ReqBase &rb, const ReqDesc &desc,
                              const float2 *pq, int token)
{
    const int lane = lane_id();
    const int64_t ob = rb.tb, tb = rb.db;
    const bool bad = desc.state == SREQ_BAD;
    const int n = desc.n;
    for (int k = lane; k < rb.nout; k += 64)
        P.out_tokens[ob + k] = bad ? -1 : (k < n ? P.tokens[tb + k] : (k == n ? token : -1));
    if (P.mode == MODE_SAMPLE) {
        const bool sampled = desc.state == SREQ_RESID || desc.state == SREQ_BONUS;
        for (int k = lane; k < rb.nout - 1; k += 64) {
            const float2 v = (sampled && k < d) ? pq[k] : make_float2(0.0f, 0.0f);
            if (P.p_draft) P.p_draft[tb + k] = v.x;
            if (P.q_draft) P.q_draft[tb + k] = v.y;
        }
    }
    if (lane == 0) P.num_accepted[b] = bad ? -1 : n;
}

// Early-exit scan of one window (one wave, lanes over the window's
// positions).  Positions are taken in order and the first one that is
// rejected or holds bad data ends the request; nothing after it is looked
// at, so bad data there is not reported.  rows: the window's rows as the
// plan lays them out (position lo + j at j; sampled draft rows after the q.d
// target rows; a greedy request's bonus row at q.d when the window reaches
// the depth).  pq[j] receives (p, q) at the drafted token of position lo + j.
// (x0, ua0): lane l's drafted token and accept uniform at position lo + l;
// us0: the draw uniform.  Returned positions n are absolute.
__device__ ReqDesc scan_window(const Params &P, int b, const ReqPlan &q, const Stat *rows, float2 *pq,
                               const double *tab, int x0, float ua0, float us0)
{
    const int nd = q.d, lo = q.lo;
    const int lane = lane_id();
    const int64_t tb = q.rb.db + lo;
    ReqDesc desc = {SREQ_BAD, 0, -1, q.T};
    if (q.kind == KIND_BAD) return desc;
    if (q.kind == KIND_DONE) return {SREQ_DONE, 0, -1, q.T};
    const bool greedy = q.kind == KIND_GREEDY;
    const double c2 = greedy ? 0.0 : scale_d(scale_of(q.kind, q.T));
    int stop = nd;          // first position (relative) that rejects or is bad
    bool stop_bad = false;
    for (int k0 = 0; k0 < nd; k0 += 64) {
        const int k = k0 + lane;
        bool badk = false, rej = false;
        if (k < nd) {
            const int x = k0 == 0 ? x0 : P.tokens[tb + k];
            const bool xbad = x < 0 || x >= P.V;
            const Stat st = rows[k];
            if (greedy) {
                badk = xbad || stat_bad(st, false);
                rej = x != st.idx;
            } else {
                const float ua = k0 == 0 ? ua0 : P.u_accept[tb + k];
                const Stat sd = rows[nd + k];
                badk = xbad || !unif_ok(ua) || stat_bad(st, true) || stat_bad(sd, true);
                double a = 0.0, c = 0.0;
                if (!badk) {
                    const float zx = __int_as_float(st.idx);
                    const float yx = __int_as_float(sd.idx);
                    a = exp2_tab(((double)zx - (double)st.m) * c2, tab) / st.s;
                    c = exp2_tab(((double)yx - (double)sd.m) * c2, tab) / sd.s;
                    const double ratio = (c > 0.0) ? fmin(1.0, a / c) : (a > 0.0 ? 1.0 : 0.0);
                    rej = !((double)ua < ratio);
                }
                pq[k] = make_float2((float)a, (float)c);
            }
        }
        const uint64_t ev = __ballot(k < nd && (badk || rej));
        if (ev && stop == nd) {
            const int f = __builtin_ctzll(ev);
            stop = k0 + f;
            stop_bad = (__ballot(badk) >> f) & 1;
        }
    }
    if (stop_bad) return desc;
    if (stop < nd) {
        if (greedy) return {SREQ_GREEDY, lo + stop, rows[stop].idx, q.T};
        if (!unif_ok(us0)) return desc;
        return {SREQ_RESID, lo + stop, -1, q.T};
    }
    if (!q.fin) return {SREQ_CONT, lo + nd, -1, q.T};
    if (greedy) {
        const Stat s = rows[nd];
        if (stat_bad(s, false)) return desc;
        return {SREQ_GREEDY, lo + nd, s.idx, q.T};
    }
    if (!unif_ok(us0)) return desc;
    return {SREQ_BONUS, lo + nd, -1, q.T};
}

// One wave writes what an early-exit window decides for request b.
// (p, q) for the window's positions up to the stop (0 after it and for
// greedy requests); when the request ends here, the outputs as the one-pass
// call writes them, zero probabilities past the window (never read) and,
// for a bad request, zero probabilities for the earlier windows too.
__device__ void write_window(const Params &P, int b, const ReqPlan &q, const ReqDesc &desc, const float2 *pq,
                             int token)
{
    const int lane = lane_id();
    const int64_t ob = q.rb.tb, tb = q.rb.db;
    const int K = q.rb.nout - 1;
    if (desc.state == SREQ_DONE) return;
    const bool bad = desc.state == SREQ_BAD, cont = desc.state == SREQ_CONT;
    const int n = desc.n, lo = q.lo, hi = q.lo + q.d;
    if (P.mode == MODE_SAMPLE) {
        const bool sampled = !bad && q.kind == KIND_SAMPLED;
        for (int k = lane; k < K; k += 64) {
            if (k < lo && !bad) continue;       // an earlier window's position
            if (cont && k >= hi) continue;      // a later window's position
            const float2 v = (sampled && k < hi && k <= n) ? pq[k - lo] : make_float2(0.0f, 0.0f);
            if (P.p_draft) P.p_draft[tb + k] = v.x;
            if (P.q_draft) P.q_draft[tb + k] = v.y;
        }
    }
    if (cont) return;
    for (int k = lane; k <= K; k += 64)
        P.out_tokens[ob + k] = bad ? -1 : (k < n ? P.tokens[tb + k] : (k == n ? token : -1));
    if (lane == 0) P.num_accepted[b] = bad ? -1 : n;
}

// ---------------------------------------------------------------------------
// Finish kernel: merge, accept scan, sampler chunk sums.
// ---------------------------------------------------------------------------

// Merge of two partial statistics of one row: (max, lowest argmax) with NaN
// propagated, or (max, sum relative to the max) rescaled to the larger max.
// Log-sum-exp partials carry the logit at the drafted token in idx (the
// row's first chunk; the other chunks and the merge identity carry
// 0x7fffffff).
__device__ __forceinline__ Stat merge2(Stat a, Stat b, bool lse, double cs, const double *tab)
{
    if (!lse) {
        if (!(a.m == a.m)) return a;
        if (!(b.m == b.m)) return b;
        argmax_merge(a.m, a.idx, b.m, b.idx);
        return a;
    }
    const int zx = (a.idx != 0x7fffffff) ? a.idx : b.idx;
    a.idx = b.idx = zx;
    if (b.m > a.m) {
        const Stat t = a;
        a = b;
        b = t;
    }
    // The rescale factor 2^((b.m - a.m) * cs) <= 1 in fp32 (hardware exp2,
    // within 2 ulp; an argument below the fp32 range gives 0): it moves S by
    // at most 2.4e-7 relative, as the row pass's own lane rescales do.
    if (b.m == -INFINITY) a.s += (b.s != b.s) ? b.s : 0.0;   // empty (or NaN-poisoned) partial
    else a.s += b.s * (double)__builtin_amdgcn_exp2f((float)(((double)b.m - (double)a.m) * cs));
    return a;
}

constexpr int MERGE_LOADS = 8;   // row-pass partials loaded at once per merging thread

// Threads per row of the merge: the largest power of two up to 64 (and up
// to the workspace's column count) with a group of rows_max rows fitting
// half the workgroup, for a request of at most rows_max rows.  It depends on
// launch constants only, so the merge's first loads wait on no device value.
__device__ __forceinline__ int merge_tpr(int rows_max, int cpr_max)
{
    int tpr = 1;
    while (tpr < 64 && tpr < cpr_max && 2 * tpr * rows_max <= WG) tpr <<= 1;
    return tpr;
}

// The first MERGE_LOADS partials of every thread of the merge's first row
// group (row tid / tpr, columns tid % tpr + i * tpr), loaded at kernel start
// before the chunk count and the request's row count are known: every slot
// read lies in request b's own slot range (rows_max rows of cpr_max
// columns); those past the request's rows or the chunk count are read and
// not folded.
struct MergePre {
    Stat v[MERGE_LOADS];
};

__device__ __forceinline__ MergePre merge_prefetch(const Params &P, int pre, int rows_max, int tpr)
{
    MergePre m;
    const int r = min((int)threadIdx.x / tpr, rows_max - 1), l = threadIdx.x & (tpr - 1);
    const Stat *pp = P.ws.part + (int64_t)(pre + r) * P.cpr_max;
#pragma unroll
    for (int i = 0; i < MERGE_LOADS; ++i) m.v[i] = pp[min(l + i * tpr, P.cpr_max - 1)];
    return m;
}

// Merges the row-pass partials of request b's rows into rows_s (all threads;
// tpr threads per row, each folding every tpr-th partial in chunk order, then
// a butterfly over the tpr lanes; rows in groups of WG / tpr).  The first
// MERGE_LOADS partials of each thread of the first group come from
// merge_prefetch.  Every workgroup of a request performs the same operations
// in the same order, so all of them hold identical statistics.
// Rows from `split` on use the scale cs2 (a confidence call's statistics at
// a request's own temperature, KIND_CONF2); the others use cs.
__device__ void merge_rows(const Params &P, int pre, int rows, int tpr, int cpr, bool lse, double cs,
                           double cs2, int split, const double *tab, const MergePre &first, Stat *rows_s)
{
    const int tid = threadIdx.x;
    const int G = WG / tpr;
    const Stat ident = {-INFINITY, 0x7fffffff, 0.0};
    for (int g0 = 0; g0 < rows; g0 += G) {
        const int r = g0 + tid / tpr, l = tid & (tpr - 1);
        const double csr = r < split ? cs : cs2;
        Stat acc = ident;
        if (r < rows) {
            int j0 = l;
            if (g0 == 0) {
#pragma unroll
                for (int i = 0; i < MERGE_LOADS; ++i)
                    if (l + i * tpr < cpr) acc = merge2(acc, first.v[i], lse, csr, tab);
                j0 += MERGE_LOADS * tpr;
            }
            // MERGE_LOADS partials in flight per thread (clamped index, no
            // branch), folded in chunk order
            const Stat *pp = P.ws.part + (int64_t)(pre + r) * P.cpr_max;
            for (; j0 < cpr; j0 += MERGE_LOADS * tpr) {
                Stat v[MERGE_LOADS];
#pragma unroll
                for (int i = 0; i < MERGE_LOADS; ++i) v[i] = pp[min(j0 + i * tpr, cpr - 1)];
#pragma unroll
                for (int i = 0; i < MERGE_LOADS; ++i)
                    if (j0 + i * tpr < cpr) acc = merge2(acc, v[i], lse, csr, tab);
            }
        }
        // butterfly over the tpr lanes of the row (levels with 2^L < tpr;
        // every workgroup of the request runs the same sequence)
        auto level = [&](auto lv) {
            constexpr int L = decltype(lv)::value;
            if ((1 << L) < tpr) {
                Stat other;
                other.m = xchg_f<L>(acc.m);
                other.idx = xchg_i<L>(acc.idx);
                other.s = xchg_d<L>(acc.s);
                acc = merge2(acc, other, lse, csr, tab);
            }
        };
        level(std::integral_constant<int, 0>());
        level(std::integral_constant<int, 1>());
        level(std::integral_constant<int, 2>());
        level(std::integral_constant<int, 3>());
        level(std::integral_constant<int, 4>());
        level(std::integral_constant<int, 5>());
        if (r < rows && l == 0) rows_s[r] = acc;
    }
    __syncthreads();
}

// Sampler units: a wave's contiguous run of UNIT_E logits of the drawn row
// pair (UNIT_V 16-byte vectors), read in SUB steps of NV vectors per lane;
// step s, slot j, lane l reads vector (s*NV + j)*64 + l of the unit, so every
// load instruction covers 64 consecutive vectors.
template <bool BF16>
constexpr int unit_v() { return UNIT_E / RowView<BF16>::EPV; }
template <bool BF16>
constexpr int sampler_nv() { return SE / RowView<BF16>::EPV; }

// Branch-free loads (clamped index) of vectors v0 + j*stride, j < N.
template <bool BF16, int N>
__device__ __forceinline__ void issue_vecs(const RowView<BF16> &rv, int v0, int stride, uint4 (&raw)[N])
{
#pragma unroll
    for (int j = 0; j < N; ++j) raw[j] = ld_plain(rv.vec + min(v0 + j * stride, rv.nvec - 1));
}

// Elements of vector vi as fp32, -inf outside the row (selects, no
// branch); NaN / +inf flagged.  With ALIGNED (every row starts on a vector
// boundary and V fills whole vectors) only vectors past the row's end hold
// elements outside it, so the test is one per vector, on the raw data.
template <bool BF16, bool ALIGNED = false>
__device__ __forceinline__ void chunk_vec(const RowView<BF16> &rv, int vi, const uint4 &raw_in,
                                          float (&f)[RowView<BF16>::EPV], int &flag)
{
    if constexpr (ALIGNED) {
        constexpr uint32_t NEG = BF16 ? 0xff80ff80u : 0xff800000u;   // -inf in every element
        const bool in = vi < rv.nvec;
        const uint4 raw = make_uint4(in ? raw_in.x : NEG, in ? raw_in.y : NEG, in ? raw_in.z : NEG,
                                     in ? raw_in.w : NEG);
        unpack<BF16>(raw, f);
    } else {
        unpack<BF16>(raw_in, f);
#pragma unroll
        for (int e = 0; e < RowView<BF16>::EPV; ++e) {
            const int x = rv.elem(vi, e);
            f[e] = ((unsigned)x < (unsigned)rv.V) ? f[e] : -INFINITY;
        }
    }
#pragma unroll
    for (int e = 0; e < RowView<BF16>::EPV; ++e) flag |= (!(f[e] == f[e]) || f[e] == INFINITY);
}

// Draft logits on the target row's vector grid.  With ALIGNED (V * element
// size a multiple of 16) every row starts on a vector boundary and that is
// the draft row's own grid; otherwise the draft row is read by token index.
template <bool BF16>
struct DraftChunk {
    RowView<BF16> ry;
    const char *yrow;
};

template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void draft_vec(const DraftChunk<BF16> &dc, const RowView<BF16> &rz, int vi,
                                          const uint4 &raw, float (&g)[RowView<BF16>::EPV])
{
    int fl = 0;
    if constexpr (ALIGNED) {
        chunk_vec<BF16, true>(dc.ry, vi, raw, g, fl);
    } else {
#pragma unroll
        for (int e = 0; e < RowView<BF16>::EPV; ++e) {
            const int x = rz.elem(vi, e);
            const float v = load_logit<BF16>(dc.yrow, min(max(x, 0), rz.V - 1));   // branch-free
            g[e] = (x >= 0 && x < rz.V) ? v : -INFINITY;
        }
    }
}

// Drawn row pair of a request: target row n (and draft row n for a residual
// draw), with the exponent constants of P = 2^((z - Mz) cd), Q = 2^((y - My) cd).
// Two forms of the exponent, used alike by the unit sums and the rescan:
//  * z * cd - fl(Mz * cd) (one FMA): the rounding of fl(Mz * cd) is one
//    offset common to every term of the row, which cancels between the row's
//    terms and its sum; it stays negligible next to the row pass's estimate
//    of Sz/Sy while |Mz cd|, |My cd| < 2^28;
//  * (z - Mz) * cd (exact): the difference of two widened fp32 values is exact
//    in double wherever the term is not vanishingly small.  Taken when either
//    |M cd| reaches 2^28 (very large |M| / T), and always for a bonus draw,
//    whose unit sums offset each lane by its own running maximum.
template <bool BF16>
struct DrawRows {
    RowView<BF16> rz;
    DraftChunk<BF16> dc;
    double cd, mzc, myc;     // log2(e)/T and the row maxima times it
    double cd5, mzc5, myc5;  // the same times 512 (arguments of exp2_512)
    double mz, my;           // the row maxima
    bool exact;              // exact-difference exponents
    __device__ void scale()
    {
        cd5 = cd * EXP2_TAB;
        mzc5 = mzc * EXP2_TAB;
        myc5 = myc * EXP2_TAB;
    }
};

constexpr double EXACT_EXP_AT = 0x1p28;

template <bool EXACT>
__device__ __forceinline__ double draw_exp_arg(float v, double m, double mc5, double cd5)
{
    if constexpr (EXACT) return ((double)v - m) * cd5;
    else return fma((double)v, cd5, -mc5);
}

template <bool BF16>
__device__ __forceinline__ DrawRows<BF16> draw_rows(const Params &P, int64_t tb, int64_t db, const ReqDesc &desc,
                                                    float Mz, float My)
{
    DrawRows<BF16> r;
    const int64_t esz = BF16 ? 2 : 4;
    r.rz = RowView<BF16>((const char *)P.target + (tb + desc.n) * P.V * esz, P.V);
    r.dc.yrow = (const char *)P.draft + (db + desc.n) * P.V * esz;
    r.dc.ry = RowView<BF16>(r.dc.yrow, P.V);
    r.cd = LOG2E / (double)desc.T;
    r.mz = (double)Mz;
    r.my = (double)My;
    r.mzc = r.mz * r.cd;
    r.myc = r.my * r.cd;
    r.exact = __builtin_fmax(__builtin_fabs(r.mzc), __builtin_fabs(r.myc)) >= EXACT_EXP_AT;
    r.scale();
    return r;
}

// Residual sums over a wave's run of VT vectors per lane (vector i of the
// run is vu + 64 i + lane), loads one vector ahead of the arithmetic: the
// unit passes of a whole batch start at once, and if every wave issued its
// whole run up front, every wave would wait for the whole burst (a row pair
// per request, tens of MB) before its first term; one vector ahead, the
// first terms start after a fraction of it and the rest streams under the
// fp64 work.
template <bool BF16, bool ALIGNED, bool EXACT, int VT>
__device__ __forceinline__ void resid_terms(const DrawRows<BF16> &dr, double rho_hat, int vu, const double *tab,
                                            int &flag, double &dsum, double &bq, double &sz, double &sy)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const int lane = lane_id();
    uint4 zc, yc = make_uint4(0, 0, 0, 0);
    {
        uint4 t1[1], t2[1];
        issue_vecs<BF16, 1>(dr.rz, vu + lane, 64, t1);
        zc = t1[0];
        if (ALIGNED) {
            issue_vecs<BF16, 1>(dr.dc.ry, vu + lane, 64, t2);
            yc = t2[0];
        }
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
        uint4 zn = zc, yn = yc;
        if (i + 1 < VT) {
            uint4 t1[1], t2[1];
            issue_vecs<BF16, 1>(dr.rz, vu + (i + 1) * 64 + lane, 64, t1);
            zn = t1[0];
            if (ALIGNED) {
                issue_vecs<BF16, 1>(dr.dc.ry, vu + (i + 1) * 64 + lane, 64, t2);
                yn = t2[0];
            }
        }
        const int vi = vu + i * 64 + lane;
        float f[EPV], g[EPV];
        // one vector at a time: unbounded interleaving of the fp64
        // exponentials would cost occupancy
        __builtin_amdgcn_sched_barrier(0);
        chunk_vec<BF16, ALIGNED>(dr.rz, vi, zc, f, flag);
        draft_vec<BF16, ALIGNED>(dr.dc, dr.rz, vi, yc, g);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const double p = exp2_512(draw_exp_arg<EXACT>(f[e], dr.mz, dr.mzc5, dr.cd5), tab);
            const double q = exp2_512(draw_exp_arg<EXACT>(g[e], dr.my, dr.myc5, dr.cd5), tab);
            sz += p;
            sy += q;
            // t > 0: add t to d and q to bq; else add zeros.  One select
            // builds the 0/1 multiplier (its low word is 0 either way), and
            // t * 1 = t, t * 0 = +-0 keep the sums bit for bit those of
            // adding max(t, 0) and (t > 0 ? q : 0).
            const double t = fma(-rho_hat, q, p);
            const double one = __longlong_as_double(t > 0.0 ? 0x3ff0000000000000ll : 0ll);
            dsum = fma(t, one, dsum);
            bq = fma(q, one, bq);
        }
        zc = zn;
        yc = yn;
    }
}

// One wave's run of the drawn row pair: NSTEP steps of NV vectors per lane
// from vector vu (a whole unit by default, UNIT_V vectors).  Residual draw:
// the sums d, bq, sz, sy (rho_hat from the row pass).  Bonus draw: the run's
// maximum and the sum of P relative to it (each lane keeps a running
// maximum; the wave rescales to the run's).
template <bool BF16, bool ALIGNED, int NSTEP = SUB, int NV = sampler_nv<BF16>()>
__device__ ChunkPart unit_sums(const DrawRows<BF16> &dr, bool resid, double rho_hat, int vu, const double *tab)
{
    constexpr int EPV = RowView<BF16>::EPV;
    const int lane = lane_id();
    ChunkPart part;
    part.pad[0] = part.pad[1] = 0;
    int flag = 0;
    if (resid) {
        double dsum = 0.0, bq = 0.0, sz = 0.0, sy = 0.0;
        if (dr.exact) resid_terms<BF16, ALIGNED, true, NSTEP * NV>(dr, rho_hat, vu, tab, flag, dsum, bq, sz, sy);
        else resid_terms<BF16, ALIGNED, false, NSTEP * NV>(dr, rho_hat, vu, tab, flag, dsum, bq, sz, sy);
        part.d = wave_sum(dsum);
        part.bq = wave_sum(bq);
        part.sz = wave_sum(sz);
        part.sy = wave_sum(sy);
        part.m = 0.0f;
        part.bad = 0;   // the residual rows were checked by the row pass
    } else {
        float m = -INFINITY;
        double s = 0.0;
        uint4 rz[NSTEP][NV];
#pragma unroll
        for (int u = 0; u < NSTEP; ++u) issue_vecs<BF16, NV>(dr.rz, vu + u * NV * 64 + lane, 64, rz[u]);
#pragma unroll
        for (int u = 0; u < NSTEP; ++u) {
            const int v0 = vu + u * NV * 64 + lane;
            float f[NV][EPV];
            float ml = -INFINITY;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                chunk_vec<BF16, ALIGNED>(dr.rz, v0 + j * 64, rz[u][j], f[j], flag);
#pragma unroll
                for (int e = 0; e < EPV; ++e) ml = fmaxf(ml, f[j][e]);
            }
            if (ml > m) {
                if (m != -INFINITY) s *= exp2_tab(((double)m - (double)ml) * dr.cd, tab);
                m = ml;
            }
            if (m != -INFINITY && m != INFINITY) {
                const double md = (double)m;
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) s += exp2_512(draw_exp_arg<true>(f[j][e], md, 0.0, dr.cd5), tab);
            }
        }
        const float M = wave_max(m);
        if (m != -INFINITY && M != INFINITY) s *= exp2_tab(((double)m - (double)M) * dr.cd, tab);
        else s = 0.0;
        part.d = part.bq = part.sy = 0.0;
        part.sz = wave_sum(s);
        part.m = M;
        part.bad = wave_or(flag);
    }
    return part;
}

// A unit's sums by S = P.usplit waves of one workgroup (S in {1, 2, 4}, a
// divisor of the four waves): wave slot c * 4 + w takes part slot % S of unit
// slot / S.  Small batches split their units so that more waves share the
// fp64 work and the latency of one unit's pass shrinks.  The parts meet in
// LDS: residual sums add; bonus parts rescale to the largest maximum.  Every
// wave of the workgroup must call this (it holds a workgroup barrier when
// S > 1); waves past the last unit contribute nothing.  Without SPLIT the
// unit is wave slot c * 4 + w itself, S = 1, and the caller has already
// retired the waves past the last unit.
template <bool BF16, bool ALIGNED, bool SPLIT>
__device__ void unit_sums_store(const Params &P, int b, int c, const DrawRows<BF16> &dr, bool resid, double rho_hat,
                                const double *tab, ChunkPart *sh)
{
    constexpr int UV = unit_v<BF16>(), NV = sampler_nv<BF16>();
    static_assert(SUB == 2 && NV % 2 == 0, "a unit splits into halves and quarters of its steps");
    if constexpr (!SPLIT) {
        const int unit = c * NWAVE + wave_id();
        const ChunkPart pp = unit_sums<BF16, ALIGNED>(dr, resid, rho_hat, unit * UV, tab);
        if (lane_id() == 0) P.ws.cp[(int64_t)b * P.cs + unit] = pp;
        return;
    }
    const int S = P.usplit, w = wave_id(), lane = lane_id();
    const int slot = c * NWAVE + w, unit = slot / S, part = slot - unit * S;
    const bool active = unit < P.cs;
    ChunkPart pp = {};
    if (active) {
        const int vu = unit * UV + part * (UV / S);
        if (S == 2) pp = unit_sums<BF16, ALIGNED, 1, NV>(dr, resid, rho_hat, vu, tab);
        else pp = unit_sums<BF16, ALIGNED, 1, NV / 2>(dr, resid, rho_hat, vu, tab);
    }
    ChunkPart *dst = P.ws.cp + (int64_t)b * P.cs + unit;
    if (lane == 0) sh[w] = pp;
    __syncthreads();
    if (!active || part != 0 || lane != 0) return;
    ChunkPart t = sh[w];
    for (int i = 1; i < S; ++i) {
        const ChunkPart o = sh[w + i];
        if (resid) {
            t.d += o.d;
            t.bq += o.bq;
            t.sz += o.sz;
            t.sy += o.sy;
        } else {
            t.bad |= o.bad;
            if (o.m == -INFINITY) continue;
            if (t.m == -INFINITY) {
                t.m = o.m;
                t.sz = o.sz;
            } else if (o.m > t.m) {
                t.sz = t.sz * exp2_tab(((double)t.m - (double)o.m) * dr.cd, tab) + o.sz;
                t.m = o.m;
            } else {
                t.sz += o.sz * exp2_tab(((double)o.m - (double)t.m) * dr.cd, tab);
            }
        }
    }
    *dst = t;
}

// Early-exit calls, last window: the sampler units of a request that ended
// in an earlier window, from the draw record that window wrote (workgroup
// (c, b), unit 4c + wave, as in the finish kernel's unit part).
template <bool BF16, bool ALIGNED, bool SPLIT>
__device__ void units_from_record(const Params &P, int b, int c, double *tab, ChunkPart *sh)
{
    const DrawRec rec = P.ws.rec[b];
    if (rec.state != SREQ_RESID && rec.state != SREQ_BONUS) return;
    // fp64 unit work: back to normal issue priority, so the merge and scan
    // of the window's own requests are not held up
    __builtin_amdgcn_s_setprio(0);
    init_exp2_table(tab);
    if (!SPLIT && c * NWAVE + wave_id() >= P.cs) return;
    const bool resid = rec.state == SREQ_RESID;
    const ReqDesc desc = {rec.state, rec.n, -1, rec.T};
    const DrawRows<BF16> dr = draw_rows<BF16>(P, rec.tb, rec.db, desc, rec.mz, rec.my);
    unit_sums_store<BF16, ALIGNED, SPLIT>(P, b, c, dr, resid, rec.rho_hat, tab, sh);
}

// Workgroup (c, b):
//  1. merges request b's row statistics from the row-pass partials (every
//     workgroup of the request does this itself, so none waits on another);
//  2. wave 0 runs the accept test and first-rejection scan; workgroup c = 0
//     writes the request's outputs (the drawn token, if any, comes from the
//     draw kernel) and the record the draw kernel reads;
//  3. for a request that draws a token (sampled calls), each wave sums one
//     unit of the drawn row pair in fp64 (unit 4c + wave).
template <bool BF16, bool ALIGNED, bool EE, bool SPLIT>
__global__ __launch_bounds__(WG) void finish_kernel(Params P)
{
    extern __shared__ Stat rows_s[];   // [2K + 1] merged row statistics, then [K] (p, q) pairs
    __shared__ double tab[EXP2_TAB];
    __shared__ ReqDesc sh_desc;
    __shared__ ChunkPart sh_parts[NWAVE];
    float2 *pq_s = (float2 *)(rows_s + 2 * P.K + 1);
    const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    // The merge and the scan are a short latency chain that every unit of the
    // request waits on; fp64 unit work of other workgroups on the same SIMD
    // would otherwise delay it.  Raised issue priority until the units start.
    __builtin_amdgcn_s_setprio(3);
    // The request's plan arguments are the first loads issued, so the wait
    // for them covers nothing else; the row pass's chunking, the merge's
    // first partials and the scan's inputs are issued after them and return
    // while the plan and the table are computed.
    const PlanArgs pa = plan_loads<EE>(P, b);
    const int cpr = P.ws.meta[0];
    const int offs_bad = P.offs ? P.ws.meta[2] : 0;   // the row pass's verdict on packed offsets
    // request b's partials start at slot row b * (2K + 1)
    const int pre = b * (2 * P.K + 1);
    // rows a request merges: at most K + 1 in greedy calls, 2K + 1 otherwise
    const int rows_max = P.mode == MODE_GREEDY ? P.K + 1 : 2 * P.K + 1;
    const int tpr = merge_tpr(rows_max, P.cpr_max);
    const MergePre first = merge_prefetch(P, pre, rows_max, tpr);
    // the scan's inputs for positions lo..lo+63, issued with the plan's loads
    // so their latencies overlap each other, the table and the merge; every
    // wave loads them (no branch), from a stand-in where an argument is
    // unused or absent, and only wave 0's are used.  (The packed layout's
    // positions depend on the request's offsets: loaded after the plan.)
    const int lo = EE ? P.win_lo : 0;
    const int l = min(lo + lane_id(), max(P.K - 1, 0));
    const bool has_tok = P.mode != MODE_CONF && P.K > 0 && !P.offs;
    const bool has_u = P.mode == MODE_SAMPLE && P.K > 0 && !P.offs;
    const int32_t *tokp = has_tok ? P.tokens + (int64_t)b * P.K + l : &k_stand_in;
    const float *uap = has_u ? P.u_accept + (int64_t)b * P.K + l : (const float *)&k_stand_in;
    const float *usp = P.mode == MODE_SAMPLE ? P.u_sample + b : (const float *)&k_stand_in;
    int x0 = *tokp;
    float ua0 = *uap;
    const float us0 = *usp;
    // the fp64 exp2 table serves the accept test and the sampler of sampled
    // calls (the merge rescales with the fp32 exp2).  Wave 0 fills it while
    // the loads above are in flight; the merge's closing barrier publishes
    // it with the merged rows.
    if (P.mode == MODE_SAMPLE && wave_id() == 0) fill_exp2_table(tab);
    const ReqPlan q = plan_request<EE>(P, b, offs_bad != 0, pa);
    if (P.offs && q.d > 0) {
        const int64_t i = q.rb.db + min(lo + lane_id(), lo + q.d - 1);
        x0 = P.tokens[i];
        ua0 = P.mode == MODE_SAMPLE ? P.u_accept[i] : 0.0f;
    }
    if (q.kind == KIND_DONE) {   // early-exit calls: ended in an earlier window
        if (c == 0 && tid == 0) P.alive_out[b] = 0;
        if (EE && P.ee_last && P.mode == MODE_SAMPLE) units_from_record<BF16, ALIGNED, SPLIT>(P, b, c, tab, sh_parts);
        return;
    }
    const bool lse = q.kind == KIND_SAMPLED || q.kind == KIND_CONF || q.kind == KIND_SAMPLED_R ||
                     q.kind == KIND_CONF2;
    if (q.kind == KIND_SAMPLED_R) {
        // draft rows 0..d-1: the given statistics, with the draft logit at the
        // drafted token in idx (the row pass's convention; a token outside
        // [0, V) is clamped here and rejected by the scan); merge_rows' barrier
        // publishes them with the merged target rows.  A record taken at
        // another temperature than the request's (the plan checked the first)
        // counts as a NaN statistic: the request is bad.
        const int64_t esz = P.bf16 ? 2 : 4;
        for (int k = tid; k < q.d; k += WG) {
            Stat st = P.dstats_in[(int64_t)b * P.K + k];
            if (st.idx != __float_as_int(q.T)) st.m = NAN;
            const int x = min(max(P.tokens[(int64_t)b * P.K + k], 0), P.V - 1);
            const char *yrow = (const char *)P.draft + ((int64_t)b * P.K + k) * P.V * esz;
            st.idx = __float_as_int(load_logit_dt(yrow, P.bf16 != 0, x));
            rows_s[q.d + k] = st;
        }
    }
    // a KIND_CONF2 request also merges its statistics at its temperature,
    // slot rows d .. 2d - 1
    const bool conf2 = q.kind == KIND_CONF2;
    const double cs = lse ? scale_d(scale_of(q.kind, q.T)) : 0.0;
    const double cs2 = conf2 ? scale_d(scale_of(KIND_SAMPLED, q.T)) : cs;
    merge_rows(P, pre, conf2 ? 2 * q.d : q.rows, tpr, cpr, lse, cs, cs2, conf2 ? q.d : 0x7fffffff, tab, first,
               rows_s);

    if (P.mode == MODE_CONF) {
        for (int k = tid; k < P.K; k += WG) {
            const bool have = q.kind != KIND_BAD && k < q.d;
            if (P.conf) {
                float v;
                if (q.kind == KIND_BAD) v = NAN;
                else if (k >= q.d) v = 0.0f;
                else v = stat_bad(rows_s[k], true) ? NAN : (float)(1.0 / rows_s[k].s);
                P.conf[(int64_t)b * P.K + k] = v;
            }
            if (P.dstats_out) {
                // the statistics at the request's temperature (KIND_CONF2:
                // merged rows d..2d-1), else at T = 1; the record carries the
                // temperature it was taken at
                const int r = q.kind == KIND_CONF2 ? q.d + k : k;
                Stat st;
                st.m = have ? rows_s[r].m : NAN;
                st.idx = __float_as_int(q.kind == KIND_CONF2 ? q.T : 1.0f);
                st.s = have ? rows_s[r].s : NAN;
                P.dstats_out[(int64_t)b * P.K + k] = st;
            }
        }
        return;
    }
    if (wave_id() == 0) {
        const ReqDesc dsc = EE ? scan_window(P, b, q, rows_s, pq_s, tab, x0, ua0, us0)
                               : scan_request(P, b, q, rows_s, pq_s, tab, x0, ua0, us0);
        if (lane_id() == 0) sh_desc = dsc;
    }
    __syncthreads();
    const ReqDesc desc = sh_desc;
    const bool draw = desc.state == SREQ_RESID || desc.state == SREQ_BONUS;
    const bool resid = desc.state == SREQ_RESID;
    const int d = q.d;
    const int nl = desc.n - q.lo;   // the drawn position within the window's rows
    const Stat sz_row = rows_s[draw ? nl : 0];
    const Stat sy_row = resid ? rows_s[d + nl] : sz_row;
    const double rho_hat = resid ? sz_row.s / sy_row.s : 0.0;
    if (c == 0 && wave_id() == 0) {
        const int token = desc.state == SREQ_GREEDY ? desc.emit : -1;
        if constexpr (EE) {
            write_window(P, b, q, desc, pq_s, token);
            if (lane_id() == 0) P.alive_out[b] = desc.state == SREQ_CONT;
        } else {
            write_outputs(P, b, d, q.rb, desc, pq_s, token);
        }
        if (P.mode == MODE_SAMPLE && lane_id() == 0) {
            DrawRec r;
            r.state = desc.state;
            r.n = desc.n;
            r.T = desc.T;
            r.mz = resid ? sz_row.m : 0.0f;
            r.my = resid ? sy_row.m : 0.0f;
            r.tb = (int32_t)q.rb.tb;
            r.db = (int32_t)q.rb.db;
            r.nout = q.rb.nout;
            r.pad[0] = r.pad[1] = 0;
            r.rho_hat = rho_hat;
            P.ws.rec[b] = r;
        }
    }
    // early-exit calls sum the drawn rows in the last window, for every
    // request that draws, whichever window it ended in
    if (!draw || (EE && !P.ee_last)) return;
    // this wave's unit of the drawn row pair (SPLIT: its part of one)
    if (!SPLIT && c * NWAVE + wave_id() >= P.cs) return;
    __builtin_amdgcn_s_setprio(0);
    const DrawRows<BF16> dr =
        draw_rows<BF16>(P, q.rb.tb, q.rb.db, desc, resid ? sz_row.m : 0.0f, resid ? sy_row.m : 0.0f);
    unit_sums_store<BF16, ALIGNED, SPLIT>(P, b, c, dr, resid, rho_hat, tab, sh_parts);
}

// ---------------------------------------------------------------------------
// Draw kernel: one workgroup per request that draws a token.
//
// After a rejection at n:  r = max(0, p_n - q_n), or p_n if that has no mass;
// without one: r = p_d (target row d).  In units of P and Q (terms relative to
// the row maxima), r = max(0, P - rho Q)/Sz with rho = Sz/Sy, which needs the
// row sums before any term; the chunk pass therefore split the terms with an
// estimate rho_hat of rho (from the row pass): D = sum over {P > rho_hat Q} of
// (P - rho_hat Q) and Bq = sum of Q over the same set, so that
// R_c = D + (rho_hat - rho) Bq is chunk c's residual mass.  The two sets
// differ only on terms where P and rho Q agree to within the estimate's
// relative error (about 1e-7), whose residual mass is negligible.  The draw
// compares u*R with prefix sums in token order: the first token whose
// inclusive prefix exceeds u*R, or the last token with mass if rounding
// leaves none.
// ---------------------------------------------------------------------------

// Terms of the chosen distribution at the elements of vector vi (rescan):
//   which 0: residual max(0, P - rho Q);  which 1: P.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void slot_terms(const DrawRows<BF16> &dr, int which, double rho, int vi, const uint4 &rz,
                                           const uint4 &ry, const double *tab, double (&val)[RowView<BF16>::EPV])
{
    constexpr int EPV = RowView<BF16>::EPV;
    int flag = 0;
    float f[EPV], g[EPV];
    chunk_vec<BF16, ALIGNED>(dr.rz, vi, rz, f, flag);
    if (which == 0) draft_vec<BF16, ALIGNED>(dr.dc, dr.rz, vi, ry, g);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        const double p = exp2_512(dr.exact ? draw_exp_arg<true>(f[e], dr.mz, dr.mzc5, dr.cd5)
                                           : draw_exp_arg<false>(f[e], dr.mz, dr.mzc5, dr.cd5), tab);
        if (which == 0) {
            const double q = exp2_512(dr.exact ? draw_exp_arg<true>(g[e], dr.my, dr.myc5, dr.cd5)
                                               : draw_exp_arg<false>(g[e], dr.my, dr.myc5, dr.cd5), tab);
            const double t = fma(-rho, q, p);
            val[e] = t > 0.0 ? t : 0.0;
        } else {
            val[e] = p;
        }
    }
}

// A wave's own copy of the exp2 table: LDS operations of one wave complete in
// program order, so the wave can read it right after writing it, with no
// workgroup barrier.
__device__ __forceinline__ void init_exp2_table_wave(double *tab)
{
    fill_exp2_table(tab);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane `src` (wave-uniform) of v.
__device__ __forceinline__ double readlane_d(double v, int src)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Unit totals of the chosen distribution (wave-redundant: every wave of the
// draw workgroup computes the same values from the same inputs).
struct UnitPick {
    int cstar;      // unit holding the draw, -1 if none
    bool over;      // u*R reached no unit's inclusive prefix (rounding)
    bool bad;       // the row pair cannot be drawn from
    double base;    // exclusive prefix of unit cstar
    double target;  // u*R
    double rho;     // Sz/Sy (residual draw)
    int which;      // 0: residual max(0, P - rho Q); 1: P
    float Mb;       // bonus draw: the row maximum
};

// Every wave of the draw workgroup, redundantly and with wave operations
// only: the unit totals of the chosen distribution in unit order (lane-
// strided, unit j = 64 h + lane), their total R, and the first unit whose
// inclusive prefix exceeds u*R (else the last unit with mass).  c0: the
// lane's unit of the first 64 (j = lane), loaded by the caller ahead of
// time; u: the draw uniform.
template <bool BF16>
__device__ UnitPick pick_unit(const Params &P, int b, const DrawRec &rec, const DrawRows<BF16> &dr, const double *tab,
                              const ChunkPart &c0, float u)
{
    const int lane = lane_id();
    const ChunkPart *cp = P.ws.cp + (int64_t)b * P.cs;
    const int ncs = P.cs;
    const int H = (int)ceil_div(ncs, 64);
    const bool resid = rec.state == SREQ_RESID;
    UnitPick k;
    k.rho = 0.0;
    k.which = 1;
    k.Mb = 0.0f;
    k.bad = false;
    // pass 1: the row sums (residual) or the row maximum (bonus)
    double lz = 0.0, ly = 0.0;
    float lm = -INFINITY;
    int lb = 0;
    for (int h = 0; h < H; ++h) {
        const int j = h * 64 + lane;
        if (j < ncs) {
            const ChunkPart c = h == 0 ? c0 : cp[j];
            lz += c.sz;
            ly += c.sy;
            lm = fmaxf(lm, c.m);
            lb |= c.bad;
        }
    }
    if (resid) {
        const double Sz = wave_sum(lz), Sy = wave_sum(ly);
        k.bad = !(Sz > 0.0) || !(Sy > 0.0);
        k.rho = k.bad ? 0.0 : Sz / Sy;
        // residual mass: draw from p if there is none
        double lr = 0.0;
        for (int h = 0; h < H; ++h) {
            const int j = h * 64 + lane;
            if (j < ncs) {
                const ChunkPart c = h == 0 ? c0 : cp[j];
                lr += fmax(0.0, fma(rec.rho_hat - k.rho, c.bq, c.d));
            }
        }
        k.which = wave_sum(lr) > 0.0 ? 0 : 1;
    } else {
        k.Mb = wave_max(lm);
        k.bad = wave_or(lb) != 0 || k.Mb == -INFINITY || k.Mb == INFINITY;
    }
    // pass 2: unit totals, prefix scan in unit order, the unit holding u*R
    double carry = 0.0;
    k.target = 0.0;
    int cand = -1, lastc = -1;
    double cbase = 0.0;
    double Rt = 0.0;
    // R first (the target depends on it), then the search
    for (int pass = 0; pass < 2; ++pass) {
        carry = 0.0;
        for (int h = 0; h < H; ++h) {
            const int j = h * 64 + lane;
            double t = 0.0;
            if (j < ncs) {
                const ChunkPart c = h == 0 ? c0 : cp[j];
                if (resid) t = k.which == 0 ? fmax(0.0, fma(rec.rho_hat - k.rho, c.bq, c.d)) : c.sz;
                else t = (c.m == -INFINITY || k.bad) ? 0.0 : c.sz * exp2_tab(((double)c.m - (double)k.Mb) * dr.cd, tab);
            }
            const double raw = wave_incl_scan(t);
            const double incl = raw + carry;
            if (pass == 1) {
                // lane l's exclusive prefix is lane l-1's inclusive one, bit for bit
                const double excl = wave_shr1(raw) + carry;
                const uint64_t hit = __ballot(j < ncs && incl > k.target);
                if (cand < 0 && hit != 0) {
                    const int l = __builtin_ctzll(hit);
                    cand = h * 64 + l;
                    cbase = readlane_d(excl, l);
                }
                const uint64_t mass = __ballot(t > 0.0);
                if (mass != 0) lastc = h * 64 + 63 - __builtin_clzll(mass);
            }
            carry = readlane_d(incl, 63);
        }
        if (pass == 0) {
            Rt = carry;
            if (!(Rt > 0.0)) k.bad = true;
            k.target = (double)u * Rt;
        }
    }
    k.over = cand < 0;
    k.cstar = k.over ? lastc : cand;
    k.base = k.over ? 0.0 : cbase;
    return k;
}

template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(WG) void draw_kernel(Params P)
{
    constexpr int EPV = RowView<BF16>::EPV, UV = unit_v<BF16>(), VPW = UV / NWAVE, ROUNDS = VPW / 64;
    static_assert(VPW % 64 == 0, "a wave rescans whole rounds of 64 vectors");
    __shared__ double tabs[NWAVE][EXP2_TAB];
    __shared__ double sh_tot[NWAVE];
    __shared__ int sh_last[NWAVE];
    __shared__ int sh_first[NWAVE];
    const int b = blockIdx.x, w = wave_id(), lane = lane_id();
    // the first 64 unit sums and the draw uniform are loaded with the record,
    // so the three latencies overlap instead of following one another
    // (clamped index, no branch: lanes past the units are never used).  The
    // compiler-only barrier keeps the first two above the record's test (the
    // compiler would otherwise sink them below it, into a second round trip);
    // the exp2 table is built while all three are in flight.
    const ChunkPart c0 = P.ws.cp[(int64_t)b * P.cs + min(lane, P.cs - 1)];
    const float u0 = P.u_sample[b];
    const DrawRec rec = P.ws.rec[b];
    __asm__ volatile("" ::: "memory");
    double *tab = tabs[w];
    init_exp2_table_wave(tab);
    if (rec.state != SREQ_RESID && rec.state != SREQ_BONUS) return;
    const bool resid = rec.state == SREQ_RESID;
    const ReqDesc desc = {rec.state, rec.n, -1, rec.T};
    DrawRows<BF16> dr = draw_rows<BF16>(P, rec.tb, rec.db, desc, rec.mz, rec.my);
    const UnitPick k = pick_unit<BF16>(P, b, rec, dr, tab, c0, u0);
    if (k.bad || k.cstar < 0) {   // the drawn row holds NaN, +inf or nothing but -inf
        if (w == 0) {
            const ReqDesc bd = {SREQ_BAD, 0, -1, rec.T};
            write_outputs(P, b, 0, {rec.tb, rec.db, rec.nout}, bd, nullptr, -1);
        }
        return;
    }
    if (!resid) {
        // the bonus rescan offsets by the row maximum, in the exact form (as
        // the unit sums it is compared with)
        dr.mz = (double)k.Mb;
        dr.mzc = dr.mz * dr.cd;
        dr.exact = true;
        dr.scale();
    }
    const int wsel = resid ? k.which : 1;

    // rescan of unit cstar in token order: wave w takes its quarter, round
    // r of it being vectors 64 r + lane
    const int v0 = k.cstar * UV + w * VPW + lane;
    uint4 rz[ROUNDS], ry[ROUNDS];
    issue_vecs<BF16, ROUNDS>(dr.rz, v0, 64, rz);
    // the draft row exists only for a residual draw (a bonus draw reads
    // target row d; draft row d may lie past the draft logits)
    if (wsel == 0 && ALIGNED) issue_vecs<BF16, ROUNDS>(dr.dc.ry, v0, 64, ry);
    double val[ROUNDS][EPV], excl[ROUNDS];
    double wtot = 0.0;
    int lastp = -1;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        slot_terms<BF16, ALIGNED>(dr, wsel, k.rho, v0 + 64 * r, rz[r], ry[r], tab, val[r]);
        double vs = 0.0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            vs += val[r][e];
            const int x = dr.rz.elem(v0 + 64 * r, e);
            if (val[r][e] > 0.0 && x >= 0 && x < P.V) lastp = max(lastp, x);
        }
        const double incl = wave_incl_scan(vs);
        excl[r] = wave_shr1(incl) + wtot;
        wtot += readlane_d(incl, 63);
    }
    if (lane == 0) {
        sh_tot[w] = wtot;
    }
    {
        // highest token with mass in this wave
        int m = lastp;
        m = max(m, xchg_i<0>(m));
        m = max(m, xchg_i<1>(m));
        m = max(m, xchg_i<2>(m));
        m = max(m, xchg_i<3>(m));
        m = max(m, xchg_i<4>(m));
        m = max(m, xchg_i<5>(m));
        if (lane == 0) sh_last[w] = m;
    }
    __syncthreads();
    double wbase = 0.0;
    for (int u = 0; u < w; ++u) wbase += sh_tot[u];
    int first = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const double slot0 = wbase + excl[r];
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            part += val[r][e];
            const int x = dr.rz.elem(v0 + 64 * r, e);
            if (first == 0x7fffffff && val[r][e] > 0.0 && x >= 0 && x < P.V && k.base + (slot0 + part) > k.target)
                first = x;
        }
    }
    {
        // lowest crossing token in this wave
        int m = first;
        m = min(m, xchg_i<0>(m));
        m = min(m, xchg_i<1>(m));
        m = min(m, xchg_i<2>(m));
        m = min(m, xchg_i<3>(m));
        m = min(m, xchg_i<4>(m));
        m = min(m, xchg_i<5>(m));
        if (lane == 0) sh_first[w] = m;
    }
    __syncthreads();
    if (w != 0) return;
    int fi = 0x7fffffff, lp = -1;
#pragma unroll
    for (int u = 0; u < NWAVE; ++u) {
        fi = min(fi, sh_first[u]);
        lp = max(lp, sh_last[u]);
    }
    const int tok = (!k.over && fi != 0x7fffffff) ? fi : lp;
    if (tok >= 0) {
        if (lane == 0) P.out_tokens[(int64_t)rec.tb + rec.n] = tok;
    } else {
        const ReqDesc bd = {SREQ_BAD, 0, -1, rec.T};
        write_outputs(P, b, 0, {rec.tb, rec.db, rec.nout}, bd, nullptr, -1);
    }
}

// Confidence as the D-cut rules read it: 0 for NaN or c <= 0, 1 above 1.
__device__ __forceinline__ float sanitize_conf(float c)
{
    if (!(c > 0.0f)) return 0.0f;
    return c > 1.0f ? 1.0f : c;
}

// ---------------------------------------------------------------------------
// Read ceiling (benchmark instrumentation): a plain stream over a buffer with
// the row pass's load width and cache policy, every byte read once, against
// which the row pass's bandwidth is compared.  A workgroup reads 16 KiB
// blocks, handed out grid-stride; each wave reads its 4 KiB quarter of a
// block (UW 16-byte loads per lane, each load instruction 1 KiB).  Of the
// shapes measured on MI355X (4 to 16 KiB per wave, per-wave or
// per-workgroup blocks, 4 to 16 workgroups per CU, streaming or plain
// loads) this one, at 16 workgroups per CU, was the fastest; the others
// were within 2 % except plain loads (about 10 % slower).  Lanes fold what
// they read so the loads stay live; the fold reaches memory only in the
// unlikely case that it equals a fixed value.
// ---------------------------------------------------------------------------

constexpr int CEIL_WGS_PER_CU = 16;

__global__ __launch_bounds__(WG) void read_ceiling_kernel(const uint4 *buf_, int64_t nvec, uint32_t *sink)
{
    const gvec_t buf = (gvec_t)buf_;
    const int64_t G = gridDim.x;
    const int w = wave_id(), lane = lane_id();
    const int64_t nblk = nvec / (NWAVE * WVEC);
    uint32_t acc = 0;
    for (int64_t blk = blockIdx.x; blk < nblk; blk += G) {
        uint4 r[UW];
#pragma unroll
        for (int j = 0; j < UW; ++j) r[j] = ld_stream(buf + blk * (NWAVE * WVEC) + (w * UW + j) * 64 + lane);
#pragma unroll
        for (int j = 0; j < UW; ++j) acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
    }
    // the vectors after the last whole block
    for (int64_t v = nblk * (NWAVE * WVEC) + (int64_t)blockIdx.x * WG + threadIdx.x; v < nvec; v += G * WG) {
        const uint4 r = ld_stream(buf + v);
        acc ^= r.x ^ r.y ^ r.z ^ r.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// ---------------------------------------------------------------------------
// Cost-aware D-cut: one workgroup of 1024 threads.
//  1. the latency table and (small inputs) the confidences into LDS, all
//     loads in flight together; cost(d) for every depth: the table read as
//     linear between neighbouring points, constant outside them.
//  2. the bids.  Small inputs (B * K up to 4096 pairs): one thread per
//     request forms its prefix products in order (double) into LDS, then one
//     thread per (request, depth) pair forms the value (P * d) / cost(d), then
//     one thread per request takes the first largest value.  Larger inputs:
//     one thread per request does all three in order, its confidence loads
//     sixteen at a time.  Either way each P is the sequential product.
//  3. the bids are ordered by (value desc, request asc): rank by counting
//     for up to 256 requests, a bitonic sort in LDS above that; requests
//     without a bid go last.
//  4. wave 0 offers the budget in that order.  Lane l holds the cost of bid
//     64 h + l, and the running total advances one bid at a time on
//     wave-uniform values with selects (no branch per bid), so it rounds as
//     the sequential sum does; a bid that does not fit is passed over.
// Arithmetic in double without contraction, in the order written.
// ---------------------------------------------------------------------------

constexpr int COST_TAB_MAX = 32;
constexpr int COST_WG = 1024;
constexpr int COST_B_MAX = 4096;
constexpr int COST_RANK_MAX = 256;   // up to this many requests, ranks by counting
constexpr int COST_PAIRS = 4096;     // up to this many (request, depth) pairs, values in parallel

struct CostTable {
    double t[COST_TAB_MAX];   // depths, strictly increasing
    double c[COST_TAB_MAX];   // costs, finite and > 0
    int n;
};

// cost(d) from the table held in LDS (depths td, costs tc, n points).
__device__ double table_cost(const double *td, const double *tc, int n, double d)
{
#pragma clang fp contract(off)
    int above = 0;   // table points at or below d
    while (above < n && td[above] <= d) ++above;
    if (above == 0) return tc[0];
    if (above == n) return tc[n - 1];
    const double w = (d - td[above - 1]) / (td[above] - td[above - 1]);
    return tc[above - 1] + w * (tc[above] - tc[above - 1]);
}

// Sort key of a bid: the value's bits (values are >= 0, so their bits order
// like them) plus 1; 0 for a request without a bid.
__device__ __forceinline__ uint64_t bid_key(double v) { return (uint64_t)__double_as_longlong(v) + 1ull; }

// Confidences up to this many are staged through LDS with one coalesced load
// per element; larger inputs are read in place.
constexpr int COST_STAGE = 8192;

// Does (a, wa) come before (c, wc): key descending, request ascending?
__device__ __forceinline__ bool bid_first(uint64_t a, int wa, uint64_t c, int wc)
{
    return a > c || (a == c && wa < wc);
}

__device__ __forceinline__ double wave_max_d(double v)
{
    v = fmax(v, xchg_d<0>(v));
    v = fmax(v, xchg_d<1>(v));
    v = fmax(v, xchg_d<2>(v));
    v = fmax(v, xchg_d<3>(v));
    v = fmax(v, xchg_d<4>(v));
    return fmax(v, xchg_d<5>(v));
}

// The window of request b (K_b, or -1 when it is outside [0, K]).
__device__ __forceinline__ int cost_window(const int32_t *max_depth, int b, int K)
{
    const int Kb = max_depth ? max_depth[b] : K;
    return (Kb >= 0 && Kb <= K) ? Kb : -1;
}

// flags: bit 0 the confidences are staged in LDS, bit 1 the bids use the
// pair-parallel values (needs bit 0)
__global__ __launch_bounds__(COST_WG) void dcut_cost_kernel(const float *conf, const int32_t *max_depth, int B,
                                                            int K, CostTable T, double max_verify, int flags,
                                                            int32_t *depth_out)
{
#pragma clang fp contract(off)
    extern __shared__ double cost_smem[];
    const bool staged = flags & 1, paired = flags & 2;
    int N = 1;
    while (N < B) N <<= 1;
    double *costd = cost_smem;                          // [K + 1]
    uint64_t *key = (uint64_t *)(costd + (K + 1));      // [N] sort keys (by request, then by rank)
    uint16_t *who = (uint16_t *)(key + N);              // [N] request of each sorted key
    uint16_t *bid = who + N;                            // [B] bid depth (0: none)
    double *pv = cost_smem + (K + 1) + N + (N + B + 3) / 4;   // [B * K] products, then values (paired)
    float *cst = (float *)(pv + (paired ? B * K : 0));        // [B * K] confidences (staged)
    __shared__ int8_t state[COST_B_MAX];                // -1 bad K_b, 0 no grant, 1 granted
    __shared__ double tab_t[COST_TAB_MAX], tab_c[COST_TAB_MAX];
    __shared__ double sh_min;
    const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();

    if (tid < T.n) {
        tab_t[tid] = T.t[tid];
        tab_c[tid] = T.c[tid];
    }
    if (staged)
        for (int i = tid; i < B * K; i += COST_WG) cst[i] = conf[i];
    __syncthreads();
    for (int d = tid; d <= K; d += COST_WG) costd[d] = d == 0 ? 0.0 : table_cost(tab_t, tab_c, T.n, (double)d);
    __syncthreads();
    if (wv == 0) {
        // the cheapest depth's cost: once it cannot fit, nothing can
        double m = INFINITY;
        for (int d = 1 + lane; d <= K; d += 64) m = fmin(m, costd[d]);
        m = -wave_max_d(-m);
        if (lane == 0) sh_min = m;
    }

    // 2. bids
    if (paired) {
        for (int b = tid; b < B; b += COST_WG) {
            const int dn = max(cost_window(max_depth, b, K), 0);
            double P = 1.0;
            for (int d = 1; d <= dn; ++d) {
                P = P * (double)sanitize_conf(cst[b * K + d - 1]);
                pv[b * K + d - 1] = P;
            }
        }
        __syncthreads();
        for (int i = tid; i < B * K; i += COST_WG) {
            const int d = i % K + 1;   // entries past a request's window are never read
            pv[i] = (pv[i] * (double)d) / costd[d];
        }
        __syncthreads();
    }
    for (int b = tid; b < N; b += COST_WG) {
        uint64_t kb = 0;
        if (b < B) {
            const int Kb = cost_window(max_depth, b, K);
            const int dn = max(Kb, 0);
            double best = 0.0;
            int dbest = 0;
            if (paired) {
                for (int d = 1; d <= dn; ++d) {
                    const double v = pv[b * K + d - 1];
                    if (d == 1 || v > best) { best = v; dbest = d; }
                }
            } else {
                double P = 1.0;
                const float *cb = conf + (int64_t)b * K;
                for (int d0 = 0; d0 < dn; d0 += 16) {
                    float c16[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int dd = min(d0 + i, dn - 1);
                        c16[i] = staged ? cst[(int64_t)b * K + dd] : cb[dd];   // all sixteen in flight
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int d = d0 + i + 1;
                        if (d <= dn) {
                            P = P * (double)sanitize_conf(c16[i]);
                            const double v = (P * (double)d) / costd[d];
                            if (d == 1 || v > best) { best = v; dbest = d; }
                        }
                    }
                }
            }
            state[b] = Kb < 0 ? -1 : 0;
            bid[b] = (uint16_t)dbest;
            if (dbest > 0) kb = bid_key(best);
        }
        key[b] = kb;
    }
    __syncthreads();

    // 3. order of the bids
    if (N <= COST_RANK_MAX) {
        // rank of request t = the bids that come before it
        uint64_t kt = 0;
        int rank = 0;
        if (tid < N) {
            kt = key[tid];
#pragma unroll 8
            for (int o = 0; o < N; ++o) rank += bid_first(key[o], o, kt, tid) ? 1 : 0;
        }
        __syncthreads();
        if (tid < N) {   // the ranks are a permutation of 0 .. N-1
            key[rank] = kt;
            who[rank] = (uint16_t)min(tid, B - 1);
        }
    } else {
        for (int t = tid; t < N; t += COST_WG) who[t] = (uint16_t)min(t, B - 1);
        __syncthreads();
        for (int size = 2; size <= N; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = tid; t < N / 2; t += COST_WG) {
                    const int lo = 2 * t - (t & (stride - 1));
                    const int hi = lo + stride;
                    const bool desc = (lo & size) == 0;
                    const uint64_t a = key[lo], c = key[hi];
                    const int wa = who[lo], wc = who[hi];
                    if (bid_first(a, wa, c, wc) != desc) {
                        key[lo] = c;
                        key[hi] = a;
                        who[lo] = (uint16_t)wc;
                        who[hi] = (uint16_t)wa;
                    }
                }
                __syncthreads();
            }
        }
    }
    __syncthreads();

    // 4. the budget, in bid order
    if (wv == 0) {
        const double minc = sh_min;
        double spent = 0.0;
        for (int h0 = 0; h0 < B; h0 += 64) {
            const int r = h0 + lane;
            const bool has = r < B && key[r] != 0;
            const int req = has ? who[r] : 0;
            const double c = has ? costd[bid[req]] : INFINITY;   // no bid: never fits
            const uint64_t bids = __ballot(has);   // a prefix of the lanes: bids sort first
            // the chunk's 64 offers, unrolled: the running total is the only
            // dependence from one offer to the next; a lane without a bid
            // costs +inf and never fits
            uint64_t granted = 0;
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                const double s2 = spent + readlane_d(c, i);
                const bool fit = s2 <= max_verify;
                spent = fit ? s2 : spent;
                granted |= (__ballot(fit) != 0 ? 1ull : 0ull) << i;
            }
            if ((granted >> lane) & 1ull) state[req] = 1;
            if (bids != ~0ull || !(spent + minc <= max_verify)) break;   // no bid left, or none can fit
        }
    }
    __syncthreads();
    for (int b = tid; b < B; b += COST_WG) depth_out[b] = state[b] < 0 ? -1 : (state[b] ? (int32_t)bid[b] : 0);
}

// ---------------------------------------------------------------------------
// Acceptance statistics: one workgroup.  Per valid request with n accepted
// drafts and window d, position k < d was tested iff n >= k and accepted iff
// n > k; with n <= d that makes accepted[k] = #{n > k} and reached[k] =
// accepted[k] + #{n == k < d} (the requests rejected at k).  So each request
// adds to two LDS histograms, and suffix sums give the counters.
// ---------------------------------------------------------------------------

constexpr int STATS_WG = 256;

__global__ __launch_bounds__(STATS_WG) void accept_stats_kernel(const int32_t *num_accepted, const int32_t *depth,
                                                                int B, int K, unsigned long long *counters)
{
    extern __shared__ unsigned int hist[];   // [K + 1] #{n}, then [K] #{rejected at k}
    __shared__ unsigned long long tot[4];    // requests, bad, sum n, sum n + 1
    unsigned int *hn = hist, *hr = hist + K + 1;
    const int tid = threadIdx.x;
    for (int i = tid; i < 2 * K + 1; i += STATS_WG) hist[i] = 0u;
    if (tid < 4) tot[tid] = 0ull;
    __syncthreads();
    unsigned long long sn = 0;
    int req = 0, bad = 0;
    for (int b = tid; b < B; b += STATS_WG) {
        const int n = num_accepted[b];
        if (n < 0) { ++bad; continue; }
        // positions outside the window [0, min(d, K)) are not counted
        const int d = min(max(depth ? depth[b] : K, 0), K);
        const int nw = min(n, d);
        ++req;
        sn += (unsigned long long)n;
        atomicAdd(&hn[nw], 1u);
        if (nw < d) atomicAdd(&hr[nw], 1u);
    }
    // one LDS add per wave for the request totals (sum n < 2^31: B <= 4096, n < 2^30)
    req = wave_sum_i(req);
    bad = wave_sum_i(bad);
    const int snw = wave_sum_i((int)sn);
    if (lane_id() == 0) {
        atomicAdd(&tot[0], (unsigned long long)req);
        atomicAdd(&tot[1], (unsigned long long)bad);
        atomicAdd(&tot[2], (unsigned long long)snw);
    }
    __syncthreads();
    // suffix sums over n: accepted[k] = #{n > k} = sum of bins k+1 .. K, stored
    // one bin up.  Wave 0: lane l sums a block of bins, a scan over the lanes
    // gives each block the count above it, then each lane walks its block
    // from the top.
    if (tid < 64) {
        const int per = (K + 63) / 64;
        const int lo = 1 + tid * per, hi = min(K, lo + per - 1);   // bins lo .. hi
        unsigned int blk = 0;
        for (int j = lo; j <= hi; ++j) blk += hn[j];
        const int incl = wave_incl_scan_i((int)blk);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        unsigned int above = (unsigned int)(total - incl);   // bins past this block
        for (int j = hi; j >= lo; --j) {
            above += hn[j];
            hn[j] = above;
        }
    }
    __syncthreads();
    for (int k = tid; k < K; k += STATS_WG) {
        const unsigned int acc = hn[k + 1];
        if (acc + hr[k]) atomicAdd(&counters[k], (unsigned long long)(acc + hr[k]));
        if (acc) atomicAdd(&counters[K + k], (unsigned long long)acc);
    }
    if (tid == 0) {
        atomicAdd(&counters[2 * K], tot[0]);
        atomicAdd(&counters[2 * K + 1], tot[1]);
        atomicAdd(&counters[2 * K + 2], tot[2]);
        atomicAdd(&counters[2 * K + 3], tot[2] + tot[0]);
    }
}

// ---------------------------------------------------------------------------
// D-cut allocation: one workgroup of 1024 threads; keys in LDS.
// ---------------------------------------------------------------------------

__device__ int block_sum_int(int v, int *sm32)
{
    v = wave_sum_i(v);
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
    const int incl = wave_incl_scan_i(v);
    __syncthreads();
    if (lane == 63) sm32[wave_id()] = incl;
    __syncthreads();
    int wb = 0;
    for (int w = 0; w < wave_id(); ++w) wb += sm32[w];
    __syncthreads();
    return wb + incl - v;
}

// keys[b*K + k]: 0 = not a candidate (k = 0, k >= K_b, invalid K_b), else the
// float bits of the running product c_{b,k} plus 1 (the products lie in
// [0, 1], so their bits order like their values).
__global__ __launch_bounds__(DCUT_WG) void dcut_kernel(const float *conf, const int32_t *max_depth, int B, int K,
                                                      int budget, int32_t *depth_out)
{
    extern __shared__ uint32_t keys[];   // [B*K]
    __shared__ int hist[256];
    __shared__ int sm32[DCUT_WG / 64];
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_kr;
    const int n = B * K;
    const int tid = threadIdx.x;
    for (int i = tid; i < n; i += DCUT_WG) keys[i] = __float_as_uint(conf[i]);
    __syncthreads();
    int floors = 0, cands = 0;
    for (int b = tid; b < B; b += DCUT_WG) {
        const int Kb = max_depth ? max_depth[b] : K;
        const bool valid = Kb >= 0 && Kb <= K;
        float c = 0.0f;
        for (int k = 0; k < K; ++k) {
            uint32_t key = 0;
            if (valid && k < Kb) {
                const float s = sanitize_conf(__uint_as_float(keys[b * K + k]));
                c = (k == 0) ? s : c * s;
                if (k >= 1) key = __float_as_uint(c) + 1u;
            }
            keys[b * K + k] = key;
        }
        if (valid) {
            floors += Kb > 0 ? 1 : 0;
            cands += Kb > 1 ? Kb - 1 : 0;
        }
    }
    __syncthreads();
    floors = block_sum_int(floors, sm32);
    cands = block_sum_int(cands, sm32);
    int take = budget - floors;
    if (take > cands) take = cands;
    if (take < 0) take = 0;

    // each thread owns the contiguous flat range [lo, hi)
    const int per = (int)ceil_div(n, DCUT_WG);
    const int lo = std::min(n, tid * per), hi = std::min(n, lo + per);

    // radix select of the take-th largest key, 8 bits at a time
    uint32_t prefix = 0;
    int kr = take;
    if (take > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += DCUT_WG) hist[i] = 0;
            __syncthreads();
            const uint32_t hmask = (shift == 24) ? 0u : (0xffffffffu << (shift + 8));
            for (int i = lo; i < hi; ++i) {
                const uint32_t key = keys[i];
                if (key != 0 && (key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 255u], 1);
            }
            __syncthreads();
            if (tid < 64) {
                // the digit: the highest bin whose count, with every bin above
                // it, reaches kr.  Lane l holds bins 255 - 4l down to 252 - 4l;
                // a scan over the lanes gives the counts above each lane.
                int h[4], sum = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h[j] = hist[255 - 4 * tid - j];
                    sum += h[j];
                }
                const int incl = wave_incl_scan_i(sum);
                const uint64_t hit = __ballot(incl >= kr);   // nonempty: kr <= the keys left
                if (tid == __builtin_ctzll(hit)) {
                    int acc = incl - sum, digit = 255 - 4 * tid - 3;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (acc + h[j] >= kr) {
                            digit = 255 - 4 * tid - j;
                            break;
                        }
                        acc += h[j];
                    }
                    sh_kr = kr - acc;
                    sh_prefix = prefix | ((uint32_t)digit << shift);
                }
            }
            __syncthreads();
            prefix = sh_prefix;
            kr = sh_kr;
            __syncthreads();
        }
    }
    // Entries above the threshold are taken; ties at the threshold go in
    // flat-index order.  Taken entries are marked 1 in place.
    const uint32_t thr = prefix;
    int eq = 0;
    if (take > 0)
        for (int i = lo; i < hi; ++i) eq += (keys[i] == thr);
    int rank = block_excl_scan_int(eq, sm32);
    for (int i = lo; i < hi; ++i) {
        const uint32_t key = keys[i];
        int taken = 0;
        if (take > 0 && key != 0) {
            if (key > thr) taken = 1;
            else if (key == thr) taken = (rank++ < kr);
        }
        keys[i] = (uint32_t)taken;
    }
    __syncthreads();
    for (int b = tid; b < B; b += DCUT_WG) {
        const int Kb = max_depth ? max_depth[b] : K;
        const bool valid = Kb >= 0 && Kb <= K;
        int dep = valid ? (Kb > 0 ? 1 : 0) : -1;
        if (valid)
            for (int k = 0; k < K; ++k) dep += (int)keys[b * K + k];
        depth_out[b] = dep;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

thread_local char g_last_error[256] = "";

sv_status hip_status(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        g_last_error[0] = 0;
        return SV_OK;
    }
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
    return SV_ERR_HIP;
}

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

// Check mode (environment variable SPECVERIFY_CHECK=1; a debugging aid, not
// for graph capture): a call that enqueued its work waits for it and returns
// SV_ERR_BAD_INPUT when a request reported bad data (a negative value in
// vals[0..n): num_accepted of a verify call, depth_out of dcut_allocate).
sv_status checked(sv_status st, const int32_t *vals, int32_t n, hipStream_t stream, const char *what)
{
    const char *e = getenv("SPECVERIFY_CHECK");
    if (st != SV_OK || !e || e[0] != '1') return st;
    std::vector<int32_t> h((size_t)n);
    if (hipMemcpyAsync(h.data(), vals, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return hip_status(what);
    for (int32_t i = 0; i < n; ++i)
        if (h[(size_t)i] < 0) {
            snprintf(g_last_error, sizeof g_last_error, "%s: request %d holds bad data", what, (int)i);
            return SV_ERR_BAD_INPUT;
        }
    return SV_OK;
}

// Resident workgroups of the persistent row pass per compute unit (from the
// occupancy calculator; the grid never exceeds what can run at once, so the
// static task assignment stays balanced).
int row_wgs_per_cu(bool bf16, bool ee, bool dual, size_t lds)
{
    static std::atomic<int> cache[2][3][64];
    const int bucket = (int)std::min<size_t>(63, lds / 1024);
    const int v = dual ? 2 : ee ? 1 : 0;
    int n = cache[bf16][v][bucket].load(std::memory_order_relaxed);
    if (n <= 0) {
        const void *fn = bf16 ? (dual ? (const void *)row_pass_kernel<true, false, true>
                                      : ee ? (const void *)row_pass_kernel<true, true, false>
                                           : (const void *)row_pass_kernel<true, false, false>)
                              : (dual ? (const void *)row_pass_kernel<false, false, true>
                                      : ee ? (const void *)row_pass_kernel<false, true, false>
                                           : (const void *)row_pass_kernel<false, false, false>);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, WG, (bucket + 1) * 1024) != hipSuccess || n <= 0)
            n = 2;
        cache[bf16][v][bucket].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The D-cut keys live in dynamic LDS (up to 128 KiB; gfx950 gives a
// workgroup up to 160 KiB).  Checked against the device's limit, with the
// kernel's dynamic-LDS ceiling raised once per device.
bool dcut_lds_ok(size_t dyn)
{
    static std::atomic<int> limit[MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return false;
    int lim = limit[dev].load(std::memory_order_relaxed);
    if (lim <= 0) {
        if (hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lim <= 0)
            lim = 65536;
        lim -= 4096;   // the kernel's static LDS, with room to spare
        if (hipFuncSetAttribute((const void *)dcut_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lim) !=
            hipSuccess) {
            (void)hipGetLastError();
            lim = 65536 - 4096;
        }
        limit[dev].store(lim, std::memory_order_relaxed);
    }
    if (dyn > (size_t)lim) {
        snprintf(g_last_error, sizeof g_last_error, "dcut_allocate: %zu bytes of keys exceed this device's LDS", dyn);
        return false;
    }
    return true;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

sv_status check_shape(int32_t B, int32_t K, int32_t V)
{
    if (B < 1 || K < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (B > B_MAX || K > K_MAX || V > V_MAX) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

// Packed layout: the number of drafted positions the packed arrays hold
// (row and slot indices stay below 2^31 with B <= B_MAX added).
constexpr int32_t PACKED_ROWS_MAX = 1 << 30;

sv_status check_packed(int32_t n_rows)
{
    if (n_rows < 0) return SV_ERR_INVALID_ARG;
    if (n_rows > PACKED_ROWS_MAX) return SV_ERR_UNSUPPORTED;
    return SV_OK;
}

sv_status check_ws(void *ws, size_t ws_bytes, const Layout &L)
{
    if (!ws || ws_bytes < L.total || ((uintptr_t)ws & 255u) != 0) return SV_ERR_WORKSPACE;
    return SV_OK;
}

// Stage timing of the calling thread's calls (benchmark instrumentation):
// four events per armed call, recorded on the call's stream around its
// kernels.
struct StageTiming {
    std::vector<hipEvent_t> ev;
    int armed = 0, used = 0;
    ~StageTiming()
    {
        for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    }
};
thread_local StageTiming g_timing;

inline hipEvent_t stage_event(int call, int s) { return g_timing.ev[(size_t)4 * call + s]; }

// Row pass, then the finish kernel with grid.x = sampler units / 4 (1 when
// nothing is drawn), then for sampled calls the draw kernel.
sv_status launch(Params &P, hipStream_t stream)
{
    const int64_t nv = nvec_max(P.V, P.bf16 ? 8 : 4);
    const int kw = P.ee ? P.win_hi - P.win_lo : P.K;   // positions one launch can verify
    const int64_t rows_max = (P.mode == MODE_SAMPLE) ? (int64_t)P.B * (2 * kw + 1)
                           : (P.mode == MODE_GREEDY) ? (int64_t)P.B * (kw + 1) : (int64_t)P.B * P.K;
    const size_t lds_a = sizeof(int) * (size_t)(3 * P.B + 1);
    const bool dual = P.mode == MODE_CONF && P.conf_temp != nullptr;
    int64_t grid = (int64_t)cu_count() * row_wgs_per_cu(P.bf16, P.ee, dual, lds_a);
    grid = std::min<int64_t>(grid, std::max<int64_t>(1, ceil_div(rows_max * ceil_div(nv, WVEC), NWAVE)));
    const size_t lds_b = sizeof(Stat) * (size_t)(2 * P.K + 1) + sizeof(float2) * (size_t)P.K;
    const bool sample = P.mode == MODE_SAMPLE;
    const bool split = sample && P.usplit > 1;
    const dim3 grid_b((unsigned)(sample && (!P.ee || P.ee_last) ? ceil_div((int64_t)P.cs * P.usplit, NWAVE) : 1),
                      (unsigned)P.B);
    const int tcall = (!P.ee && g_timing.used < g_timing.armed) ? g_timing.used++ : -1;
    (void)hipGetLastError();
#define SV_MARK(s)                                                            \
    do {                                                                      \
        if (tcall >= 0) (void)hipEventRecord(stage_event(tcall, s), stream); \
    } while (0)
#define SV_LAUNCH_PATH(BF, AL)                                                                              \
    do {                                                                                                    \
        SV_MARK(0);                                                                                         \
        if (P.ee) {                                                                                         \
            hipLaunchKernelGGL((row_pass_kernel<BF, true, false>), dim3((unsigned)grid), dim3(WG), lds_a, stream, P); \
            if (split) hipLaunchKernelGGL((finish_kernel<BF, AL, true, true>), grid_b, dim3(WG), lds_b, stream, P); \
            else hipLaunchKernelGGL((finish_kernel<BF, AL, true, false>), grid_b, dim3(WG), lds_b, stream, P); \
        } else {                                                                                            \
            if (dual) hipLaunchKernelGGL((row_pass_kernel<BF, false, true>), dim3((unsigned)grid), dim3(WG), lds_a, stream, P); \
            else hipLaunchKernelGGL((row_pass_kernel<BF, false, false>), dim3((unsigned)grid), dim3(WG), lds_a, stream, P); \
            SV_MARK(1);                                                                                     \
            if (split) hipLaunchKernelGGL((finish_kernel<BF, AL, false, true>), grid_b, dim3(WG), lds_b, stream, P); \
            else hipLaunchKernelGGL((finish_kernel<BF, AL, false, false>), grid_b, dim3(WG), lds_b, stream, P); \
        }                                                                                                   \
        SV_MARK(2);                                                                                         \
        if (sample && (!P.ee || P.ee_last))                                                                 \
            hipLaunchKernelGGL((draw_kernel<BF, AL>), dim3((unsigned)P.B), dim3(WG), 0, stream, P);         \
        SV_MARK(3);                                                                                         \
    } while (0)
    if (P.bf16) {
        if (P.aligned) SV_LAUNCH_PATH(true, true);
        else SV_LAUNCH_PATH(true, false);
    } else {
        if (P.aligned) SV_LAUNCH_PATH(false, true);
        else SV_LAUNCH_PATH(false, false);
    }
#undef SV_LAUNCH_PATH
#undef SV_MARK
    return hip_status("kernel launch");
}

// Window ends of an early-exit call: strictly increasing, the first >= 1;
// the list is cut after the first end that reaches K (no request is left
// after it), and must contain one.  Ends are clipped to max(K, 1).
bool window_plan(const int32_t *ends, int32_t n, int32_t K, std::vector<int> &out)
{
    out.clear();
    if (!ends || n < 1) return false;
    int prev = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (ends[i] <= prev) return false;
        prev = ends[i];
        out.push_back(std::min(ends[i], std::max(K, 1)));
        if (ends[i] >= K) return true;
    }
    return false;
}

// Early-exit verification: per window a row pass and a finish kernel
// (merge, scan, outputs, draw record), back to back on the stream (the host
// never waits).  For sampled calls the last window's finish kernel also sums
// the drawn row pair of every request that draws, whichever window it ended
// in, and the draw kernel follows it.
// Window w verifies positions [ends[w-1], ends[w]) (ends[-1] = 0) of the
// requests that accepted every earlier position; the last window reaches K.
// The still-verifying flags alternate between two arrays so that a window
// never overwrites what its own kernels read.
sv_status launch_windows(Params &P, const std::vector<int> &ends, hipStream_t stream)
{
    const int nwin = (int)ends.size();
    P.ee = 1;
    for (int w = 0; w < nwin; ++w) {
        P.win_lo = w == 0 ? 0 : ends[(size_t)w - 1];
        P.win_hi = ends[(size_t)w];
        P.alive_in = P.ws.alive + (size_t)(w & 1) * (size_t)P.B;
        P.alive_out = P.ws.alive + (size_t)((w + 1) & 1) * (size_t)P.B;
        P.ee_last = w == nwin - 1;
        const sv_status st = launch(P, stream);
        if (st != SV_OK) return st;
    }
    return SV_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free sampled verification: a file-scope
// device array, one copy per GPU, held until the process ends.  In host
// code its name is only a stand-in: its device address is taken once per
// device with hipGetSymbolAddress (with that device current) and kept here,
// and only that address reaches kernels.  Every call on a GPU shares the
// array, so calls that overlap on one GPU race; the verify kernels write
// every part of their workspace before reading it, so nothing needs
// clearing between calls.
// ---------------------------------------------------------------------------

constexpr size_t STATIC_SCRATCH_BYTES = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES];

// The current device's address of the scratch array, or nullptr (with the
// last error set) when it cannot be had.
void *static_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hip_status("hipGetDevice");
        return nullptr;
    }
    if (dev < 0 || dev >= MAX_DEVICES) {
        snprintf(g_last_error, sizeof g_last_error, "device %d beyond the %d this library tracks", dev, MAX_DEVICES);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            snprintf(g_last_error, sizeof g_last_error, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
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
    P.row_cus = cu_count();
    P.row_skew = mode == MODE_GREEDY ? ROW_SKEW_GREEDY : ROW_SKEW_LSE;
    // SPECVERIFY_CHUNK=n: force n chunks per logit row in the row pass (a
    // different decomposition of the same work; outputs must not change)
    const char *ce = getenv("SPECVERIFY_CHUNK");
    P.chunks = ce ? std::max(0, atoi(ce)) : 0;
    P.cs = (int)ceil_div(nvec_max(V, P.bf16 ? 8 : 4), (int64_t)UNIT_E / (P.bf16 ? 8 : 4));
    // A batch whose units would fill few wave slots splits each unit over two
    // or four waves (measured on MI355X on the B = 4, K = 3 shape).
    const int64_t units = (int64_t)B * P.cs;
    P.usplit = units >= 2048 ? 1 : units >= 1024 ? 2 : 4;
    P.aligned = ((int64_t)V * (P.bf16 ? 2 : 4)) % 16 == 0;
    P.ws = carve(ws, L, B);
    return P;
}

}  // namespace

extern "C" {

sv_status spec_verify_read_ceiling(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || !aligned16(buf)) return SV_ERR_INVALID_ARG;
    const int64_t grid = (int64_t)cu_count() * CEIL_WGS_PER_CU;
    (void)hipGetLastError();
    hipLaunchKernelGGL(read_ceiling_kernel, dim3((unsigned)grid), dim3(WG), 0, stream, (const uint4 *)buf,
                       (int64_t)(bytes / 16), sink);
    return hip_status("read_ceiling_kernel launch");
}

sv_status spec_verify_timing_begin(int32_t n)
{
    if (n < 0 || n > (1 << 20)) return SV_ERR_INVALID_ARG;
    for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
    g_timing.ev.clear();
    g_timing.armed = g_timing.used = 0;
    (void)hipGetLastError();
    for (int i = 0; i < 4 * n; ++i) {
        hipEvent_t e;
        if (hipEventCreateWithFlags(&e, hipEventDefault) != hipSuccess) return hip_status("hipEventCreate");
        g_timing.ev.push_back(e);
    }
    g_timing.armed = n;
    return SV_OK;
}

sv_status spec_verify_timing_end(float *ms, int32_t n)
{
    if (n < 0 || n > g_timing.used || (n > 0 && !ms)) return SV_ERR_INVALID_ARG;
    (void)hipGetLastError();
    for (int i = 0; i < n; ++i) {
        if (hipEventSynchronize(stage_event(i, 3)) != hipSuccess) return hip_status("hipEventSynchronize");
        for (int s = 0; s < 3; ++s) {
            float t = 0.0f;
            if (hipEventElapsedTime(&t, stage_event(i, s), stage_event(i, s + 1)) != hipSuccess)
                return hip_status("hipEventElapsedTime");
            ms[3 * i + s] = t;
        }
    }
    for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
    g_timing.ev.clear();
    g_timing.armed = g_timing.used = 0;
    return SV_OK;
}

int32_t spec_verify_abi_version(void) { return 1; }

const char *spec_verify_last_error(void) { return g_last_error; }

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
    return checked(launch(P, stream), num_accepted, B, stream, "spec_verify_greedy");
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
    return checked(launch(P, stream), num_accepted, B, stream, "spec_verify_sample");
}

sv_status spec_verify_greedy_packed(const void *target_logits, sv_dtype dt, const int32_t *draft_tokens,
                                    const int32_t *draft_offsets, int32_t B, int32_t K_max, int32_t n_draft_rows,
                                    int32_t V, int32_t *out_tokens, int32_t *num_accepted, void *workspace,
                                    size_t ws_bytes, hipStream_t stream)
{
    sv_status st = check_shape(B, K_max, V);
    if (st != SV_OK) return st;
    if ((st = check_packed(n_draft_rows)) != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!target_logits || !draft_offsets || !out_tokens || !num_accepted || (n_draft_rows > 0 && !draft_tokens))
        return SV_ERR_INVALID_ARG;
    if (!aligned16(target_logits)) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K_max, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K_max, V, dt, MODE_GREEDY, L, workspace);
    P.target = target_logits;
    P.tokens = draft_tokens;
    P.offs = draft_offsets;
    P.n_rows = n_draft_rows;
    P.out_tokens = out_tokens;
    P.num_accepted = num_accepted;
    return checked(launch(P, stream), num_accepted, B, stream, "spec_verify_greedy_packed");
}

sv_status spec_verify_sample_packed(const void *target_logits, const void *draft_logits, sv_dtype dt,
                                    const int32_t *draft_tokens, const int32_t *draft_offsets,
                                    const float *temperature, const float *u_accept, const float *u_sample,
                                    int32_t B, int32_t K_max, int32_t n_draft_rows, int32_t V, int32_t *out_tokens,
                                    int32_t *num_accepted, float *p_draft, float *q_draft, void *workspace,
                                    size_t ws_bytes, hipStream_t stream)
{
    sv_status st = check_shape(B, K_max, V);
    if (st != SV_OK) return st;
    if ((st = check_packed(n_draft_rows)) != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!target_logits || !draft_offsets || !temperature || !u_sample || !out_tokens || !num_accepted)
        return SV_ERR_INVALID_ARG;
    if (n_draft_rows > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
    if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits))) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K_max, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K_max, V, dt, MODE_SAMPLE, L, workspace);
    P.target = target_logits;
    P.draft = draft_logits;
    P.tokens = draft_tokens;
    P.offs = draft_offsets;
    P.n_rows = n_draft_rows;
    P.temperature = temperature;
    P.u_accept = u_accept;
    P.u_sample = u_sample;
    P.out_tokens = out_tokens;
    P.num_accepted = num_accepted;
    P.p_draft = p_draft;
    P.q_draft = q_draft;
    return checked(launch(P, stream), num_accepted, B, stream, "spec_verify_sample_packed");
}

sv_status spec_verify_sample_noalloc(const void *target_logits, const void *draft_logits, sv_dtype dt,
                                     const int32_t *draft_tokens, const int32_t *depth, const float *temperature,
                                     const float *u_accept, const float *u_sample, int32_t B, int32_t K, int32_t V,
                                     int32_t *out_tokens, int32_t *num_accepted, float *p_draft, float *q_draft,
                                     hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!target_logits || !temperature || !u_sample || !out_tokens || !num_accepted) return SV_ERR_INVALID_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
    if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits))) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K, V, L);
    if (L.total > STATIC_SCRATCH_BYTES) {
        snprintf(g_last_error, sizeof g_last_error,
                 "spec_verify_sample_noalloc: B=%d K=%d V=%d needs %zu bytes of scratch, above its %zu-byte static array",
                 (int)B, (int)K, (int)V, L.total, STATIC_SCRATCH_BYTES);
        return SV_ERR_UNSUPPORTED;
    }
    void *ws = static_scratch();
    if (!ws) return SV_ERR_HIP;
    Params P = base_params(B, K, V, dt, MODE_SAMPLE, L, ws);
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
    return launch(P, stream);
}

sv_status spec_verify_greedy_early_exit(const void *target_logits, sv_dtype dt, const int32_t *draft_tokens,
                                        const int32_t *depth, int32_t B, int32_t K, int32_t V,
                                        const int32_t *window_ends, int32_t n_windows, int32_t *out_tokens,
                                        int32_t *num_accepted, void *workspace, size_t ws_bytes,
                                        hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    std::vector<int> ends;
    if (!window_plan(window_ends, n_windows, K, ends)) return SV_ERR_INVALID_ARG;
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
    const sv_status ls = launch_windows(P, ends, stream);
    return checked(ls, num_accepted, B, stream, "spec_verify_greedy_early_exit");
}

sv_status spec_verify_sample_early_exit(const void *target_logits, const void *draft_logits, sv_dtype dt,
                                        const int32_t *draft_tokens, const int32_t *depth,
                                        const float *temperature, const float *u_accept, const float *u_sample,
                                        int32_t B, int32_t K, int32_t V, const int32_t *window_ends,
                                        int32_t n_windows, int32_t *out_tokens, int32_t *num_accepted,
                                        float *p_draft, float *q_draft, void *workspace, size_t ws_bytes,
                                        hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    std::vector<int> ends;
    if (!window_plan(window_ends, n_windows, K, ends)) return SV_ERR_INVALID_ARG;
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
    const sv_status ls = launch_windows(P, ends, stream);
    return checked(ls, num_accepted, B, stream, "spec_verify_sample_early_exit");
}

sv_status spec_verify_sample_reuse(const void *target_logits, const void *draft_logits, sv_dtype dt,
                                   const int32_t *draft_tokens, const int32_t *depth, const float *temperature,
                                   const float *u_accept, const float *u_sample, const void *draft_stats,
                                   int32_t B, int32_t K, int32_t V, int32_t *out_tokens, int32_t *num_accepted,
                                   float *p_draft, float *q_draft, void *workspace, size_t ws_bytes,
                                   hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (!target_logits || !temperature || !u_sample || !out_tokens || !num_accepted) return SV_ERR_INVALID_ARG;
    if (K > 0 && (!draft_logits || !draft_tokens || !u_accept || !draft_stats)) return SV_ERR_INVALID_ARG;
    if (!aligned16(target_logits) || (draft_logits && !aligned16(draft_logits))) return SV_ERR_INVALID_ARG;
    if (draft_stats && ((uintptr_t)draft_stats & 15u) != 0) return SV_ERR_INVALID_ARG;
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
    P.dstats_in = (const Stat *)draft_stats;
    return checked(launch(P, stream), num_accepted, B, stream, "spec_verify_sample_reuse");
}

sv_status spec_draft_confidence_stats(const void *draft_logits, sv_dtype dt, const int32_t *max_depth, int32_t B,
                                      int32_t K, int32_t V, float *conf, void *draft_stats, void *workspace,
                                      size_t ws_bytes, hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (K == 0) return SV_OK;
    if (!draft_logits || !draft_stats || ((uintptr_t)draft_stats & 15u) != 0) return SV_ERR_INVALID_ARG;
    if (!aligned16(draft_logits)) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K, V, dt, MODE_CONF, L, workspace);
    P.draft = draft_logits;
    P.max_depth = max_depth;
    P.conf = conf;
    P.dstats_out = (Stat *)draft_stats;
    return launch(P, stream);
}

sv_status spec_draft_confidence_stats_t(const void *draft_logits, sv_dtype dt, const int32_t *max_depth,
                                        const float *temperature, int32_t B, int32_t K, int32_t V, float *conf,
                                        void *draft_stats, void *workspace, size_t ws_bytes, hipStream_t stream)
{
    sv_status st = check_shape(B, K, V);
    if (st != SV_OK) return st;
    if (dt != SV_F32 && dt != SV_BF16) return SV_ERR_INVALID_ARG;
    if (K == 0) return SV_OK;
    if (!draft_logits || !draft_stats || !temperature || ((uintptr_t)draft_stats & 15u) != 0)
        return SV_ERR_INVALID_ARG;
    if (!aligned16(draft_logits)) return SV_ERR_INVALID_ARG;
    Layout L;
    make_layout(B, K, V, L);
    if ((st = check_ws(workspace, ws_bytes, L)) != SV_OK) return st;
    Params P = base_params(B, K, V, dt, MODE_CONF, L, workspace);
    P.draft = draft_logits;
    P.max_depth = max_depth;
    P.conf_temp = temperature;
    P.conf = conf;
    P.dstats_out = (Stat *)draft_stats;
    return launch(P, stream);
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
    return launch(P, stream);
}

sv_status spec_early_exit_plan(const double *alpha, int32_t K, double window_cost, int32_t *ends,
                               int32_t *n_windows)
{
    if (!ends || !n_windows || K < 0 || K > K_MAX || (K > 0 && !alpha)) return SV_ERR_INVALID_ARG;
    if (!(window_cost >= 0.0) || window_cost > 1e30) return SV_ERR_INVALID_ARG;
    // a NaN rate is a position no request reached: it counts as 0
    for (int32_t k = 0; k < K; ++k)
        if (!(alpha[k] >= 0.0 && alpha[k] <= 1.0) && alpha[k] == alpha[k]) return SV_ERR_INVALID_ARG;
    if (K == 0) {
        ends[0] = 1;
        *n_windows = 1;
        return SV_OK;
    }
    // live[p]: probability that a request still verifies position p
    std::vector<double> live((size_t)K + 1), best((size_t)K + 1);
    std::vector<int32_t> next((size_t)K + 1);
    live[0] = 1.0;
    for (int32_t p = 0; p < K; ++p) live[(size_t)p + 1] = live[(size_t)p] * (alpha[p] == alpha[p] ? alpha[p] : 0.0);
    // best[p]: least expected cost of the windows covering positions p..K-1
    best[(size_t)K] = 0.0;
    for (int32_t p = K - 1; p >= 0; --p) {
        double bc = 0.0;
        int32_t bq = -1;
        for (int32_t q = K; q > p; --q) {   // ties keep the longer window
            const double c = window_cost + live[(size_t)p] * (double)(q - p) + best[(size_t)q];
            if (bq < 0 || c < bc) {
                bc = c;
                bq = q;
            }
        }
        best[(size_t)p] = bc;
        next[(size_t)p] = bq;
    }
    int32_t n = 0;
    for (int32_t p = 0; p < K; p = next[(size_t)p]) ends[n++] = next[(size_t)p];
    *n_windows = n;
    return SV_OK;
}

sv_status spec_accept_stats_summary(const unsigned long long *counters, int32_t K, double *alpha,
                                    double *mean_accepted, double *tau)
{
    if (!counters || K < 0 || K > K_MAX || (K > 0 && !alpha) || !mean_accepted || !tau) return SV_ERR_INVALID_ARG;
    for (int32_t k = 0; k < K; ++k) {
        const unsigned long long reached = counters[k], accepted = counters[K + k];
        alpha[k] = reached ? (double)accepted / (double)reached : NAN;
    }
    const unsigned long long req = counters[2 * K];
    *mean_accepted = req ? (double)counters[2 * K + 2] / (double)req : NAN;
    *tau = req ? (double)counters[2 * K + 3] / (double)req : NAN;
    return SV_OK;
}

sv_status dcut_allocate_cost(const float *conf, const int32_t *max_depth, int32_t B, int32_t K,
                             const double *table_depth, const double *table_cost, int32_t table_n,
                             double max_verify, int32_t *depth_out, hipStream_t stream)
{
    if (B < 1 || K < 0 || !depth_out || (K > 0 && !conf)) return SV_ERR_INVALID_ARG;
    if (B > COST_B_MAX || K > K_MAX) return SV_ERR_UNSUPPORTED;
    if (!table_depth || !table_cost || table_n < 1 || table_n > COST_TAB_MAX) return SV_ERR_INVALID_ARG;
    if (!(max_verify >= 0.0) || max_verify == INFINITY) return SV_ERR_INVALID_ARG;
    CostTable T;
    memset(&T, 0, sizeof T);
    T.n = table_n;
    for (int i = 0; i < table_n; ++i) {
        const double t = table_depth[i], c = table_cost[i];
        if (!std::isfinite(t) || !std::isfinite(c) || !(c > 0.0)) return SV_ERR_INVALID_ARG;
        if (i > 0 && !(t > table_depth[i - 1])) return SV_ERR_INVALID_ARG;
        T.t[i] = t;
        T.c[i] = c;
    }
    int64_t N = 1;
    while (N < B) N <<= 1;
    // costs per depth, sort keys and requests, bids (rounded up to whole
    // doubles), then the staged confidences of small inputs
    constexpr size_t LDS_DYN_MAX = 60 * 1024;   // with the kernel's 4.6 KiB of static LDS, within 64 KiB
    size_t lds = sizeof(double) * (size_t)((K + 1) + N + (N + B + 3) / 4);
    if (lds > LDS_DYN_MAX) return SV_ERR_UNSUPPORTED;
    // small inputs: confidences staged (4 B per pair), and with room for
    // them the pair-parallel values (8 B per pair)
    const size_t pairs = (size_t)B * (size_t)K;
    int flags = 0;
    if ((int64_t)pairs <= COST_PAIRS && lds + 12 * pairs <= LDS_DYN_MAX) {
        flags = 3;
        lds += 12 * pairs;
    } else if ((int64_t)pairs <= COST_STAGE && lds + 4 * pairs <= LDS_DYN_MAX) {
        flags = 1;
        lds += 4 * pairs;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(dcut_cost_kernel, dim3(1), dim3(COST_WG), lds, stream, conf, max_depth, B, K, T, max_verify,
                       flags, depth_out);
    return hip_status("dcut_cost_kernel launch");
}

sv_status spec_accept_stats_update(const int32_t *num_accepted, const int32_t *depth, int32_t B, int32_t K,
                                   unsigned long long *counters, hipStream_t stream)
{
    if (B < 1 || K < 0 || !num_accepted || !counters) return SV_ERR_INVALID_ARG;
    if (B > B_MAX || K > K_MAX) return SV_ERR_UNSUPPORTED;
    if (((uintptr_t)counters & 7u) != 0) return SV_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const size_t lds = sizeof(unsigned int) * (size_t)(2 * K + 1);
    hipLaunchKernelGGL(accept_stats_kernel, dim3(1), dim3(STATS_WG), lds, stream, num_accepted, depth, B, K,
                       counters);
    return hip_status("accept_stats_kernel launch");
}

sv_status dcut_allocate(const float *conf, const int32_t *max_depth, int32_t B, int32_t K, int32_t budget,
                        int32_t *depth_out, hipStream_t stream)
{
    if (B < 1 || K < 0) return SV_ERR_INVALID_ARG;
    if ((int64_t)B * K > DCUT_MAX || B > B_MAX || K > K_MAX) return SV_ERR_UNSUPPORTED;
    if (!depth_out || (K > 0 && !conf)) return SV_ERR_INVALID_ARG;
    if (budget < B) return SV_ERR_BUDGET;
    const size_t lds = sizeof(uint32_t) * (size_t)std::max<int64_t>(1, (int64_t)B * K);
    if (!dcut_lds_ok(lds)) return SV_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    hipLaunchKernelGGL(dcut_kernel, dim3(1), dim3(DCUT_WG), lds, stream, conf, max_depth, B, K, budget, depth_out);
    return checked(hip_status("dcut_kernel launch"), depth_out, B, stream, "dcut_allocate");
}

}  // extern "C"
