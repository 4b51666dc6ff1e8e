// Team selection of one query head (gfx950): representative scores, team
// softmax, inverse-CDF draws, dedupe and inclusion probabilities.
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract: the draws depend only on the query's
//         dot products with the teams' summary keys; a drawn team's terms
//         count 1/pi times, pi its chance of being drawn.
//   [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
//         section 三 steps 2-3: team scores, a softmax over teams, M draws.
//   [PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
//         1, 2, 3", SC'11 (Philox4x32-10).
//   [SAN] "Stochastic Sparse Attention for Memory-Bound Inference" (the
//         SANTA page), abstract: stratified and systematic sampling as
//         lower-variance draws; here they place the team draws.
//
// Every quantity is computed in a fixed order that does not depend on the
// shape of the block running it, so the standalone selection kernel and the
// fused decode kernel produce the same bits:
//   score    four parts of D/4 channels each; in a part, one float64 FMA
//            chain over the even channel offsets and one over the odd ones,
//            in channel order from 0.0; s = ((p0 + p1) + (p2 + p3)) / sqrt(d)
//            with p_k = even_k + odd_k. Products of two bfloat16 or two
//            float32 values are exact in float64.
//   softmax  m = the largest float32-rounded score; e_t = exp(s_t - m) in
//            float64 (any shift near the max cancels in the draws and in p).
//   scan     one wavefront per head: lane l owns teams [l per, (l + 1) per),
//            per = ceil(K / 64); lane sums in team order, an inclusive scan
//            of the 64 lane sums in the fixed order of wave_incl_scan, then
//            C_t = (incl_l - sum_l) + e_(l per) + ... + e_t in team order.
//            Z = C_(K-1).
//   draws    point_j from Philox word j mod 4 of counter (j / 4, h, b, offset)
//            (scheme as in [SAN]), target = point_j Z, team = the binary
//            search result for the first t with target < C_t.
//   pi       float64 for every drawn team; log w = -log(pi) and w = 1/pi are
//            rounded to float32 once.
// The score may be formed by any thread layout that keeps these four chains
// and the ((p0 + p1) + (p2 + p3)) sum: four lanes per row with DPP quad
// exchanges (row_score) or one lane per row over the four parts in turn.
#pragma once

#include "device_common.h"

namespace santa {
namespace sel {

using namespace dev;

constexpr int kParts = 4;          // consecutive lanes per representative row

// Value of lane (lane ^ 1) or (lane ^ 2) inside each group of four lanes,
// by a DPP quad permutation of the two 32-bit halves (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ double quad_perm(double x) {
    const long long v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, int(v >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]

template <typename KV, int D>
struct Part {
    static constexpr int VPC = KVTraits<KV>::kPerChunk;   // values per 16 bytes
    static constexpr int N = D / kParts;                  // channels per part
    static constexpr int LOADS = N / VPC;                 // 16-byte loads per part
};

// The 16-byte pieces of part `part` of a representative row.
template <typename KV, int D>
__device__ __forceinline__ void load_part(const KV *row, int part, uint4 (&raw)[Part<KV, D>::LOADS]) {
    const KV *r = row + part * Part<KV, D>::N;
#pragma unroll
    for (int j = 0; j < Part<KV, D>::LOADS; ++j) raw[j] = ld16(r + j * Part<KV, D>::VPC);
}

// The part's channels as float64 (exact), in channel order.
template <typename KV, int D>
__device__ __forceinline__ void part_to_f64(const uint4 (&raw)[Part<KV, D>::LOADS], double (&x)[Part<KV, D>::N]) {
    constexpr int VPC = Part<KV, D>::VPC;
#pragma unroll
    for (int j = 0; j < Part<KV, D>::LOADS; ++j) {
        float f[8];
        unpack(raw[j], f, KV{});
#pragma unroll
        for (int e = 0; e < VPC; ++e) x[j * VPC + e] = double(f[e]);
    }
}

// Sum of one part: even and odd channel chains (q: the head's float64 query
// at the part's first channel).
template <int N>
__device__ __forceinline__ double part_dot(const double (&x)[N], const double *q) {
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        a0 = fma(x[i], q[i], a0);
        a1 = fma(x[i + 1], q[i + 1], a1);
    }
    return a0 + a1;
}

// The same sum with the part's query values in registers (float64) and the
// row's values converted as they are used.
template <typename KV, int D>
__device__ __forceinline__ double part_dot_raw(const uint4 (&raw)[Part<KV, D>::LOADS],
                                               const double (&q)[Part<KV, D>::N]) {
    constexpr int VPC = Part<KV, D>::VPC;
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int j = 0; j < Part<KV, D>::LOADS; ++j) {
        float f[8];
        unpack(raw[j], f, KV{});
#pragma unroll
        for (int e = 0; e < VPC; e += 2) {
            a0 = fma(double(f[e]), q[j * VPC + e], a0);
            a1 = fma(double(f[e + 1]), q[j * VPC + e + 1], a1);
        }
    }
    return a0 + a1;
}

// The same sum with the part's query values held as float32 (the query is a
// float32 value; each is widened as it is used, so the products are those
// of the float64 form).
template <typename KV, int D>
__device__ __forceinline__ double part_dot_raw(const uint4 (&raw)[Part<KV, D>::LOADS],
                                               const float (&q)[Part<KV, D>::N]) {
    constexpr int VPC = Part<KV, D>::VPC;
    double a0 = 0.0, a1 = 0.0;
#pragma unroll
    for (int j = 0; j < Part<KV, D>::LOADS; ++j) {
        float f[8];
        unpack(raw[j], f, KV{});
#pragma unroll
        for (int e = 0; e < VPC; e += 2) {
            a0 = fma(double(f[e]), double(q[j * VPC + e]), a0);
            a1 = fma(double(f[e + 1]), double(q[j * VPC + e + 1]), a1);
        }
    }
    return a0 + a1;
}

// Score of a row from its four parts' sums (lanes 4i .. 4i + 3); every lane
// of the quad gets the same value.
__device__ __forceinline__ double row_score(double pk, double scale) {
    pk += quad_perm<kQuadXor1>(pk);
    pk += quad_perm<kQuadXor2>(pk);
    return pk * scale;
}

// Wavefront-wide operations on DPP (no LDS round trip). The inclusive scan
// runs in a fixed order: Hillis-Steele inside each row of 16 lanes (row
// shifts by 1, 2, 4, 8), then lane 15 of rows 0 and 2 is added to rows 1 and
// 3, then lane 31 to rows 2 and 3.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int x, int old) {
    return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_zero_d(double x) {       // lanes not written or out of row get 0
    const long long v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, int(v), CTRL, ROWS, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, int(v >> 32), CTRL, ROWS, 0xF, true);
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}

__device__ __forceinline__ double wave_incl_scan(double x) {
    x += dpp_zero_d<kRowShr1, 0xF>(x);
    x += dpp_zero_d<kRowShr2, 0xF>(x);
    x += dpp_zero_d<kRowShr4, 0xF>(x);
    x += dpp_zero_d<kRowShr8, 0xF>(x);
    x += dpp_zero_d<kRowBcast15, 0xA>(x);
    x += dpp_zero_d<kRowBcast31, 0xC>(x);
    return x;
}

__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_i<kRowShr1, 0xF>(x, 0);
    x += dpp_i<kRowShr2, 0xF>(x, 0);
    x += dpp_i<kRowShr4, 0xF>(x, 0);
    x += dpp_i<kRowShr8, 0xF>(x, 0);
    x += dpp_i<kRowBcast15, 0xA>(x, 0);
    x += dpp_i<kRowBcast31, 0xC>(x, 0);
    return x;
}

// Sum over the wavefront (in the fixed order of the scan), the same in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    int v = __float_as_int(x);
    v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<kRowShr1, 0xF>(v, 0)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<kRowShr2, 0xF>(v, 0)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<kRowShr4, 0xF>(v, 0)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<kRowShr8, 0xF>(v, 0)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<kRowBcast15, 0xA>(v, 0)));
    v = __float_as_int(__int_as_float(v) + __int_as_float(dpp_i<kRowBcast31, 0xC>(v, 0)));
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// Largest value over the wavefront, the same in every lane.
__device__ __forceinline__ float wave_max(float x) {
    int v = __float_as_int(x);
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<kRowShr1, 0xF>(v, v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<kRowShr2, 0xF>(v, v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<kRowShr4, 0xF>(v, v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<kRowShr8, 0xF>(v, v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<kRowBcast15, 0xA>(v, v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<kRowBcast31, 0xC>(v, v))));
    return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__device__ __forceinline__ double readlane_d(double x, int lane) {
    const long long v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_readlane(int(v), lane);
    const int hi = __builtin_amdgcn_readlane(int(v >> 32), lane);
    return __longlong_as_double((long long)(unsigned)lo | ((long long)hi << 32));
}

// Everything a head's selection tail needs besides its LDS rows.
struct TailArgs {
    int K;                 // teams of the sequence
    int M;                 // draws
    int scheme;            // santa_draw_scheme
    uint32_t seed_lo, seed_hi, offset;
    int h, b;              // query head and sequence (Philox counter words)
};

// Draw points in [0, 1): point j is u_j (independent draws), (j + u_0) / M
// (systematic) or (j + u_j) / M (stratified, [SAN]), u = (x + 1/2) 2^-32
// with x word j mod 4 of Philox4x32-10 at counter (j / 4, h, b, offset) and
// key (seed lo, seed hi) ([PHX]). j + u is exact in float64. Thread `first`
// of `stride` threads writes points first, first + stride, ... below M.
__device__ __forceinline__ void draw_points(const TailArgs &a, double *pts, int first, int stride) {
    double u0 = 0.0;
    if (a.scheme == SANTA_DRAW_SYSTEMATIC) {
        const uint4 r0 = philox4x32_10(make_uint4(0u, uint32_t(a.h), uint32_t(a.b), a.offset), a.seed_lo, a.seed_hi);
        u0 = (double(r0.x) + 0.5) * 0x1p-32;
    }
    for (int j = first; j < a.M; j += stride) {
        const uint4 r = philox4x32_10(make_uint4(uint32_t(j) >> 2, uint32_t(a.h), uint32_t(a.b), a.offset),
                                      a.seed_lo, a.seed_hi);
        const uint32_t x = (j & 3) == 0 ? r.x : (j & 3) == 1 ? r.y : (j & 3) == 2 ? r.z : r.w;
        const double uj = (double(x) + 0.5) * 0x1p-32;
        double point = uj;
        if (a.scheme == SANTA_DRAW_SYSTEMATIC) point = (double(j) + u0) / double(a.M);
        else if (a.scheme == SANTA_DRAW_STRATIFIED) point = (double(j) + uj) / double(a.M);
        pts[j] = point;
    }
}

// Inclusion probability of drawn team t, from e_t, the cumulative sums C and
// Z = C_(K-1): independent draws 1 - (1 - p)^M = -expm1(M log1p(-p)) ([ABS]:
// the weight of a drawn team is 1/pi); systematic min(1, M p);
// stratified ([SAN]): in units of 1/M the team covers [a, a + w),
// a = M C_(t-1) / Z, w = M p, meeting unit floor(a) over
// q1 = min(w, floor(a) + 1 - a) and the next units over r = w - q1, so
// pi = 1 if r >= 1 (a whole unit inside), else w - q1 r. Every operation
// rounds as written (no contraction), so all callers get the same bits.
__device__ __forceinline__ double inclusion(const double *e, const double *c, int t, double Z, int M, int scheme) {
#pragma clang fp contract(off)
    const double pt = e[t] / Z;
    if (scheme == SANTA_DRAW_SYSTEMATIC) return fmin(1.0, double(M) * pt);
    if (scheme == SANTA_DRAW_STRATIFIED) {
        const double cprev = t > 0 ? c[t - 1] : 0.0;
        const double wd = double(M) * pt;
        const double av = double(M) * cprev / Z;
        const double q1 = fmin(wd, (floor(av) + 1.0) - av);
        const double rest = wd - q1;
        return rest >= 1.0 ? 1.0 : wd - q1 * rest;
    }
    return -expm1(double(M) * log1p(-pt));
}

// log w = -log(pi) as the float32 logarithm of the float32-rounded pi. It
// only shifts a drawn team's logits (a relative error near 1e-7 in that
// team's terms); the weights reported as 1/pi are float64 quotients.
__device__ __forceinline__ float log_weight(double pi) { return -logf(float(pi)); }

// Team softmax numerators of one head, by `stride` threads of the block
// (thread `first` takes teams first, first + stride, ...): m is the largest
// of the nw per-wavefront maxima in wmax, each the largest float32-rounded
// score of its wavefront's rows (-inf for none), so m is the float32-rounded
// maximum score; s_t is overwritten with e_t = exp(s_t - m). The caller
// makes the block wait before the scan reads them.
__device__ __forceinline__ void team_exps(double *s, int K, const float *wmax, int nw, int first, int stride) {
    float mx = -INFINITY;
    for (int w = 0; w < nw; ++w) mx = fmaxf(mx, wmax[w]);
    const double m = double(mx);
    for (int t = first; t < K; t += stride) s[t] = exp(s[t] - m);
}

// Selection tail of one head, run by one whole wavefront (all 64 lanes call
// it; no block barrier inside), after team_exps: cumulative sums and draws.
//   e     [K] float64 e_t in LDS
//   c     [K] float64 in LDS: the cumulative sums C_t
//   bits  [ceil(K/32)] team bitmap in LDS, cleared, then set for drawn teams
//         (every team when M >= K)
//   pts   [M] draw points (draw_points), read when M < K
//   lnw_t, ipi_t  optional [K] LDS arrays by team: the lane that draws team
//         t stores log_weight(pi_t) and float(1 / pi_t) there (several draws
//         of one team store the same values); untouched when M >= K
// Draw j takes the first team t with pts[j] Z < C_t (binary search); if none
// qualifies (points below 1 cannot cause that) the last team with mass.
// Returns Z = C_(K-1) (0 for an empty sequence).
__device__ __forceinline__ double head_tail(const double *s, double *c, uint32_t *bits, const double *pts,
                                            const TailArgs &a, float *lnw_t = nullptr, float *ipi_t = nullptr) {
    const int lane = threadIdx.x & 63;
    const int K = a.K;
    const int words = (K + 31) >> 5;
    for (int w = lane; w < words; w += 64) bits[w] = 0u;
    if (K == 0) return 0.0;

    const int per = (K + 63) >> 6;
    const int t0 = min(K, lane * per), t1 = min(K, t0 + per);
    double local = 0.0;
    for (int t = t0; t < t1; ++t) local += s[t];
    const double incl = wave_incl_scan(local);
    double run = incl - local;
    for (int t = t0; t < t1; ++t) {
        run += s[t];
        c[t] = run;
    }
    const double Z = readlane_d(run, (K - 1) / per);        // C_(K-1): its owner's last sum
    __builtin_amdgcn_wave_barrier();

    if (a.M >= K) {
        for (int w = lane; w < words; w += 64)
            bits[w] = (w < words - 1 || (K & 31) == 0) ? 0xffffffffu : ((1u << (K & 31)) - 1u);
    } else {
        for (int j = lane; j < a.M; j += 64) {
            const double target = pts[j] * Z;
            int t;
            if (target < Z) {
                int lo = 0, hi = K - 1;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (target < c[mid]) hi = mid; else lo = mid + 1;
                }
                t = lo;
            } else {
                t = K - 1;
                while (t > 0 && !(s[t] > 0.0)) --t;
            }
            atomicOr(&bits[t >> 5], 1u << (t & 31));
            if (lnw_t) {
                const double pi = inclusion(s, c, t, Z, a.M, a.scheme);
                lnw_t[t] = log_weight(pi);
                if (ipi_t) ipi_t[t] = float(1.0 / pi);
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    return Z;
}

// Drawn teams of one head in ascending order, with their weights (one
// wavefront): rank r = position of the team in the bitmap. For each drawn
// team t: lnw[t] = log w_t = log_weight(pi_t) (0 under full coverage), and,
// when `sampled` is given, sampled[r] = t and
// inv_pi[r] = 1/pi_t, -1 / 0 padded to M. `pre` is [ceil(K/32) + 1] LDS
// scratch.
__device__ __forceinline__ void drawn_weights(const double *e, const double *c, const uint32_t *bits, double Z,
                                              const TailArgs &a, int32_t *pre, float *lnw, int32_t *sampled,
                                              float *inv_pi) {
    const int lane = threadIdx.x & 63;
    const int K = a.K;
    const int words = (K + 31) >> 5;
    int drawn = 0;
    for (int w0 = 0; w0 < words; w0 += 64) {
        const int w = w0 + lane;
        const int cnt = w < words ? __popc(bits[w]) : 0;
        const int ic = wave_incl_scan(cnt);
        if (w < words) pre[w] = drawn + ic - cnt;
        drawn += __builtin_amdgcn_readlane(ic, 63);
    }
    __builtin_amdgcn_wave_barrier();
    const bool full = a.M >= K;
    for (int r = lane; r < drawn; r += 64) {
        int lo = 0, hi = words - 1;                         // last word whose prefix is <= r
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= r) lo = mid; else hi = mid - 1;
        }
        uint32_t u = bits[lo];
        for (int k = r - pre[lo]; k > 0; --k) u &= u - 1u;
        const int t = lo * 32 + __ffs(u) - 1;
        const double pi = full ? 1.0 : inclusion(e, c, t, Z, a.M, a.scheme);
        lnw[t] = full ? 0.0f : log_weight(pi);
        if (sampled) {
            sampled[r] = t;
            inv_pi[r] = full ? 1.0f : float(1.0 / pi);
        }
    }
    if (sampled)
        for (int r = drawn + lane; r < a.M; r += 64) {
            sampled[r] = -1;
            inv_pi[r] = 0.0f;
        }
}

}  // namespace sel
}  // namespace santa
