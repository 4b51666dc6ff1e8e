// HIP kernels of libsanta for gfx950 (CDNA4, 64-lane wavefronts).
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract.
//   [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
//         section 三 (core method).
//   [PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
//         1, 2, 3", SC'11, Philox4x32 with 10 rounds.
//
// Kernels, in the order a decode step runs them:
//   build_reps  (once per prefill / page append) mean key per (page, KV head)
//   select      one block per (sequence, query head): representative scores,
//               team softmax and cumulative sums, Philox draws, inverse-CDF
//               lookup, dedupe, inclusion probabilities; writes the head's
//               team bitmap and log-weights
//   given       (test / advanced entry) the same bitmap + log-weights from a
//               caller-supplied team list
//   gather      split-K over the union of a KV head's drawn teams: streams
//               each union team's K and V tile once, scores it for the query
//               heads that drew it, and runs a weighted online softmax
//   combine     merges the split partials of each (sequence, query head) in
//               a fixed order
// Dense decode is gather (every team, weight 1) + combine.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "santa_internal.h"

namespace santa {

namespace {

constexpr float kNegInfF = -INFINITY;

// ---------------------------------------------------------------------------
// Storage types
// ---------------------------------------------------------------------------

using bf16_t = uint16_t;   // bfloat16 bits

// The score type of a storage type: products of two bfloat16 values are exact
// in float32, and float32 accumulation is within the bfloat16 tolerance;
// float32 caches are scored in float64 (products of two float32 values are
// exact in float64).
template <typename KV> struct KVTraits;
template <> struct KVTraits<bf16_t> { using Score = float; static constexpr int kPerChunk = 8; };
template <> struct KVTraits<float> { using Score = double; static constexpr int kPerChunk = 4; };

__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// 16 bytes of cache -> floats (8 bfloat16 or 4 float32), exact.
__device__ __forceinline__ void unpack(const uint4 v, float *f, bf16_t) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack(const uint4 v, float *f, float) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

__device__ __forceinline__ uint4 ld16(const void *ptr) {
    return *reinterpret_cast<const uint4 *>(ptr);
}

// Round a float64 to the nearest bfloat16 in one step, ties to even. The
// spacing of bfloat16 values near |x| = f 2^e (f in [0.5, 1)) is 2^(e-8),
// or the subnormal step 2^-133 below 2^-126; scaling by it is exact, and
// rint rounds to the nearest integer with ties to even.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
    if (x != x) return bf16_t(0x7fc0);
    const bf16_t sign = signbit(x) ? bf16_t(0x8000) : bf16_t(0);
    const double ax = fabs(x);
    if (ax == 0.0) return sign;
    int e;
    (void)frexp(ax, &e);
    const int qe = (e - 1 < -126) ? -133 : e - 8;
    const double r = ldexp(rint(ldexp(ax, -qe)), qe);
    if (r > 0x1.fep127) return bf16_t(sign | 0x7f80);
    return bf16_t(sign | (__float_as_uint(float(r)) >> 16));   // r is a bfloat16 value: exact
}

__device__ __forceinline__ void store_rounded(bf16_t *dst, double x) { *dst = f64_to_bf16(x); }
__device__ __forceinline__ void store_rounded(float *dst, double x) { *dst = float(x); }  // IEEE RNE

__device__ __forceinline__ int clamp_len(int L, int max_len) {
    return L < 0 ? 0 : (L > max_len ? max_len : L);
}
__device__ __forceinline__ int64_t clamp_page(int32_t pg, int64_t num_pages) {
    return pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : int64_t(pg));
}

// ---------------------------------------------------------------------------
// Philox4x32-10 [PHX]: per round, the 64-bit products of counter words 0 and
// 2 with two fixed multipliers; new counter = (hi1 ^ c1 ^ k0, lo1,
// hi0 ^ c3 ^ k1, lo0); the key is bumped by two Weyl constants between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// ---------------------------------------------------------------------------
// Block-wide reductions for 256-thread blocks (4 wavefronts)
// ---------------------------------------------------------------------------
constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

__device__ double block_max(double v, double *red) {
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = red[0];
    for (int i = 1; i < kWaves; ++i) r = fmax(r, red[i]);
    return r;
}

// Exclusive prefix sum of one double per thread, in thread order.
__device__ double block_exclusive_sum(double v, double *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    double base = 0.0;
    for (int i = 0; i < wave; ++i) base += red[i];
    return base + excl;
}

// ---------------------------------------------------------------------------
// build_reps: one wavefront per (team, KV head, sequence). [EXP] section 三
// step 2 (one representative key per team; the mean is used): the float64
// sum of the n valid keys, one correctly rounded divide, one rounding to the
// cache type.
// ---------------------------------------------------------------------------
template <typename KV, int D>
__global__ __launch_bounds__(64) void build_reps_kernel(Params p) {
    constexpr int CPL = D / 64;                     // channels per lane
    const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int L = clamp_len(p.seq_lens[b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    if (t >= K) return;
    const int64_t page = clamp_page(p.page_table[size_t(b) * p.P + t], p.num_pages);
    const int n = min(p.T, L - t * p.T);
    const KV *keys = static_cast<const KV *>(p.k_pages) + (size_t(page) * p.Hkv + g) * p.T * D;
    double acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.0;
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[i] += double(to_f32(keys[size_t(j) * D + lane * CPL + i]));
    }
    KV *reps = static_cast<KV *>(p.reps_out) + (size_t(page) * p.Hkv + g) * D;
#pragma unroll
    for (int i = 0; i < CPL; ++i) store_rounded(&reps[lane * CPL + i], acc[i] / double(n));
}

// ---------------------------------------------------------------------------
// select: one 256-thread block per (sequence b, query head h).
// [ABS]: the query scores one representative per team to decide which teams
// to sample; each sampled team is weighted by the inverse of its inclusion
// probability. [EXP] section 三 steps 2-3: s_i = q . rep_i, p = softmax(s),
// sample M teams with probability p.
// ---------------------------------------------------------------------------
template <typename KV, int D>
__global__ __launch_bounds__(kBlock) void select_kernel(Params p) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    __shared__ double q_s[D];
    __shared__ double e_s[kMaxTeams];     // scores, then exp(s - max)
    __shared__ double c_s[kMaxTeams];     // inclusive cumulative sums of e
    __shared__ uint32_t bits_s[kMaxWords];
    __shared__ int32_t wpre_s[kMaxWords];
    __shared__ double red_s[kWaves];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const int L = clamp_len(p.seq_lens[b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;

    const KV *q = static_cast<const KV *>(p.q) + size_t(bh) * D;
    for (int c = tid; c < D; c += kBlock) q_s[c] = double(to_f32(q[c]));
    for (int w = tid; w < p.words; w += kBlock) bits_s[w] = 0u;
    __syncthreads();

    // 1. Representative scores, float64 (exact products, float64 sums).
    const KV *reps = static_cast<const KV *>(p.reps);
    const int32_t *pt = p.page_table + size_t(b) * p.P;
    for (int t = tid; t < K; t += kBlock) {
        const int64_t page = clamp_page(pt[t], p.num_pages);
        const KV *r = reps + (size_t(page) * p.Hkv + g) * D;
        double acc = 0.0;
#pragma unroll 4
        for (int c0 = 0; c0 < D; c0 += VPC) {
            float f[8];
            unpack(ld16(r + c0), f, KV{});
#pragma unroll
            for (int i = 0; i < VPC; ++i) acc = fma(double(f[i]), q_s[c0 + i], acc);
        }
        e_s[t] = acc * p.scale;
    }
    __syncthreads();

    // 2. Team softmax numerators and cumulative sums (float64).
    double m = -INFINITY;
    for (int t = tid; t < K; t += kBlock) m = fmax(m, e_s[t]);
    m = block_max(m, red_s);
    for (int t = tid; t < K; t += kBlock) e_s[t] = exp(e_s[t] - m);
    __syncthreads();
    const int per = (K + kBlock - 1) / kBlock;
    const int t0 = min(K, tid * per), t1 = min(K, t0 + per);
    double local = 0.0;
    for (int t = t0; t < t1; ++t) local += e_s[t];
    double run = block_exclusive_sum(local, red_s);
    for (int t = t0; t < t1; ++t) {
        run += e_s[t];
        c_s[t] = run;
    }
    __syncthreads();

    const bool full = K > 0 && p.M >= K;
    if (K > 0) {
        const double Z = c_s[K - 1];
        if (full) {
            for (int t = tid; t < K; t += kBlock) atomicOr(&bits_s[t >> 5], 1u << (t & 31));
        } else {
            // 3. M draws with replacement, inverse CDF: first t with u Z < C_t.
            for (int j = tid; j < p.M; j += kBlock) {
                const uint4 r = philox4x32_10(make_uint4(uint32_t(j) >> 2, uint32_t(h), uint32_t(b), p.offset),
                                              p.seed_lo, p.seed_hi);
                const uint32_t x = (j & 3) == 0 ? r.x : (j & 3) == 1 ? r.y : (j & 3) == 2 ? r.z : r.w;
                const double u = (double(x) + 0.5) * 0x1p-32;
                const double target = u * Z;
                int t;
                if (target < c_s[K - 1]) {
                    int lo = 0, hi = K - 1;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (target < c_s[mid]) hi = mid; else lo = mid + 1;
                    }
                    t = lo;
                } else {            // unreachable for u < 1; last team with mass
                    t = K - 1;
                    while (t > 0 && !(e_s[t] > 0.0)) --t;
                }
                atomicOr(&bits_s[t >> 5], 1u << (t & 31));
            }
        }
        __syncthreads();

        // 4. Inclusion probability pi = 1 - (1 - p)^M and log-weight -log(pi).
        if (p.sampled) {
            for (int w = tid; w < p.words; w += kBlock) {
                int s = 0;
                for (int i = 0; i < w; ++i) s += __popc(bits_s[i]);
                wpre_s[w] = s;
            }
            __syncthreads();
        }
        float *lnw = p.lnw + size_t(bh) * p.P;
        for (int t = tid; t < K; t += kBlock) {
            const uint32_t word = bits_s[t >> 5];
            if (!((word >> (t & 31)) & 1u)) continue;
            double lw = 0.0, w = 1.0;
            if (!full) {
                const double pt_ = e_s[t] / Z;
                const double pi = -expm1(double(p.M) * log1p(-pt_));
                w = 1.0 / pi;
                lw = -log(pi);
            }
            lnw[t] = float(lw);
            if (p.sampled) {
                const int rank = wpre_s[t >> 5] + __popc(word & ((1u << (t & 31)) - 1u));
                p.sampled[size_t(bh) * p.M + rank] = t;
                p.inv_pi[size_t(bh) * p.M + rank] = float(w);
            }
        }
    }
    for (int w = tid; w < p.words; w += kBlock) p.bitmaps[size_t(bh) * p.words + w] = bits_s[w];
    if (p.sampled) {
        int total = 0;
        for (int i = 0; i < p.words; ++i) total += __popc(bits_s[i]);
        for (int r = total + tid; r < p.M; r += kBlock) {
            p.sampled[size_t(bh) * p.M + r] = -1;
            p.inv_pi[size_t(bh) * p.M + r] = 0.0f;
        }
    }
}

// ---------------------------------------------------------------------------
// given: team bitmap and log-weights of one (sequence, query head) from a
// caller-supplied list (entries outside [0, K_b) ignored).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void given_kernel(Params p) {
    __shared__ uint32_t bits_s[kMaxWords];
    const int tid = threadIdx.x, bh = blockIdx.x;
    const int b = bh / p.Hq;
    const int L = clamp_len(p.seq_lens[b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    for (int w = tid; w < p.words; w += kBlock) bits_s[w] = 0u;
    __syncthreads();
    for (int j = tid; j < p.M; j += kBlock) {
        const int t = p.given_teams[size_t(bh) * p.M + j];
        if (t < 0 || t >= K) continue;
        atomicOr(&bits_s[t >> 5], 1u << (t & 31));
        p.lnw[size_t(bh) * p.P + t] = logf(p.given_w[size_t(bh) * p.M + j]);
    }
    __syncthreads();
    for (int w = tid; w < p.words; w += kBlock) p.bitmaps[size_t(bh) * p.words + w] = bits_s[w];
}

// ---------------------------------------------------------------------------
// gather: split-K block (split s, KV head g, sequence b) over union teams
// [s * tps, (s + 1) * tps) of the G query heads of g (dense mode: teams
// [s * tps, ...) of the sequence, every head, weight 1).
//
// [EXP] section 三 steps 4-5 and [ABS]: exact attention scores inside the
// sampled teams, each team re-weighted by 1/pi. The weight is folded into
// the logit, s_j + log w_t, so the online softmax carries it on both the
// numerator and the denominator and never overflows.
//
// Lane layout: a cache row (one token, d channels) is LPR lanes x 16 bytes;
// a wavefront covers RPI rows per load; the block's 4 wavefronts cover RPB
// rows; each lane keeps NB row loads of K and of V in flight per batch.
// Each lane runs its own online softmax over its rows; lanes are merged
// across rows, then wavefronts, at the end.
// ---------------------------------------------------------------------------
template <typename KV, int D, int GMAX>
__global__ __launch_bounds__(kBlock) void gather_kernel(Params p) {
    using S = typename KVTraits<KV>::Score;
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    constexpr int LPR = D / VPC;
    constexpr int RPI = 64 / LPR;
    constexpr int RPB = kWaves * RPI;
    constexpr int NB = 8;

    __shared__ S q_s[GMAX][D];
    __shared__ int64_t tpage_s[kMaxTeamsPerSplit];
    __shared__ int32_t tn_s[kMaxTeamsPerSplit];
    __shared__ uint32_t tmask_s[kMaxTeamsPerSplit];
    __shared__ float tlnw_s[kMaxTeamsPerSplit][GMAX];
    __shared__ uint32_t uword_s[kMaxWords];
    __shared__ int32_t upre_s[kMaxWords + 1];
    __shared__ int32_t nteams_s;
    __shared__ S red_m[kWaves][GMAX];
    __shared__ float red_l[kWaves][GMAX];
    __shared__ float red_acc[kWaves][GMAX][D];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = p.G;
    const int L = clamp_len(p.seq_lens[b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    const int hbase = b * p.Hq + g * G;
    const int32_t *pt = p.page_table + size_t(b) * p.P;

    // Team list of this split.
    if (p.mode == kModeDense) {
        if (tid == 0) nteams_s = max(0, min(p.tps, K - s * p.tps));
        if (tid < p.tps) {
            const int t = s * p.tps + tid;
            if (t < K) {
                tpage_s[tid] = clamp_page(pt[t], p.num_pages);
                tn_s[tid] = min(p.T, L - t * p.T);
                tmask_s[tid] = (G >= 32) ? 0xffffffffu : ((1u << G) - 1u);
                for (int h = 0; h < GMAX; ++h) tlnw_s[tid][h] = 0.0f;
            }
        }
    } else {
        for (int w = tid; w < p.words; w += kBlock) {
            uint32_t u = 0u;
            for (int h = 0; h < G; ++h) u |= p.bitmaps[size_t(hbase + h) * p.words + w];
            uword_s[w] = u;
        }
        __syncthreads();
        if (tid == 0) {
            int acc = 0;
            for (int w = 0; w < p.words; ++w) {
                upre_s[w] = acc;
                acc += __popc(uword_s[w]);
            }
            upre_s[p.words] = acc;
            nteams_s = max(0, min(p.tps, acc - s * p.tps));
        }
        __syncthreads();
        if (tid < nteams_s) {
            const int r = s * p.tps + tid;
            int w = 0;
            while (upre_s[w + 1] <= r) ++w;
            uint32_t u = uword_s[w];
            for (int k = r - upre_s[w]; k > 0; --k) u &= u - 1u;
            const int bit = __ffs(u) - 1;
            const int t = w * 32 + bit;
            tpage_s[tid] = clamp_page(pt[t], p.num_pages);
            tn_s[tid] = min(p.T, L - t * p.T);
            uint32_t mask = 0u;
            for (int h = 0; h < G; ++h) {
                const uint32_t hw = p.bitmaps[size_t(hbase + h) * p.words + w];
                if ((hw >> bit) & 1u) {
                    mask |= 1u << h;
                    tlnw_s[tid][h] = p.lnw[size_t(hbase + h) * p.P + t];
                }
            }
            tmask_s[tid] = mask;
        }
    }
    const KV *qg = static_cast<const KV *>(p.q) + size_t(hbase) * D;
    for (int i = tid; i < G * D; i += kBlock) q_s[i / D][i % D] = S(to_f32(qg[i]));
    __syncthreads();
    const int nteams = nteams_s;
    if (nteams == 0) return;

    const int rw = lane / LPR;          // row within the wavefront's load
    const int cc = lane % LPR;          // 16-byte chunk within the row
    S m_[GMAX];
    float l_[GMAX];
    float acc[GMAX][VPC];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        m_[h] = S(-INFINITY);
        l_[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < VPC; ++c) acc[h][c] = 0.0f;
    }
    const S scale = S(p.scale);
    uint32_t block_mask = 0u;

    for (int ti = 0; ti < nteams; ++ti) {
        const int64_t page = tpage_s[ti];
        const int n = tn_s[ti];
        const uint32_t mask = tmask_s[ti];
        block_mask |= mask;
        const size_t tile = (size_t(page) * p.Hkv + g) * p.T * D;
        const KV *kt = static_cast<const KV *>(p.k_pages) + tile;
        const KV *vt = static_cast<const KV *>(p.v_pages) + tile;
        for (int base = 0; base < n; base += RPB * NB) {
            uint4 kr[NB], vr[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int row = base + i * RPB + wave * RPI + rw;
                if (row < n) {
                    kr[i] = ld16(kt + size_t(row) * D + cc * VPC);
                    vr[i] = ld16(vt + size_t(row) * D + cc * VPC);
                } else {
                    kr[i] = make_uint4(0u, 0u, 0u, 0u);
                    vr[i] = make_uint4(0u, 0u, 0u, 0u);
                }
            }
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h >= G || !((mask >> h) & 1u)) continue;     // uniform over the block
                S qv[VPC];
#pragma unroll
                for (int c = 0; c < VPC; ++c) qv[c] = q_s[h][cc * VPC + c];
                const S lw = S(tlnw_s[ti][h]);
                S sc[NB];
                S bmax = S(-INFINITY);
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    float kf[8];
                    unpack(kr[i], kf, KV{});
                    S part = S(0);
#pragma unroll
                    for (int c = 0; c < VPC; ++c) part = fma(S(kf[c]), qv[c], part);
#pragma unroll
                    for (int off = LPR / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
                    const int row = base + i * RPB + wave * RPI + rw;
                    sc[i] = (row < n) ? part * scale + lw : S(-INFINITY);
                    bmax = sc[i] > bmax ? sc[i] : bmax;
                }
                const S mnew = m_[h] > bmax ? m_[h] : bmax;
                const float corr = (m_[h] == S(-INFINITY)) ? 0.0f : float(exp(m_[h] - mnew));
                l_[h] *= corr;
#pragma unroll
                for (int c = 0; c < VPC; ++c) acc[h][c] *= corr;
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    const float pe = (sc[i] == S(-INFINITY)) ? 0.0f : float(exp(sc[i] - mnew));
                    float vf[8];
                    unpack(vr[i], vf, KV{});
                    l_[h] += pe;
#pragma unroll
                    for (int c = 0; c < VPC; ++c) acc[h][c] = fmaf(pe, vf[c], acc[h][c]);
                }
                m_[h] = mnew;
            }
        }
    }

    // Merge the RPI row groups of each wavefront (lanes LPR apart).
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= G || !((block_mask >> h) & 1u)) continue;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
            const S mo = __shfl_xor(m_[h], off, 64);
            const float lo = __shfl_xor(l_[h], off, 64);
            const S mn = m_[h] > mo ? m_[h] : mo;
            const float ca = (m_[h] == S(-INFINITY)) ? 0.0f : float(exp(m_[h] - mn));
            const float cb = (mo == S(-INFINITY)) ? 0.0f : float(exp(mo - mn));
            l_[h] = l_[h] * ca + lo * cb;
#pragma unroll
            for (int c = 0; c < VPC; ++c) {
                const float ao = __shfl_xor(acc[h][c], off, 64);
                acc[h][c] = acc[h][c] * ca + ao * cb;
            }
            m_[h] = mn;
        }
        if (rw == 0) {
#pragma unroll
            for (int c = 0; c < VPC; ++c) red_acc[wave][h][cc * VPC + c] = acc[h][c];
            if (cc == 0) {
                red_m[wave][h] = m_[h];
                red_l[wave][h] = l_[h];
            }
        }
    }
    __syncthreads();

    // Merge the wavefronts in a fixed order and write this split's partials.
    float2 *part_ml = reinterpret_cast<float2 *>(p.part_ml);
    for (int i = tid; i < G * D; i += kBlock) {
        const int h = i / D, c = i % D;
        const size_t slot = size_t(hbase + h) * p.P + s;
        if (!((block_mask >> h) & 1u)) {
            if (c == 0) part_ml[slot] = make_float2(kNegInfF, 0.0f);
            continue;
        }
        S mx = red_m[0][h];
        for (int w = 1; w < kWaves; ++w) mx = red_m[w][h] > mx ? red_m[w][h] : mx;
        const float mstore = float(mx);
        float l = 0.0f, a = 0.0f;
        for (int w = 0; w < kWaves; ++w) {
            if (red_m[w][h] == S(-INFINITY)) continue;
            const float f = float(exp(red_m[w][h] - S(mstore)));
            l += f * red_l[w][h];
            a += f * red_acc[w][h][c];
        }
        p.part_acc[slot * D + c] = a;
        if (c == 0) part_ml[slot] = make_float2(mstore, l);
    }
}

// ---------------------------------------------------------------------------
// combine: one block per (sequence, query head), one thread per channel.
// Merges the split partials in split order: out = sum_s e^{m_s - m*} acc_s /
// sum_s e^{m_s - m*} l_s, lse = m* + log(sum_s e^{m_s - m*} l_s).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(Params p) {
    __shared__ int u_s;
    const int bh = blockIdx.x, c = threadIdx.x;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const int L = clamp_len(p.seq_lens[b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    int U = K;
    if (p.mode != kModeDense) {
        if (c == 0) u_s = 0;
        __syncthreads();
        const int hbase = b * p.Hq + g * p.G;
        int cnt = 0;
        for (int w = c; w < p.words; w += D) {
            uint32_t u = 0u;
            for (int k = 0; k < p.G; ++k) u |= p.bitmaps[size_t(hbase + k) * p.words + w];
            cnt += __popc(u);
        }
        atomicAdd(&u_s, cnt);
        __syncthreads();
        U = u_s;
    }
    const int nsplit = (U + p.tps - 1) / p.tps;
    const float2 *ml = reinterpret_cast<const float2 *>(p.part_ml) + size_t(bh) * p.P;
    float mstar = kNegInfF;
    for (int s = 0; s < nsplit; ++s) mstar = fmaxf(mstar, ml[s].x);
    float l = 0.0f, a = 0.0f;
    if (mstar > kNegInfF) {
        for (int s = 0; s < nsplit; ++s) {
            const float2 v = ml[s];
            if (!(v.x > kNegInfF)) continue;
            const float f = expf(v.x - mstar);
            l += f * v.y;
            a += f * p.part_acc[(size_t(bh) * p.P + s) * D + c];
        }
    }
    p.out[size_t(bh) * D + c] = (l > 0.0f) ? a / l : 0.0f;
    if (c == 0 && p.lse) p.lse[bh] = (l > 0.0f) ? mstar + logf(l) : kNegInfF;
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
santa_status launched() {
    return hipGetLastError() == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

template <typename KV, int D>
santa_status gather_dispatch_g(const Params &p, hipStream_t st) {
    const dim3 grid(p.max_splits, p.Hkv, p.B);
    if (p.G <= 1) hipLaunchKernelGGL((gather_kernel<KV, D, 1>), grid, dim3(kBlock), 0, st, p);
    else if (p.G <= 2) hipLaunchKernelGGL((gather_kernel<KV, D, 2>), grid, dim3(kBlock), 0, st, p);
    else if (p.G <= 4) hipLaunchKernelGGL((gather_kernel<KV, D, 4>), grid, dim3(kBlock), 0, st, p);
    else if (p.G <= 8) hipLaunchKernelGGL((gather_kernel<KV, D, 8>), grid, dim3(kBlock), 0, st, p);
    else hipLaunchKernelGGL((gather_kernel<KV, D, 16>), grid, dim3(kBlock), 0, st, p);
    return launched();
}

}  // namespace

template <template <typename, int> class F>
santa_status dispatch_kv_d(const Params &p, hipStream_t st) {
    if (p.dtype == SANTA_BF16) return p.d == 64 ? F<bf16_t, 64>::run(p, st) : F<bf16_t, 128>::run(p, st);
    return p.d == 64 ? F<float, 64>::run(p, st) : F<float, 128>::run(p, st);
}

template <typename KV, int D> struct BuildRepsLaunch {
    static santa_status run(const Params &p, hipStream_t st) {
        hipLaunchKernelGGL((build_reps_kernel<KV, D>), dim3(p.P, p.Hkv, p.B), dim3(64), 0, st, p);
        return launched();
    }
};
template <typename KV, int D> struct SelectLaunch {
    static santa_status run(const Params &p, hipStream_t st) {
        hipLaunchKernelGGL((select_kernel<KV, D>), dim3(p.B * p.Hq), dim3(kBlock), 0, st, p);
        return launched();
    }
};
template <typename KV, int D> struct GatherLaunch {
    static santa_status run(const Params &p, hipStream_t st) { return gather_dispatch_g<KV, D>(p, st); }
};

santa_status launch_build_reps(const Params &p, void *stream) {
    return dispatch_kv_d<BuildRepsLaunch>(p, static_cast<hipStream_t>(stream));
}

santa_status launch_select(const Params &p, void *stream) {
    return dispatch_kv_d<SelectLaunch>(p, static_cast<hipStream_t>(stream));
}

santa_status launch_given(const Params &p, void *stream) {
    hipLaunchKernelGGL(given_kernel, dim3(p.B * p.Hq), dim3(kBlock), 0, static_cast<hipStream_t>(stream), p);
    return launched();
}

santa_status launch_gather(const Params &p, void *stream) {
    return dispatch_kv_d<GatherLaunch>(p, static_cast<hipStream_t>(stream));
}

santa_status launch_combine(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.d == 64) hipLaunchKernelGGL((combine_kernel<64>), dim3(p.B * p.Hq), dim3(64), 0, st, p);
    else hipLaunchKernelGGL((combine_kernel<128>), dim3(p.B * p.Hq), dim3(128), 0, st, p);
    return launched();
}

}  // namespace santa
