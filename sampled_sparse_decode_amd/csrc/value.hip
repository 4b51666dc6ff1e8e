// SANTA++ team draws followed by value samples inside the drawn teams
// (gfx950).
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract: the teams to read are drawn from the
//         team scores and a drawn team's terms count 1/pi times.
//   [SAN] "Stochastic Sparse Attention for Memory-Bound Inference" (the
//         SANTA page), abstract: drawing token indices from the post-softmax
//         weights and averaging only those value rows estimates the weighted
//         value sum without bias; stratified and systematic points lower the
//         variance.
//
// After the selection kernel (bitmaps and log weights in the workspace), one
// 512-thread block per (sequence, query head) does the rest:
//   1. the drawn teams in ascending order (rank r), and n, the number of
//      their tokens: every team holds T tokens except the sequence's last,
//      which, when drawn, has the highest rank, so drawn token g is token
//      g mod T of the rank-(g / T) team;
//   2. the weighted logit l_g = s_g + log w of every drawn token in float64
//      (selection.h's score arithmetic: bf16 or fp32 products are exact in
//      float64), 128 tokens per pass with four passes of rows in flight,
//      kept in LDS;
//   3. e_g = exp(l_g - max l), and the cumulative sums C in a fixed order
//      (thread ranges in token order, a DPP scan over the wavefront, the
//      wavefront totals added in wavefront order); lse = max l + log C_last;
//   4. S points from the value stream (Philox4x32-10 word k mod 4 of counter
//      (k / 4, h, b, offset), key (seed lo ^ kValueKeyXor, seed hi)), each
//      taking the first token g with point * C_last < C_g;
//   5. out = (1 / S) sum over the samples of the sampled tokens' values,
//      summed per channel in a fixed order.
// The K tiles of the drawn teams are read once per head (the heads of a group
// share them through their XCD's L2: blocks are placed by XCD as in the
// selection kernel); of the V tiles only the lines the samples touch.
#include "selection.h"

namespace santa {
namespace {

using namespace dev;

constexpr int kVsThreads = 512;
constexpr int kVsWaves = kVsThreads / 64;
constexpr int kVsTokensPerPass = kVsThreads / sel::kParts;     // 128
constexpr int kVsDepth = 4;                                     // passes of rows in flight
constexpr int kVsMaxTeamsDrawn = kVsMaxTokens / 16;             // T >= 16
constexpr uint32_t kValueKeyXor = 0x56414C55u;

struct VsLds {
    double l[kVsMaxTokens];             // logits, then exponentials, then cumulative sums
    double q64[128];
    double wred[kVsWaves];              // per-wavefront maxima, then totals
    int32_t page[kVsMaxTeamsDrawn];     // page of the rank-r drawn team
    int32_t team[kVsMaxTeamsDrawn];
    float lnw[kVsMaxTeamsDrawn];
    uint32_t bits[kMaxWords];
    int32_t spre[kMaxWords + 1];
    int32_t pick[kVsMaxSamples];        // drawn-token index of sample k
    float acc[kVsThreads / 64][128];    // per (sample subset, channel) sums
};

// Point k of the value stream (scheme as for the team draws).
__device__ __forceinline__ double value_point(const Params &p, int k, int h, int b) {
    const uint32_t k0 = p.seed_lo ^ kValueKeyXor;
    auto word = [&](int j) {
        const uint4 r = philox4x32_10(make_uint4(uint32_t(j) >> 2, uint32_t(h), uint32_t(b), p.offset), k0, p.seed_hi);
        return (j & 3) == 0 ? r.x : (j & 3) == 1 ? r.y : (j & 3) == 2 ? r.z : r.w;
    };
    const int S = p.vs_samples;
    if (p.vs_scheme == SANTA_DRAW_SYSTEMATIC) return (double(k) + (double(word(0)) + 0.5) * 0x1p-32) / double(S);
    const double u = (double(word(k)) + 0.5) * 0x1p-32;
    if (p.vs_scheme == SANTA_DRAW_STRATIFIED) return (double(k) + u) / double(S);
    return u;
}

__device__ __forceinline__ double wave_max_d(double x) {
    for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
    return x;
}

template <typename KV, int D>
__global__ __launch_bounds__(kVsThreads, 1) void value_sample_kernel(Params p) {
    using Pt = sel::Part<KV, D>;
    constexpr int NSUB = kVsThreads / D;                 // sample subsets in the value sums
    __shared__ VsLds lds;

    const int bh = int(blockIdx.x & 7) * int(gridDim.x >> 3) + int(blockIdx.x >> 3);
    if (bh >= p.B * p.Hq) return;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = p.T, S = p.vs_samples;

    // Round trip 1: length, query, the head's bitmap words.
    const int Lraw = p.seq_lens[b];
    const KV *qg = static_cast<const KV *>(p.q) + size_t(bh) * D;
    if (tid < D) lds.q64[tid] = double(to_f32(qg[tid]));
    if (tid < p.words) lds.bits[tid] = p.bitmaps[size_t(bh) * p.words + tid];
    const int L = clamp_len(Lraw, p.P * T);
    const int K = (L + T - 1) / T;
    __syncthreads();
    if (K == 0) {                                        // empty sequence (uniform)
        if (tid < D) p.out[size_t(bh) * D + tid] = 0.0f;
        if (tid == 0 && p.lse) p.lse[bh] = kNegInfF;
        if (p.vs_positions)
            for (int k = tid; k < S; k += kVsThreads) p.vs_positions[size_t(bh) * S + k] = -1;
        return;
    }
    const int words = (K + 31) >> 5;
    if (wave == 0) {
        const int cnt = lane < words ? __popc(lds.bits[lane]) : 0;
        const int ic = sel::wave_incl_scan(cnt);
        if (lane < words) lds.spre[lane] = ic - cnt;
        if (lane == 63) lds.spre[words] = ic;
    }
    __syncthreads();
    const int nd = lds.spre[words];                      // drawn teams (>= 1: at least one draw)
    for (int r = tid; r < nd; r += kVsThreads) {
        int lo = 0, hi = words - 1;                      // last word whose prefix is <= r
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (lds.spre[mid] <= r) lo = mid; else hi = mid - 1;
        }
        uint32_t u = lds.bits[lo];
        for (int k = r - lds.spre[lo]; k > 0; --k) u &= u - 1u;
        const int t = lo * 32 + __ffs(u) - 1;
        lds.team[r] = t;
        lds.page[r] = int32_t(clamp_page(p.page_table[size_t(b) * p.P + t], p.num_pages));
        lds.lnw[r] = p.lnw[size_t(bh) * p.P + t];
    }
    __syncthreads();
    const int n = nd * T - (lds.team[nd - 1] == K - 1 ? K * T - L : 0);

    // 2. Weighted logits of the drawn tokens, four passes of rows in flight.
    const int part = tid % sel::kParts;
    double qp[Pt::N];
#pragma unroll
    for (int i = 0; i < Pt::N; ++i) qp[i] = lds.q64[part * Pt::N + i];
    const KV *kbase = static_cast<const KV *>(p.k_pages);
    const int npass = (n + kVsTokensPerPass - 1) / kVsTokensPerPass;
    auto load_pass = [&](int pass, uint4 (&raw)[Pt::LOADS]) {
        int gt = pass * kVsTokensPerPass + tid / sel::kParts;
        if (gt >= n) gt = 0;                             // in bounds; the score is dropped
        const int r = gt / T, j = gt - r * T;
        const KV *row = kbase + (size_t(lds.page[r]) * p.Hkv + g) * size_t(T) * D +
                        k_offset(j, part * Pt::N, T, D);
#pragma unroll
        for (int x = 0; x < Pt::LOADS; ++x) raw[x] = ld16_stream(row + x * Pt::VPC);
    };
    uint4 buf[kVsDepth][Pt::LOADS];
#pragma unroll
    for (int d = 0; d < kVsDepth; ++d)
        if (d < npass) load_pass(d, buf[d]);
    double mx = -INFINITY;
    for (int p0 = 0; p0 < npass; p0 += kVsDepth) {
#pragma unroll
        for (int d = 0; d < kVsDepth; ++d) {
            const int pass = p0 + d;
            if (pass >= npass) break;                    // uniform
            const double sc = sel::row_score(sel::part_dot_raw<KV, D>(buf[d], qp), p.scale);
            const int gt = pass * kVsTokensPerPass + tid / sel::kParts;
            if (pass + kVsDepth < npass) load_pass(pass + kVsDepth, buf[d]);
            if (part == 0 && gt < n) {
                const double l = sc + double(lds.lnw[gt / T]);
                lds.l[gt] = l;
                mx = fmax(mx, l);
            }
        }
    }
    mx = wave_max_d(mx);
    if (lane == 0) lds.wred[wave] = mx;
    __syncthreads();
    double m = lds.wred[0];
    for (int w = 1; w < kVsWaves; ++w) m = fmax(m, lds.wred[w]);
    __syncthreads();                                     // wred is reused below

    // 3. Exponentials and cumulative sums in a fixed order.
    const int per = (n + kVsThreads - 1) / kVsThreads;
    const int t0 = min(n, tid * per), t1 = min(n, t0 + per);
    double local = 0.0;
    for (int j = t0; j < t1; ++j) {
        const double e = exp(lds.l[j] - m);
        lds.l[j] = e;
        local += e;
    }
    const double incl = sel::wave_incl_scan(local);
    if (lane == 63) lds.wred[wave] = incl;
    __syncthreads();
    double base = 0.0, Z = 0.0;
    for (int w = 0; w < kVsWaves; ++w) {
        if (w < wave) base += lds.wred[w];
        Z += lds.wred[w];
    }
    double run = base + (incl - local);
    for (int j = t0; j < t1; ++j) {
        run += lds.l[j];
        lds.l[j] = run;
    }
    __syncthreads();
    Z = lds.l[n - 1];                                    // C_last as stored (every thread reads the same)

    // 4. Samples: the first drawn token g with point * Z < C_g.
    for (int k = tid; k < S; k += kVsThreads) {
        const double target = value_point(p, k, h, b) * Z;
        int j;
        if (target < Z) {
            int lo = 0, hi = n - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (target < lds.l[mid]) hi = mid; else lo = mid + 1;
            }
            j = lo;
        } else {                                         // not reachable for points below 1
            j = n - 1;
            while (j > 0 && !(lds.l[j] > lds.l[j - 1])) --j;
        }
        lds.pick[k] = j;
        if (p.vs_positions) p.vs_positions[size_t(bh) * S + k] = lds.team[j / T] * T + (j % T);
    }
    __syncthreads();

    // 5. Values: thread (subset, channel) sums the samples k = subset,
    // subset + NSUB, ... in order; the subsets are then added in order.
    const KV *vbase = static_cast<const KV *>(p.v_pages);
    const int ch = tid % D, sub = tid / D;
    float a = 0.0f;
    for (int k0 = sub; k0 < S; k0 += 8 * NSUB) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {                    // every load of the batch first
            const int k = k0 + u * NSUB;
            x[u] = 0.0f;
            if (k < S) {
                const int j = lds.pick[k];
                const int r = j / T, jj = j - r * T;
                const KV *tile = vbase + (size_t(lds.page[r]) * p.Hkv + g) * size_t(T) * D;
                x[u] = to_f32(tile[v_offset(jj, ch, T, D)]);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) a += x[u];
    }
    lds.acc[sub][ch] = a;
    __syncthreads();
    if (tid < D) {
        float s = 0.0f;
        for (int u = 0; u < NSUB; ++u) s += lds.acc[u][tid];
        p.out[size_t(bh) * D + tid] = s / float(S);
    }
    if (tid == 0 && p.lse) p.lse[bh] = float(m + log(Z));
}

}  // namespace

santa_status launch_value_sample(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t groups = int64_t(p.B) * p.Hkv;
    const dim3 grid(unsigned(8 * ((groups + 7) / 8) * p.G)), block(kVsThreads);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) hipLaunchKernelGGL((value_sample_kernel<bf16_t, 64>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((value_sample_kernel<bf16_t, 128>), grid, block, 0, st, p);
    } else {
        if (p.d == 64) hipLaunchKernelGGL((value_sample_kernel<float, 64>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((value_sample_kernel<float, 128>), grid, block, 0, st, p);
    }
    return launched();
}

}  // namespace santa
