// Team selection of SANTA++ (gfx950): representative scores, team softmax,
// Philox inverse-CDF draws, dedupe and inclusion probabilities.
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract: the query scores one representative
//         from each team to decide which teams to sample; each sampled team
//         is re-weighted by the inverse of its inclusion probability.
//   [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
//         section 三 steps 2-3: s_i = Q . rep_i, p = softmax(s_1..s_K),
//         sample M teams with probability p_i.
//   [PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
//         1, 2, 3", SC'11 (Philox4x32-10).
//
// Selection is decided in float64: products of two bfloat16 (or float32)
// values are exact in float64 and the sums are accurate to ~1e-16, so a draw
// can land on a different team than an exact computation only when its
// uniform lies within ~1e-15 of a cumulative-probability boundary.
#include "device_common.h"

namespace santa {
namespace {

using namespace dev;

// One 256-thread block per (sequence b, query head h). Writes the head's team
// bitmap and, for every drawn team t, log w_t = -log(pi_t) (0 under full
// coverage), plus the optional sorted team list and 1/pi.
template <typename KV, int D>
__global__ __launch_bounds__(kBlock) void select_kernel(Params p) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    constexpr int CH = D / VPC;                    // 16-byte chunks per representative row
    __shared__ double q_s[D];
    __shared__ double e_s[kMaxTeams];              // scores, then exp(s - max)
    __shared__ double c_s[kMaxTeams];              // inclusive cumulative sums of e
    __shared__ uint32_t bits_s[kMaxWords];
    __shared__ int32_t wpre_s[kMaxWords];
    __shared__ double red_s[kWaves];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const KV *reps = static_cast<const KV *>(p.reps) + size_t(b) * p.P * p.Hkv * D;

    // Round trip 1: sequence length, query, and (speculatively, every row is
    // in bounds) the first representative row of this thread.
    const int Lraw = p.seq_lens[b];
    const KV *q = static_cast<const KV *>(p.q) + size_t(bh) * D;
    for (int c = tid; c < D; c += kBlock) q_s[c] = double(to_f32(q[c]));
    for (int w = tid; w < p.words; w += kBlock) bits_s[w] = 0u;
    uint4 raw[CH];
    {
        const KV *r = reps + (size_t(tid < p.P ? tid : 0) * p.Hkv + g) * D;
#pragma unroll
        for (int j = 0; j < CH; ++j) raw[j] = ld16(r + j * VPC);
    }
    const int L = clamp_len(Lraw, p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    __syncthreads();

    // 1. Representative scores s_t = q . rep_t / sqrt(d) in float64 (the
    //    representatives are indexed by logical team: no page-table lookup).
    //    Four partial sums keep the float64 FMA chains short.
    for (int t = tid; t < K; t += kBlock) {
        if (t != tid) {
            const KV *r = reps + (size_t(t) * p.Hkv + g) * D;
#pragma unroll
            for (int j = 0; j < CH; ++j) raw[j] = ld16(r + j * VPC);
        }
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            float f[8];
            unpack(raw[j], f, KV{});
#pragma unroll
            for (int e = 0; e < VPC; ++e) acc[e & 3] = fma(double(f[e]), q_s[j * VPC + e], acc[e & 3]);
        }
        e_s[t] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * p.scale;
    }
    __syncthreads();

    // 2. Team softmax numerators e_t = exp(s_t - max s) and cumulative sums.
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
            // 3. M draws with replacement: u = (x + 1/2) 2^-32 from Philox word
            //    j mod 4 of counter (j / 4, h, b, offset); team = first t with
            //    u Z < C_t.
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
                } else {            // unreachable for u < 1: last team with mass
                    t = K - 1;
                    while (t > 0 && !(e_s[t] > 0.0)) --t;
                }
                atomicOr(&bits_s[t >> 5], 1u << (t & 31));
            }
        }
        __syncthreads();

        // 4. pi_t = 1 - (1 - p_t)^M, written -expm1(M log1p(-p_t)); log w_t = -log pi_t.
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

// Team bitmap and log-weights of one (sequence, query head) from a
// caller-supplied list; entries outside [0, K_b) are ignored.
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

}  // namespace

santa_status launch_select(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(p.B * p.Hq);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) hipLaunchKernelGGL((select_kernel<bf16_t, 64>), grid, dim3(kBlock), 0, st, p);
        else hipLaunchKernelGGL((select_kernel<bf16_t, 128>), grid, dim3(kBlock), 0, st, p);
    } else {
        if (p.d == 64) hipLaunchKernelGGL((select_kernel<float, 64>), grid, dim3(kBlock), 0, st, p);
        else hipLaunchKernelGGL((select_kernel<float, 128>), grid, dim3(kBlock), 0, st, p);
    }
    return launched();
}

santa_status launch_given(const Params &p, void *stream) {
    hipLaunchKernelGGL(given_kernel, dim3(p.B * p.Hq), dim3(kBlock), 0, static_cast<hipStream_t>(stream), p);
    return launched();
}

}  // namespace santa
