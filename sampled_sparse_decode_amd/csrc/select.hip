// Standalone team selection (gfx950): representative scores, team softmax,
// Philox inverse-CDF draws, dedupe and inclusion probabilities for every
// (sequence, query head), written to the workspace for santa_attend_selected.
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract (team scores decide the draws; drawn
//         teams are weighted by 1/pi).
//   [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
//         section 三 steps 2-3.
//
// The arithmetic is that of selection.h, which the fused decode kernel runs
// too, so select + attend and one decode call give the same bits.
#include "selection.h"

namespace santa {
namespace {

using namespace dev;

constexpr int kSelThreads = 512;                    // 8 wavefronts score; wavefront 0 runs the tail
constexpr int kRowsPerPass = kSelThreads / sel::kParts;
constexpr int kUpfrontPasses = 4;                   // page tables up to 512 rows: every pass requested at once

// One block per (sequence b, query head h). Writes the head's team bitmap,
// log w_t of every drawn team, and the optional sorted list with 1/pi.
// Blocks are placed by XCD (block i runs on XCD i mod 8; the grid is 8 n8
// with n8 a whole number of groups' heads, and XCD x takes heads
// [x n8, (x + 1) n8)), so the G heads of a group, which read the same
// representative rows, share one L2.
template <typename KV, int D, bool UPFRONT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
    using Pt = sel::Part<KV, D>;
    __shared__ double q_s[D];
    __shared__ double s_s[kMaxTeams];
    __shared__ double c_s[kMaxTeams];
    __shared__ double pts_s[kMaxTeams];
    __shared__ uint32_t bits_s[kMaxWords];
    __shared__ int32_t pre_s[kMaxWords + 1];
    __shared__ float wmax_s[kSelThreads / 64];

    const int tid = threadIdx.x;
    const int bh = int(blockIdx.x & 7) * int(gridDim.x >> 3) + int(blockIdx.x >> 3);
    if (bh >= p.B * p.Hq) return;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const KV *reps = static_cast<const KV *>(p.reps) + size_t(b) * p.P * p.Hkv * D;
    const int row0 = tid / sel::kParts, part = tid % sel::kParts;

    // Round trip 1: length, query and the rows of the first passes (every
    // row index below P is inside the buffer, so they are loaded
    // speculatively; with P <= 512 every pass is requested here).
    const int Lraw = p.seq_lens[b];
    const KV *q = static_cast<const KV *>(p.q) + size_t(bh) * D;
    float qv = 0.0f;
    if (tid < D) qv = to_f32(q[tid]);
    uint4 up[UPFRONT ? kUpfrontPasses : 1][Pt::LOADS];
    uint4 raw[Pt::LOADS];
    if constexpr (UPFRONT) {
#pragma unroll
        for (int ps = 0; ps < kUpfrontPasses; ++ps) {
            const int row = row0 + ps * kRowsPerPass;
            if (row < p.P) sel::load_part<KV, D>(reps + (size_t(row) * p.Hkv + g) * D, part, up[ps]);
        }
    } else {
        sel::load_part<KV, D>(reps + (size_t(row0 < p.P ? row0 : 0) * p.Hkv + g) * D, part, raw);
    }
    // Draw points while the rows are in flight (needed when M < K <= P).
    sel::TailArgs a{0, p.M, p.scheme, p.seed_lo, p.seed_hi, p.offset, h, b};
    if (p.M < p.P) sel::draw_points(a, pts_s, tid, kSelThreads);
    if (tid < D) q_s[tid] = double(qv);
    const int L = clamp_len(Lraw, p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    __syncthreads();
    double qp[Pt::N];                                    // this thread's part of the query, every pass
#pragma unroll
    for (int i = 0; i < Pt::N; ++i) qp[i] = q_s[part * Pt::N + i];

    float mx = -INFINITY;                                // largest float32-rounded score of the thread's rows
    if constexpr (UPFRONT) {
#pragma unroll
        for (int ps = 0; ps < kUpfrontPasses; ++ps) {
            if (ps * kRowsPerPass >= K) break;                  // uniform
            const int t = row0 + ps * kRowsPerPass;
            const double sc = sel::row_score(sel::part_dot_raw<KV, D>(up[ps], qp), p.scale);
            if (part == 0 && t < K) {
                s_s[t] = sc;
                mx = fmaxf(mx, float(sc));
            }
        }
    }
    // Scores, one pass of kRowsPerPass rows at a time; the next pass's rows
    // are requested before this pass is scored.
    const int tEnd = UPFRONT ? 0 : ((K + kRowsPerPass - 1) / kRowsPerPass) * kRowsPerPass;
    for (int t = row0; t < tEnd; t += kRowsPerPass) {
        uint4 nxt[Pt::LOADS];
        const bool more = t + kRowsPerPass < tEnd;
        if (more) {
            const int tn = t + kRowsPerPass;
            sel::load_part<KV, D>(reps + (size_t(tn < K ? tn : 0) * p.Hkv + g) * D, part, nxt);
        }
        const double sc = sel::row_score(sel::part_dot_raw<KV, D>(raw, qp), p.scale);
        if (part == 0 && t < K) {
            s_s[t] = sc;
            mx = fmaxf(mx, float(sc));
        }
        if (more) {
#pragma unroll
            for (int j = 0; j < Pt::LOADS; ++j) raw[j] = nxt[j];
        }
    }
    mx = sel::wave_max(mx);
    if ((tid & 63) == 0) wmax_s[tid >> 6] = mx;
    __syncthreads();
    sel::team_exps(s_s, K, wmax_s, kSelThreads / 64, tid, kSelThreads);
    __syncthreads();
    if (tid >= 64) return;

    a.K = K;
    int32_t *sampled = p.sampled ? p.sampled + size_t(bh) * p.M : nullptr;
    float *inv_pi = p.sampled ? p.inv_pi + size_t(bh) * p.M : nullptr;
    const double Z = sel::head_tail(s_s, c_s, bits_s, pts_s, a);
    sel::drawn_weights(s_s, c_s, bits_s, Z, a, pre_s, p.lnw + size_t(bh) * p.P, sampled, inv_pi);
    __builtin_amdgcn_wave_barrier();
    for (int w = tid; w < p.words; w += 64)
        p.bitmaps[size_t(bh) * p.words + w] = w < (K + 31) / 32 ? bits_s[w] : 0u;
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
    const int64_t groups = int64_t(p.B) * p.Hkv;
    const dim3 grid(unsigned(8 * ((groups + 7) / 8) * p.G)), block(kSelThreads);
    const bool up = p.dtype == SANTA_BF16 && p.P <= kUpfrontPasses * kRowsPerPass;   // float32 rows would spill
#define SANTA_SELECT_LAUNCH(KV, DD)                                                                            \
    if (up) hipLaunchKernelGGL((select_kernel<KV, DD, true>), grid, block, 0, st, p);                          \
    else hipLaunchKernelGGL((select_kernel<KV, DD, false>), grid, block, 0, st, p);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) { SANTA_SELECT_LAUNCH(bf16_t, 64) } else { SANTA_SELECT_LAUNCH(bf16_t, 128) }
    } else {
        if (p.d == 64) hipLaunchKernelGGL((select_kernel<float, 64, false>), grid, block, 0, st, p);
        else hipLaunchKernelGGL((select_kernel<float, 128, false>), grid, block, 0, st, p);
    }
#undef SANTA_SELECT_LAUNCH
    return launched();
}

santa_status launch_given(const Params &p, void *stream) {
    hipLaunchKernelGGL(given_kernel, dim3(p.B * p.Hq), dim3(kBlock), 0, static_cast<hipStream_t>(stream), p);
    return launched();
}

}  // namespace santa
