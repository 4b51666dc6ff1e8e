// SANTA++ team draws followed by value samples inside the drawn teams
// (gfx950).
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract: the teams to read are drawn from the
//         team scores and a drawn team's terms count 1/pi times.
//   [SAN] "Stochastic Sparse Attention for Memory-Bound Inference" (the
//         SANTA page), abstract: positions picked with probability equal to
//         their attention weight, then the mean of their values, stand in for
//         the attention output without bias; evenly spread (stratified or
//         systematic) picks reduce the variance.
//
// After the selection kernel (bitmaps and log weights in the workspace), the
// drawn tokens of a head, in team order then token order (drawn token g is
// token g mod T of the rank-(g / T) drawn team: every team holds T tokens
// except the sequence's last, which, when drawn, has the highest rank), are
// cut into chunks of kVsChunk tokens and two launches finish the call:
//   logits  one 512-thread block per (head, chunk): the weighted logits
//           l_g = s_g + log w in float64 (selection.h's score arithmetic:
//           bf16 or fp32 products are exact in float64), the chunk's max m_c,
//           e_g = exp(l_g - m_c) and their running sums cs_g inside the chunk
//           (a DPP scan per wavefront, the wavefront totals added in order),
//           written with the pair (m_c, chunk total) to the workspace; the
//           key rows of all four 128-token passes are in flight at once;
//   samples one 512-thread block per head: m = max m_c, the chunk totals
//           rescaled by exp(m_c - m) and scanned in chunk order (C at the
//           chunk ends), Z the last; S points from the value stream
//           (Philox4x32-10 word k mod 4 of counter (k / 4, h, b, offset), key
//           (seed lo ^ kValueKeyXor, seed hi)); point k takes the first token
//           g with point * Z < C_(end of previous chunk) + cs_g exp(m_c - m),
//           found by chunk, then by 16-token piece (its last running sum),
//           then by token; out = (1 / S) sum over the distinct sampled
//           tokens of (times sampled) x value, summed per channel in a fixed
//           order (each sampled value line is read once); lse = m + log Z.
// These running sums are the flat token-order sums up to the rounding of the
// two-level sum: a sample they move has its point within a rounding of a
// token boundary. A group's logit blocks run on one XCD (on 8 / groups XCDs
// when there are fewer than 8 groups, so that every XCD works), where its
// heads share the key tiles; the sample blocks are placed by XCD as in the
// selection kernel, so a head's running sums are read from the L2 that holds
// them. Each block's first round trip also fetches the sequence's page-table
// row (and, for the logits, the head's log weights), so no load waits on
// another one before the key rows.
#include "selection.h"

namespace santa {
namespace {

using namespace dev;

constexpr int kVsThreads = 512;
constexpr int kVsWaves = kVsThreads / 64;
constexpr int kVsTokensPerPass = kVsThreads / sel::kParts;     // 128
constexpr int kVsPasses = kVsChunk / kVsTokensPerPass;          // 4, all in flight
constexpr int kVsPiece = 16;                                    // tokens per search piece
constexpr int kVsPieces = kVsChunk / kVsPiece;                  // 32
constexpr int kVsBatch = 32;                                    // value loads in flight per thread
constexpr uint32_t kValueKeyXor = 0x56414C55u;
static_assert(kVsChunk % 256 == 0 && kVsPasses * kVsTokensPerPass == kVsChunk, "chunk shape");
static_assert(kVsMaxChunks <= 64, "chunk totals are scanned by one wavefront");

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

// A head's drawn-team bitmap in LDS and its word prefix counts.
struct HeadTeams {
    uint32_t bits[kMaxWords];
    int32_t spre[kMaxWords + 1];    // drawn teams before word w; spre[words] = all drawn
};

// Wavefront 0 fills ht.spre for the first `words` words (words <= 64).
__device__ __forceinline__ void team_prefix(HeadTeams &ht, int words) {
    const int lane = threadIdx.x & 63;
    const int cnt = lane < words ? __popc(ht.bits[lane]) : 0;
    const int ic = sel::wave_incl_scan(cnt);
    if (lane < words) ht.spre[lane] = ic - cnt;
    if (lane == 63) ht.spre[words] = ic;
}

// Team index of the rank-r drawn team (r < drawn).
__device__ __forceinline__ int team_of_rank(const HeadTeams &ht, int words, int r) {
    int lo = 0, hi = words - 1;                          // last word whose prefix is <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ht.spre[mid] <= r) lo = mid; else hi = mid - 1;
    }
    uint32_t u = ht.bits[lo];
    for (int k = r - ht.spre[lo]; k > 0; --k) u &= u - 1u;
    return lo * 32 + __ffs(u) - 1;
}

// Drawn tokens of a head: every drawn team's T, less the missing tail of the
// sequence's last team when that team is drawn.
__device__ __forceinline__ int drawn_tokens(const HeadTeams &ht, int words, int K, int L, int T) {
    const int nd = ht.spre[words];
    const bool last = (ht.bits[(K - 1) >> 5] >> ((K - 1) & 31)) & 1u;
    return nd * T - (last ? K * T - L : 0);
}

// Waves per SIMD the logit kernel is built for: two 512-thread blocks per CU,
// except for float32 rows of 128 channels, whose four passes in flight need
// 128 registers of their own.
template <typename KV, int D>
constexpr int vs_logit_waves() { return sizeof(KV) == 4 && D == 128 ? 2 : 4; }

template <typename KV, int D>
__global__ __launch_bounds__(kVsThreads, (vs_logit_waves<KV, D>())) void vs_logits_kernel(Params p) {
    using Pt = sel::Part<KV, D>;
    __shared__ HeadTeams ht;
    __shared__ float q_s[D];
    __shared__ double e_s[kVsChunk];
    __shared__ double wred[kVsWaves];
    __shared__ int32_t pt_s[kMaxTeams];                  // the sequence's page-table row
    __shared__ float lnw_s[kMaxTeams];                   // the head's log weights (drawn teams meaningful)
    __shared__ int32_t page_s[kVsChunk / 16];
    __shared__ float rlnw_s[kVsChunk / 16];

    // Block -> (group, chunk, head of the group), as launch_value_sample lays them out.
    const int NC = p.vs_chunks;
    const int per_group = NC * p.G;
    const int groups = p.B * p.Hkv;
    const int xcd = int(blockIdx.x & 7), local = int(blockIdx.x >> 3);
    int group, idx;
    if (groups >= 8) {
        const int gpx = (groups + 7) >> 3;
        group = xcd * gpx + local / per_group;
        idx = local % per_group;
    } else {
        const int R = 8 / groups;                        // XCDs per group
        group = xcd / R;
        idx = local * R + xcd % R;
    }
    if (group >= groups || idx >= per_group) return;
    const int c = idx / p.G;
    const int bh = group * p.G + idx % p.G;
    const int b = bh / p.Hq, g = group % p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = p.T;

    const int Lraw = p.seq_lens[b];
    const KV *qg = static_cast<const KV *>(p.q) + size_t(bh) * D;
    if (tid < D) q_s[tid] = to_f32(qg[tid]);
    if (tid < p.words) ht.bits[tid] = p.bitmaps[size_t(bh) * p.words + tid];
    for (int t = tid; t < p.P; t += kVsThreads) {
        pt_s[t] = p.page_table[size_t(b) * p.P + t];
        lnw_s[t] = p.lnw[size_t(bh) * p.P + t];
    }
    const int L = clamp_len(Lraw, p.P * T);
    const int K = (L + T - 1) / T;
    __syncthreads();
    if (K == 0) return;                                  // empty sequence (uniform)
    const int words = (K + 31) >> 5;
    if (wave == 0) team_prefix(ht, words);
    __syncthreads();
    const int n = drawn_tokens(ht, words, K, L, T);
    const int g0 = c * kVsChunk;
    if (g0 >= n) return;                                 // uniform
    const int r0 = g0 / T;                               // first rank of the chunk (T divides kVsChunk)
    const int nr = min(kVsChunk / T, ht.spre[words] - r0);
    if (tid < nr) {
        const int t = team_of_rank(ht, words, r0 + tid);
        page_s[tid] = int32_t(clamp_page(pt_s[t], p.num_pages));
        rlnw_s[tid] = lnw_s[t];
    }
    __syncthreads();

    // Every pass's key rows in flight, then the scores.
    const int part = tid % sel::kParts, slot = tid / sel::kParts;
    float qp[Pt::N];
#pragma unroll
    for (int i = 0; i < Pt::N; ++i) qp[i] = q_s[part * Pt::N + i];
    const KV *kbase = static_cast<const KV *>(p.k_pages);
    uint4 raw[kVsPasses][Pt::LOADS];
#pragma unroll
    for (int ps = 0; ps < kVsPasses; ++ps) {
        int gl = ps * kVsTokensPerPass + slot;
        if (g0 + gl >= n) gl = 0;                        // in bounds; the score is dropped
        const int r = gl / T, j = gl - r * T;
        const KV *row = kbase + (size_t(page_s[r]) * p.Hkv + g) * size_t(T) * D + k_offset(j, part * Pt::N, T, D);
#pragma unroll
        for (int x = 0; x < Pt::LOADS; ++x) raw[ps][x] = ld16(row + x * Pt::VPC);
    }
    double l[kVsPasses];
    double mx = -INFINITY;
#pragma unroll
    for (int ps = 0; ps < kVsPasses; ++ps) {
        const int gl = ps * kVsTokensPerPass + slot;
        const double sc = sel::row_score(sel::part_dot_raw<KV, D>(raw[ps], qp), p.scale);
        l[ps] = g0 + gl < n ? sc + double(rlnw_s[gl / T]) : -INFINITY;
        mx = fmax(mx, l[ps]);
    }
    mx = wave_max_d(mx);
    if (lane == 0) wred[wave] = mx;
    __syncthreads();
    double m = wred[0];
    for (int w = 1; w < kVsWaves; ++w) m = fmax(m, wred[w]);
    // Thread (slot, part) writes the exponential of pass `part`'s token.
    double mine = l[0];
#pragma unroll
    for (int ps = 1; ps < kVsPasses; ++ps)
        if (part == ps) mine = l[ps];
    e_s[part * kVsTokensPerPass + slot] = mine == -INFINITY ? 0.0 : exp(mine - m);
    __syncthreads();                                     // e_s complete; wred is reused below

    // Running sums inside the chunk, in token order.
    const double incl = sel::wave_incl_scan(e_s[tid]);
    if (lane == 63) wred[wave] = incl;
    __syncthreads();
    double base = 0.0;
    for (int w = 0; w < wave; ++w) base += wred[w];
    const double cs = base + incl;
    const size_t hoff = size_t(bh) * NC;
    if (g0 + tid < n) {
        p.vs_cs[hoff * kVsChunk + g0 + tid] = cs;
        if ((tid & (kVsPiece - 1)) == kVsPiece - 1 || g0 + tid == n - 1)
            p.vs_piece[(hoff + c) * kVsPieces + tid / kVsPiece] = cs;
    }
    if (tid == kVsThreads - 1) {
        p.vs_sum[(hoff + c) * 2] = m;
        p.vs_sum[(hoff + c) * 2 + 1] = cs;
    }
}

template <typename KV, int D>
__global__ __launch_bounds__(kVsThreads) void vs_sample_kernel(Params p) {
    constexpr int NSUB = kVsThreads / D;                 // sample subsets in the value sums
    __shared__ HeadTeams ht;
    __shared__ int32_t pt_s[kMaxTeams];                  // the sequence's page-table row
    __shared__ double sum_s[kVsMaxChunks * 2];           // the chunks' (max, total) pairs
    __shared__ double cum_s[kVsMaxChunks];               // C at each chunk's end
    __shared__ double f_s[kVsMaxChunks];                 // exp(m_c - m)
    __shared__ double mz_s[2];                           // m, Z
    __shared__ double piece_s[kVsMaxChunks * kVsPieces]; // running sums at the pieces' ends
    __shared__ int32_t owner[kVsMaxTokens];              // first sample of each sampled drawn token
    __shared__ int32_t cnt_s[kVsMaxSamples];             // samples of the token whose first sample is k
    __shared__ int32_t pick_g[kVsMaxSamples];            // drawn-token index of sample k
    __shared__ int32_t pick_page[kVsMaxSamples];
    __shared__ int32_t pick_j[kVsMaxSamples];
    __shared__ int32_t u_page[kVsMaxSamples];            // distinct sampled tokens, first-sample order
    __shared__ int32_t u_j[kVsMaxSamples];
    __shared__ float u_w[kVsMaxSamples];                 // their sample counts
    __shared__ int32_t wcnt[kVsWaves + 1];
    __shared__ float acc[kVsThreads / 64][128];

    const int bh = int(blockIdx.x & 7) * int(gridDim.x >> 3) + int(blockIdx.x >> 3);
    if (bh >= p.B * p.Hq) return;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = p.T, S = p.vs_samples, NC = p.vs_chunks;

    const int Lraw = p.seq_lens[b];
    if (tid < p.words) ht.bits[tid] = p.bitmaps[size_t(bh) * p.words + tid];
    if (tid < 2 * NC) sum_s[tid] = p.vs_sum[size_t(bh) * NC * 2 + tid];
    for (int i = tid; i < NC * kVsPieces; i += kVsThreads) piece_s[i] = p.vs_piece[size_t(bh) * NC * kVsPieces + i];
    for (int t = tid; t < p.P; t += kVsThreads) pt_s[t] = p.page_table[size_t(b) * p.P + t];
    const int L = clamp_len(Lraw, p.P * T);
    const int K = (L + T - 1) / T;
    __syncthreads();
    int n = 0, words = 0;
    if (K > 0) {                                         // uniform
        words = (K + 31) >> 5;
        if (wave == 0) team_prefix(ht, words);
        __syncthreads();
        n = drawn_tokens(ht, words, K, L, T);
    }
    if (n <= 0) {                                        // empty sequence (uniform)
        if (tid < D) p.out[size_t(bh) * D + tid] = 0.0f;
        if (tid == 0 && p.lse) p.lse[bh] = kNegInfF;
        if (p.vs_positions)
            for (int k = tid; k < S; k += kVsThreads) p.vs_positions[size_t(bh) * S + k] = -1;
        return;
    }
    const int nc = (n + kVsChunk - 1) / kVsChunk;
    if (wave == 0) {
        // Chunk totals rescaled to the head's max and scanned in chunk order.
        const double mc = lane < nc ? sum_s[lane * 2] : -INFINITY;
        const double zc = lane < nc ? sum_s[lane * 2 + 1] : 0.0;
        const double m = wave_max_d(mc);
        const double f = lane < nc ? exp(mc - m) : 0.0;
        const double cum = sel::wave_incl_scan(zc * f);
        if (lane < nc) {
            cum_s[lane] = cum;
            f_s[lane] = f;
        }
        if (lane == nc - 1) {
            mz_s[0] = m;
            mz_s[1] = cum;
        }
    }
    __syncthreads();
    const double m = mz_s[0], Z = mz_s[1];

    // Samples: chunk, then 16-token piece, then token.
    for (int k = tid; k < S; k += kVsThreads) {
        const double target = value_point(p, k, h, b) * Z;
        int c = nc - 1;
        for (int i = nc - 1; i >= 0; --i)
            if (target < cum_s[i]) c = i;
        const double base = c > 0 ? cum_s[c - 1] : 0.0, f = f_s[c];
        const int cnt = min(kVsChunk, n - c * kVsChunk);
        const int npiece = (cnt + kVsPiece - 1) / kVsPiece;
        const double *cs = p.vs_cs + (size_t(bh) * NC + c) * kVsChunk;
        const double *ends = piece_s + c * kVsPieces;
        int pc = npiece - 1;
        for (int i = npiece - 1; i >= 0; --i)
            if (target < base + ends[i] * f) pc = i;
        const int lo = pc * kVsPiece, len = min(kVsPiece, cnt - lo);
        double v[kVsPiece];                              // the piece (128 bytes; tail entries repeat)
#pragma unroll
        for (int j = 0; j < kVsPiece; j += 2) {
            if (j + 1 < len) {
                const uint4 w2 = ld16(cs + lo + j);
                v[j] = __hiloint2double(int(w2.y), int(w2.x));
                v[j + 1] = __hiloint2double(int(w2.w), int(w2.z));
            } else {
                v[j] = cs[lo + min(j, len - 1)];
                v[j + 1] = v[j];
            }
        }
        int jj = -1;
#pragma unroll
        for (int j = kVsPiece - 1; j >= 0; --j)
            if (j < len && target < base + v[j] * f) jj = j;
        if (jj < 0) {                                    // rounding at the piece's end: its last token with mass
            jj = len - 1;
            while (jj > 0 && !(v[jj] > v[jj - 1])) --jj;
        }
        const int gi = c * kVsChunk + lo + jj;
        const int r = gi / T, j = gi - r * T;
        const int t = team_of_rank(ht, words, r);
        pick_g[k] = gi;
        pick_page[k] = int32_t(clamp_page(pt_s[t], p.num_pages));
        pick_j[k] = j;
        if (p.vs_positions) p.vs_positions[size_t(bh) * S + k] = t * T + j;
    }
    __syncthreads();

    // Distinct sampled tokens and their counts, in the order of their first
    // sample: a token's value lines are read once however often it is drawn.
    if (tid < S) {
        owner[pick_g[tid]] = kVsMaxSamples;              // only the entries the samples touch
        cnt_s[tid] = 0;
    }
    __syncthreads();
    if (tid < S) atomicMin(&owner[pick_g[tid]], tid);
    __syncthreads();
    int first = 0;
    if (tid < S) {
        const int o = owner[pick_g[tid]];
        first = o == tid;
        atomicAdd(&cnt_s[o], 1);
    }
    __syncthreads();
    const int count = tid < S ? cnt_s[tid] : 0;
    const int fin = sel::wave_incl_scan(first);
    if (lane == 63) wcnt[wave] = fin;
    __syncthreads();
    int before = 0, nu = 0;
    for (int w = 0; w < kVsWaves; ++w) {
        if (w < wave) before += wcnt[w];
        nu += wcnt[w];
    }
    if (first) {
        const int u = before + fin - 1;
        u_page[u] = pick_page[tid];
        u_j[u] = pick_j[tid];
        u_w[u] = float(count);
    }
    __syncthreads();

    // Values: thread (subset, channel) sums count x value over the distinct
    // tokens u = subset, subset + NSUB, ... in order; the subsets are then
    // added in order.
    const KV *vbase = static_cast<const KV *>(p.v_pages);
    const int ch = tid % D, sub = tid / D;
    float a = 0.0f;
    for (int u0 = sub; u0 < nu; u0 += kVsBatch * NSUB) {
        float x[kVsBatch];
#pragma unroll
        for (int i = 0; i < kVsBatch; ++i) {             // every load of the batch first
            const int u = u0 + i * NSUB;
            x[i] = 0.0f;
            if (u < nu) {
                const KV *tile = vbase + (size_t(u_page[u]) * p.Hkv + g) * size_t(T) * D;
                x[i] = to_f32(tile[v_offset(u_j[u], ch, T, D)]);
            }
        }
#pragma unroll
        for (int i = 0; i < kVsBatch; ++i)
            if (u0 + i * NSUB < nu) a = fmaf(u_w[u0 + i * NSUB], x[i], a);
    }
    acc[sub][ch] = a;
    __syncthreads();
    if (tid < D) {
        float s = 0.0f;
        for (int u = 0; u < NSUB; ++u) s += acc[u][tid];
        p.out[size_t(bh) * D + tid] = s / float(S);
    }
    if (tid == 0 && p.lse) p.lse[bh] = float(m + log(Z));
}

}  // namespace

santa_status launch_value_sample(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t groups = int64_t(p.B) * p.Hkv, gpx = (groups + 7) / 8;
    const int64_t per_group = int64_t(p.vs_chunks) * p.G;
    // Logit blocks: 8 XCD columns of gpx groups each, or, with fewer than 8
    // groups, each group's blocks dealt over 8 / groups XCDs.
    const int64_t lrows = groups >= 8 ? gpx * per_group : (per_group + 8 / groups - 1) / (8 / groups);
    const dim3 lgrid(unsigned(8 * lrows)), sgrid(unsigned(8 * gpx * p.G)), block(kVsThreads);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) {
            hipLaunchKernelGGL((vs_logits_kernel<bf16_t, 64>), lgrid, block, 0, st, p);
            hipLaunchKernelGGL((vs_sample_kernel<bf16_t, 64>), sgrid, block, 0, st, p);
        } else {
            hipLaunchKernelGGL((vs_logits_kernel<bf16_t, 128>), lgrid, block, 0, st, p);
            hipLaunchKernelGGL((vs_sample_kernel<bf16_t, 128>), sgrid, block, 0, st, p);
        }
    } else {
        if (p.d == 64) {
            hipLaunchKernelGGL((vs_logits_kernel<float, 64>), lgrid, block, 0, st, p);
            hipLaunchKernelGGL((vs_sample_kernel<float, 64>), sgrid, block, 0, st, p);
        } else {
            hipLaunchKernelGGL((vs_logits_kernel<float, 128>), lgrid, block, 0, st, p);
            hipLaunchKernelGGL((vs_sample_kernel<float, 128>), sgrid, block, 0, st, p);
        }
    }
    return launched();
}

}  // namespace santa
