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
//   [SAN] "Stochastic Sparse Attention for Memory-Bound Inference" (the
//         SANTA page), abstract: stratified and systematic sampling give
//         lower-variance variants; here they place the team draws.
//
// Selection is decided in float64: products of two bfloat16 (or float32)
// values are exact in float64 and the sums are accurate to ~1e-16, so a draw
// can land on a different team than an exact computation only when its
// uniform lies within ~1e-15 of a cumulative-probability boundary.
#include "device_common.h"

namespace santa {
namespace {

using namespace dev;

// One block per (sequence b, query head h) of 512 or 1024 threads (8 or 16
// wavefronts; at about 120 registers, four wavefronts per SIMD, so one
// 1024-thread or two 512-thread blocks fill a CU and the float64 chains of
// one wavefront hide behind the others). 512 threads when the page table has
// at most 256 teams (two pipelined scoring passes measured faster than one
// pass of twice the wavefronts) or when there are more heads than CUs (so
// every head runs in the first round); 1024 threads otherwise. Writes the
// head's team bitmap and, for every drawn team t, log w_t = -log(pi_t) (0
// under full coverage), plus the optional sorted team list and 1/pi.
constexpr int kSel = 1024;
constexpr int kSelCUs = 256;                       // 1024-thread blocks that run at once (one per CU)
constexpr int kParts = 4;                          // threads per representative row

// Order-preserving map of a float to a signed integer (for LDS atomicMax).
__device__ __forceinline__ int float_key(float f) {
    const int i = __float_as_int(f);
    return i >= 0 ? i : (i ^ 0x7fffffff);
}
__device__ __forceinline__ float key_float(int k) { return __int_as_float(k >= 0 ? k : (k ^ 0x7fffffff)); }

// PIPE: request each scoring pass's representative rows before the previous
// pass is scored (chosen by the host when the page table allows more than
// one pass; same arithmetic either way).
template <typename KV, int D, bool PIPE, int NT>
__global__ __launch_bounds__(NT, 4) void select_kernel(Params p) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    constexpr int CPP = D / VPC / kParts;          // 16-byte chunks per thread and row
    constexpr int ROWS = NT / kParts;              // rows scored per pass
    constexpr bool kPipe = PIPE && CPP <= 4;       // float32 rows at d = 128 do not fit the registers
    __shared__ double q_s[D];
    __shared__ double e_s[kMaxTeams];              // scores, then exp(s - m)
    __shared__ double c_s[kMaxTeams];              // cumulative sums of e within a wavefront's teams
    __shared__ float lnw_s[kMaxTeams];             // log weight of each team if drawn
    __shared__ float w_s[kMaxTeams];               // 1 / pi of each team if drawn
    __shared__ double pts_s[kMaxTeams];            // draw points in [0, 1) (M < K <= kMaxTeams)
    __shared__ uint32_t bits_s[kMaxWords];
    __shared__ int32_t wpre_s[kMaxWords + 1];
    __shared__ int maxkey_s;

    const int tid = threadIdx.x, lane = tid & 63;
    const int bh = blockIdx.x;
    const int b = bh / p.Hq, h = bh - b * p.Hq, g = h / p.G;
    const KV *reps = static_cast<const KV *>(p.reps) + size_t(b) * p.P * p.Hkv * D;
    const int row0 = tid / kParts, part = tid % kParts;

    // Round trip 1: sequence length, query, and (speculatively, every row is
    // in bounds) this thread's quarter of representative row row0.
    const int Lraw = p.seq_lens[b];
    const KV *q = static_cast<const KV *>(p.q) + size_t(bh) * D;
    if (tid < D) q_s[tid] = double(to_f32(q[tid]));
    if (tid < p.words) bits_s[tid] = 0u;
    if (tid == 0) maxkey_s = float_key(-INFINITY);
    uint4 raw[CPP];
    {
        const KV *r = reps + (size_t(row0 < p.P ? row0 : 0) * p.Hkv + g) * D + part * CPP * VPC;
#pragma unroll
        for (int j = 0; j < CPP; ++j) raw[j] = ld16(r + j * VPC);
    }
    // Draw points, computed while the rows are in flight. Draw j's uniform is
    // u_j = (x + 1/2) 2^-32 from Philox word j mod 4 of counter
    // (j / 4, h, b, offset); its point is u_j (independent draws),
    // (j + u_0) / M (systematic) or (j + u_j) / M (stratified; [SAN]).
    // j + u is exact in float64. Not needed when M covers every team.
    if (p.M < p.P) {
        double u0 = 0.0;                          // the systematic scheme's shared offset
        if (p.scheme == SANTA_DRAW_SYSTEMATIC) {
            const uint4 r0 = philox4x32_10(make_uint4(0u, uint32_t(h), uint32_t(b), p.offset), p.seed_lo,
                                           p.seed_hi);
            u0 = (double(r0.x) + 0.5) * 0x1p-32;
        }
        for (int j = tid; j < p.M; j += NT) {
            const uint4 r = philox4x32_10(make_uint4(uint32_t(j) >> 2, uint32_t(h), uint32_t(b), p.offset),
                                          p.seed_lo, p.seed_hi);
            const uint32_t x = (j & 3) == 0 ? r.x : (j & 3) == 1 ? r.y : (j & 3) == 2 ? r.z : r.w;
            const double uj = (double(x) + 0.5) * 0x1p-32;
            double point = uj;
            if (p.scheme == SANTA_DRAW_SYSTEMATIC) point = (double(j) + u0) / double(p.M);
            else if (p.scheme == SANTA_DRAW_STRATIFIED) point = (double(j) + uj) / double(p.M);
            pts_s[j] = point;
        }
    }
    const int L = clamp_len(Lraw, p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    __syncthreads();

    // 1. Representative scores s_t = q . rep_t / sqrt(d) in float64 (products
    //    of two bfloat16 or two float32 values are exact in float64); four
    //    threads per row, two partial sums each, added in a fixed order. The
    //    float32-rounded maximum is gathered on the way (LDS atomic max).
    float mloc = -INFINITY;
    const int tEnd = ((K + ROWS - 1) / ROWS) * ROWS;
    for (int t = row0; t < tEnd; t += ROWS) {
        if (!kPipe && t != row0) {
            const KV *r = reps + (size_t(t < K ? t : 0) * p.Hkv + g) * D + part * CPP * VPC;
#pragma unroll
            for (int j = 0; j < CPP; ++j) raw[j] = ld16(r + j * VPC);
        }
        // The next pass's rows are requested before this pass is scored, so
        // K > ROWS teams cost one memory latency, not one per pass (bfloat16
        // rows; float32 rows would need more registers than 1024 threads have).
        const bool more = t + ROWS < tEnd;                  // uniform over the block
        uint4 nxt[CPP];
        if (kPipe && more) {
            const int tn = t + ROWS;
            const KV *r = reps + (size_t(tn < K ? tn : 0) * p.Hkv + g) * D + part * CPP * VPC;
#pragma unroll
            for (int j = 0; j < CPP; ++j) nxt[j] = ld16(r + j * VPC);
        }
        double a0 = 0.0, a1 = 0.0;
#pragma unroll
        for (int j = 0; j < CPP; ++j) {
            float f[8];
            unpack(raw[j], f, KV{});
            const int c0 = part * CPP * VPC + j * VPC;
#pragma unroll
            for (int e = 0; e < VPC; e += 2) {
                a0 = fma(double(f[e]), q_s[c0 + e], a0);
                a1 = fma(double(f[e + 1]), q_s[c0 + e + 1], a1);
            }
        }
        double acc = a0 + a1;
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        const double sc = acc * p.scale;
        if (t < K) {
            if (part == 0) e_s[t] = sc;
            mloc = fmaxf(mloc, float(sc));
        }
        if (kPipe && more) {
#pragma unroll
            for (int j = 0; j < CPP; ++j) raw[j] = nxt[j];
        }
    }
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off, 64));
    if (lane == 0) atomicMax(&maxkey_s, float_key(mloc));
    __syncthreads();

    // 2. Team softmax numerators e_t = exp(s_t - m) in float64, with the
    //    float32-rounded max as the shift (any shift at or near the max
    //    cancels in C_t / C_last and in p_t = e_t / C_last). Thread tid owns
    //    the contiguous teams [tid per, (tid + 1) per); c_s holds cumulative
    //    sums within each wavefront's range, so C_t = B_w + c_s[t] with B_w
    //    the sum of the previous wavefronts' last entries.
    const double m = double(key_float(maxkey_s));
    const int per = (K + NT - 1) / NT;
    const int t0 = min(K, tid * per), t1 = min(K, t0 + per);
    double local = 0.0;
    for (int t = t0; t < t1; ++t) {
        const double e = exp(e_s[t] - m);
        e_s[t] = e;
        local += e;
    }
    double incl = local;
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    double run = incl - local;
    for (int t = t0; t < t1; ++t) {
        run += e_s[t];
        c_s[t] = run;
    }
    __syncthreads();

    // Wavefront bases B_w = sum of the previous wavefronts' last cumulative
    // entries, added in wavefront order (the same way in every thread), so
    // C is one monotone sequence and Z = C_last.
    constexpr int kW = NT / 64;
    auto wave_end = [&](int w, double bw) {
        const int lo = min(K, w * 64 * per), hi = min(K, (w + 1) * 64 * per);
        return hi > lo ? bw + c_s[hi - 1] : bw;
    };
    double Z = 0.0;
    double base[kW];                               // B_w, kept for the draws' first search step
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        base[w] = Z;
        Z = wave_end(w, Z);
    }
    const bool full = K > 0 && p.M >= K;

    // 3. Draws: draw j (thread j, then j + NT, ...) lands on the first team
    //    t with target_j = point_j Z below C_t: the first wavefront range
    //    whose end exceeds the target, then a binary search inside it. If no
    //    team qualifies (unreachable for u < 1), the last team with mass.
    //    Meanwhile the threads counted from the top compute pi_t and log w_t.
    if (K > 0) {
        if (full) {
            for (int t = tid; t < K; t += NT) atomicOr(&bits_s[t >> 5], 1u << (t & 31));
        } else {
            for (int j = tid; j < p.M; j += NT) {
                const double target = pts_s[j] * Z;
                int t;
                if (target < Z) {
                    // First wavefront whose end exceeds the target: the ends
                    // are the next bases (non-decreasing; ranges fill in order),
                    // so it is the number of bases B_1 .. B_(kW-1) <= target.
                    int w = 0;
#pragma unroll
                    for (int i = 1; i < kW; ++i) w += base[i] <= target ? 1 : 0;
                    double bw = 0.0;
#pragma unroll
                    for (int i = 0; i < kW; ++i)
                        if (i == w) bw = base[i];
                    int lo = min(K, w * 64 * per), hi = min(K, (w + 1) * 64 * per) - 1;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (target < bw + c_s[mid]) hi = mid; else lo = mid + 1;
                    }
                    t = lo;
                } else {
                    t = K - 1;
                    while (t > 0 && !(e_s[t] > 0.0)) --t;
                }
                atomicOr(&bits_s[t >> 5], 1u << (t & 31));
            }
        }
        // Inclusion probabilities. Independent: 1 - (1 - p)^M =
        // -expm1(M log1p(-p)). Systematic: min(1, M p). Stratified: in units
        // of 1/M the team covers [a, a + w), a = M C_(t-1) / Z, w = M p; it
        // meets unit k = floor(a) over q1 = min(w, k + 1 - a) and the next
        // units over r = w - q1, so pi = 1 if r >= 1 (a whole unit inside)
        // else 1 - (1 - q1)(1 - r) = w - q1 r.
        for (int t = NT - 1 - tid; t < K; t += NT) {
            double lw = 0.0, w = 1.0;
            if (!full) {
                const double pt_ = e_s[t] / Z;
                double pi;
                if (p.scheme == SANTA_DRAW_SYSTEMATIC) {
                    pi = fmin(1.0, double(p.M) * pt_);
                } else if (p.scheme == SANTA_DRAW_STRATIFIED) {
                    double cprev = 0.0;
                    if (t > 0) {
                        const int ww = (t - 1) / (64 * per);
                        double bw = 0.0;
                        for (int i = 0; i < ww; ++i) bw = wave_end(i, bw);
                        cprev = bw + c_s[t - 1];
                    }
                    const double wd = double(p.M) * pt_;
                    const double a = double(p.M) * cprev / Z;
                    const double q1 = fmin(wd, (floor(a) + 1.0) - a);
                    const double rest = wd - q1;
                    pi = rest >= 1.0 ? 1.0 : wd - q1 * rest;
                } else {
                    const float pf = float(pt_);
                    if (pf >= 1e-30f) {                 // float32 (relative error below 1e-6)
                        const float pif = -expm1f(float(p.M) * log1pf(-pf));
                        lnw_s[t] = -logf(pif);
                        w_s[t] = 1.0f / pif;
                        continue;
                    }
                    pi = -expm1(double(p.M) * log1p(-pt_));
                }
                w = 1.0 / pi;
                lw = -log(pi);
            }
            lnw_s[t] = float(lw);
            w_s[t] = float(w);
        }
    }
    __syncthreads();

    // 4. Outputs: bitmap, log weights of drawn teams, optional sorted list.
    if (tid < p.words) p.bitmaps[size_t(bh) * p.words + tid] = bits_s[tid];
    float *lnw = p.lnw + size_t(bh) * p.P;
    for (int t = tid; t < K; t += NT)
        if ((bits_s[t >> 5] >> (t & 31)) & 1u) lnw[t] = lnw_s[t];
    if (p.sampled) {
        if (tid == 0) {
            int acc = 0;
            for (int i = 0; i < p.words; ++i) {
                wpre_s[i] = acc;
                acc += __popc(bits_s[i]);
            }
            wpre_s[p.words] = acc;
        }
        __syncthreads();
        for (int t = tid; t < K; t += NT) {
            const uint32_t word = bits_s[t >> 5];
            if (!((word >> (t & 31)) & 1u)) continue;
            const int rank = wpre_s[t >> 5] + __popc(word & ((1u << (t & 31)) - 1u));
            p.sampled[size_t(bh) * p.M + rank] = t;
            p.inv_pi[size_t(bh) * p.M + rank] = w_s[t];
        }
        for (int r = wpre_s[p.words] + tid; r < p.M; r += NT) {
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

template <typename KV, int D, int NT>
static void launch_select_as(const Params &p, hipStream_t st, bool pipe) {
    const dim3 grid(p.B * p.Hq);
    if (pipe) hipLaunchKernelGGL((select_kernel<KV, D, true, NT>), grid, dim3(NT), 0, st, p);
    else hipLaunchKernelGGL((select_kernel<KV, D, false, NT>), grid, dim3(NT), 0, st, p);
}

template <typename KV, int D>
static void launch_select_d(const Params &p, hipStream_t st) {
    const bool many_heads = int64_t(p.B) * p.Hq > kSelCUs;
    const bool short_table = p.P <= kSel / kParts;
    // pipe: more than one scoring pass
    if (many_heads || short_table) launch_select_as<KV, D, kSel / 2>(p, st, p.P > kSel / 2 / kParts);
    else launch_select_as<KV, D, kSel>(p, st, p.P > kSel / kParts);
}

santa_status launch_select(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) launch_select_d<bf16_t, 64>(p, st);
        else launch_select_d<bf16_t, 128>(p, st);
    } else {
        if (p.d == 64) launch_select_d<float, 64>(p, st);
        else launch_select_d<float, 128>(p, st);
    }
    return launched();
}

santa_status launch_given(const Params &p, void *stream) {
    hipLaunchKernelGGL(given_kernel, dim3(p.B * p.Hq), dim3(kBlock), 0, static_cast<hipStream_t>(stream), p);
    return launched();
}

}  // namespace santa
