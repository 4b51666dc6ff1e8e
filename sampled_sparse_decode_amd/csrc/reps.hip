// Representative keys of SANTA++ teams (gfx950).
//
// [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
// section 三 step 2: one representative key per team (mean, medoid or random
// are listed; this library uses the mean). [ABS] "SANTA++: Sampling Attention
// through Representative Keys", arXiv 2609.35629, abstract: the query scores
// one representative from each team.
//
// rep = round_to_cache_type(sum of the team's n valid keys / n): float64 sums
// (exact for bfloat16 keys), one correctly rounded float64 divide, one
// rounding to nearest even into the cache type. The same kernel refreshes
// only the teams that received appended tokens (update mode), with the same
// arithmetic, so an updated row equals a rebuilt one bit for bit.
#include "device_common.h"

namespace santa {
namespace {

using namespace dev;

// One 256-thread block per (team t, KV head g, sequence b). Threads are
// (16-byte chunk, row lane): each sums every RL-th key row of its chunk, then
// the row lanes are added in a fixed order.
template <typename KV, int D>
__global__ __launch_bounds__(kBlock) void build_reps_kernel(Params p) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    constexpr int CH = D / VPC;
    constexpr int RL = kBlock / CH;
    constexpr int UNROLL = 8;
    __shared__ double part_s[RL][D];

    const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int L = clamp_len(p.seq_lens[b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    // Update mode: block x recomputes team first + x, first being the team
    // that held the sequence's token prev_len (the first appended token).
    const int first = p.prev_lens ? clamp_len(p.prev_lens[b], p.P * p.T) / p.T : 0;
    const int t = first + blockIdx.x;
    if (t >= K) return;
    const int64_t page = clamp_page(p.page_table[size_t(b) * p.P + t], p.num_pages);
    const int n = min(p.T, L - t * p.T);
    const KV *keys = static_cast<const KV *>(p.k_pages) + (size_t(page) * p.Hkv + g) * size_t(p.T) * D;
    const int ch = tid % CH, rl = tid / CH;

    double acc[VPC];
#pragma unroll
    for (int e = 0; e < VPC; ++e) acc[e] = 0.0;
    for (int r0 = rl; r0 < n; r0 += RL * UNROLL) {
        uint4 v[UNROLL];
#pragma unroll
        for (int i = 0; i < UNROLL; ++i) {
            const int r = r0 + i * RL;
            v[i] = (r < n) ? ld16(keys + k_offset(r, ch * VPC, p.T, D)) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < UNROLL; ++i) {
            float f[8];
            unpack(v[i], f, KV{});
#pragma unroll
            for (int e = 0; e < VPC; ++e) acc[e] += double(f[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < VPC; ++e) part_s[rl][ch * VPC + e] = acc[e];
    __syncthreads();
    KV *reps = static_cast<KV *>(p.reps_out) + ((size_t(b) * p.P + t) * p.Hkv + g) * D;
    for (int c = tid; c < D; c += kBlock) {
        double sum = 0.0;
        for (int r = 0; r < RL; ++r) sum += part_s[r][c];
        store_rounded(&reps[c], sum / double(n));
    }
}

}  // namespace

santa_status launch_build_reps(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(p.prev_lens ? p.update_teams : p.P, p.Hkv, p.B);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) hipLaunchKernelGGL((build_reps_kernel<bf16_t, 64>), grid, dim3(kBlock), 0, st, p);
        else hipLaunchKernelGGL((build_reps_kernel<bf16_t, 128>), grid, dim3(kBlock), 0, st, p);
    } else {
        if (p.d == 64) hipLaunchKernelGGL((build_reps_kernel<float, 64>), grid, dim3(kBlock), 0, st, p);
        else hipLaunchKernelGGL((build_reps_kernel<float, 128>), grid, dim3(kBlock), 0, st, p);
    }
    return launched();
}

}  // namespace santa
