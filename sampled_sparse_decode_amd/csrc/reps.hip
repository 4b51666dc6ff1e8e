// Representative keys of SANTA++ teams (gfx950).
//
// [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
// section 三 step 2: one representative key per team (mean, medoid or random
// are listed; this library uses the mean). [ABS] "SANTA++: Sampling Attention
// through Representative Keys", arXiv 2609.35629, abstract: selection reads
// these summary keys instead of the whole cache.
//
// Mean: rep = round_to_cache_type(sum of the team's n valid keys / n):
// float64 sums (exact for bfloat16 keys), one correctly rounded float64
// divide, one rounding to nearest even into the cache type.
// Medoid: the member whose summed Euclidean distance to all n members is
// smallest (float64, channel order inside a distance, member order across
// distances, lowest index on ties), copied exactly.
// Random: member floor(x n / 2^32) for one Philox4x32-10 word x of its own
// key stream, copied exactly.
// Every kernel also refreshes only the teams that received appended tokens
// (update mode), with the same arithmetic, so an updated row equals a rebuilt
// one bit for bit.
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
    // Update mode: block x recomputes team prev / T + x, the first being the
    // team that holds token prev (the first appended token); a sequence that
    // did not grow keeps every row.
    const int prev = p.prev_lens ? clamp_len(p.prev_lens[b], p.P * p.T) : 0;
    if (p.prev_lens && prev >= L) return;      // nothing appended: no team changed
    const int t = prev / p.T + blockIdx.x;
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
            v[i] = (r < n) ? ld16_stream(keys + k_offset(r, ch * VPC, p.T, D)) : make_uint4(0, 0, 0, 0);
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

// Team t, KV head g and sequence b of the block, or false if the team is
// past the sequence's end. Update mode shifts x by the first touched team.
struct TeamOfBlock {
    int t, g, b, n;
    const void *tile;
};
template <typename KV, int D>
__device__ __forceinline__ bool team_of_block(const Params &p, TeamOfBlock &tm) {
    tm.g = blockIdx.y;
    tm.b = blockIdx.z;
    const int L = clamp_len(p.seq_lens[tm.b], p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    const int prev = p.prev_lens ? clamp_len(p.prev_lens[tm.b], p.P * p.T) : 0;
    if (p.prev_lens && prev >= L) return false;   // nothing appended: no team changed
    tm.t = prev / p.T + blockIdx.x;
    if (tm.t >= K) return false;
    const int64_t page = clamp_page(p.page_table[size_t(tm.b) * p.P + tm.t], p.num_pages);
    tm.n = min(p.T, L - tm.t * p.T);
    tm.tile = static_cast<const KV *>(p.k_pages) + (size_t(page) * p.Hkv + tm.g) * size_t(p.T) * D;
    return true;
}

// Copies key row `member` of the block's team into its representative row
// (16-byte pieces; a piece never crosses a 32-channel slab).
template <typename KV, int D>
__device__ __forceinline__ void copy_member(const Params &p, const TeamOfBlock &tm, int member) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    const KV *keys = static_cast<const KV *>(tm.tile);
    KV *rep = static_cast<KV *>(p.reps_out) + ((size_t(tm.b) * p.P + tm.t) * p.Hkv + tm.g) * D;
    for (int c = threadIdx.x; c < D / VPC; c += blockDim.x)
        *reinterpret_cast<uint4 *>(rep + c * VPC) = ld16(keys + k_offset(member, c * VPC, p.T, D));
}

// Medoid. Block of max(64, T) threads; thread i owns member i (its key in
// registers as float, exact for both cache types) and adds its n distances
// in member order. The other members are staged through LDS JC at a time,
// as float64, and read by every lane at the same address (broadcast). Four distances
// are formed at once so that their channel-ordered sums interleave.
template <typename KV, int D>
__global__ __launch_bounds__(256) void medoid_reps_kernel(Params p) {
#pragma clang fp contract(off)
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    constexpr int CH = D / VPC;               // 16-byte pieces per key row
    constexpr int JC = 32;                    // members per LDS stage
    __shared__ double sk[JC][D];             // staged members, widened once
    __shared__ double red_v[4];
    __shared__ int red_i[4];

    TeamOfBlock tm;
    if (!team_of_block<KV, D>(p, tm)) return;
    const KV *keys = static_cast<const KV *>(tm.tile);
    const int tid = threadIdx.x, n = tm.n;
    const int i = tid < n ? tid : n - 1;      // lanes past n shadow the last member; their totals are dropped

    float ki[D];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        float f[8];
        unpack(ld16(keys + k_offset(i, c * VPC, p.T, D)), f, KV{});
#pragma unroll
        for (int e = 0; e < VPC; ++e) ki[c * VPC + e] = f[e];
    }

    double total = 0.0;
    for (int j0 = 0; j0 < n; j0 += JC) {
        const int jn = min(JC, n - j0);
        __syncthreads();
        for (int q = tid; q < JC * CH; q += blockDim.x) {
            const int jj = q / CH, c = q % CH;
            float f[8];
            unpack(jj < jn ? ld16(keys + k_offset(j0 + jj, c * VPC, p.T, D)) : make_uint4(0, 0, 0, 0),
                   f, KV{});
#pragma unroll
            for (int e = 0; e < VPC; ++e) sk[jj][c * VPC + e] = double(f[e]);
        }
        __syncthreads();
        for (int jj = 0; jj < jn; jj += 4) {        // jj + 3 < JC: rows past jn are zeros
            // Keep the own key as float: without this the compiler hoists its
            // D float64 conversions out of the loop and spills at D = 128.
#pragma unroll
            for (int c = 0; c < D; ++c) asm volatile("" : "+v"(ki[c]));
            double s2[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int c = 0; c < D; c += 2) {
                double2 v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const double2 *>(&sk[jj + u][c]);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const double a = double(ki[c + e]);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const double diff = a - (e == 0 ? v[u].x : v[u].y);
                        s2[u] = s2[u] + diff * diff;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (jj + u < jn) total = total + __dsqrt_rn(s2[u]);
        }
    }

    // Block argmin of (total, member), lowest member on equal totals.
    double v = tid < n ? total : INFINITY;
    int vi = tid < n ? tid : 0x7fffffff;
    for (int off = 32; off > 0; off >>= 1) {
        const double ov = __shfl_xor(v, off, 64);
        const int oi = __shfl_xor(vi, off, 64);
        if (ov < v || (ov == v && oi < vi)) { v = ov; vi = oi; }
    }
    if ((tid & 63) == 0) { red_v[tid >> 6] = v; red_i[tid >> 6] = vi; }
    __syncthreads();
    double bv = red_v[0];
    int bi = red_i[0];
    for (int w = 1; w < int(blockDim.x >> 6); ++w)
        if (red_v[w] < bv || (red_v[w] == bv && red_i[w] < bi)) { bv = red_v[w]; bi = red_i[w]; }
    // Non-finite keys can leave no member below +inf: stay inside the team.
    copy_member<KV, D>(p, tm, bi < n ? bi : 0);
}

// Random member: one 64-thread block per team; every lane forms the same index.
template <typename KV, int D>
__global__ __launch_bounds__(64) void random_reps_kernel(Params p) {
    TeamOfBlock tm;
    if (!team_of_block<KV, D>(p, tm)) return;
    const uint4 x = philox4x32_10(make_uint4(uint32_t(tm.t), uint32_t(tm.g), uint32_t(tm.b), 0u),
                                  p.seed_lo ^ kRepKeyXor, p.seed_hi);
    const int member = int((uint64_t(x.x) * uint64_t(tm.n)) >> 32);
    copy_member<KV, D>(p, tm, member);
}

template <typename KV, int D>
void launch_reps_kind(const Params &p, dim3 grid, hipStream_t st) {
    if (p.rep_kind == SANTA_REP_MEDOID) {
        const int threads = p.T < 64 ? 64 : p.T;
        hipLaunchKernelGGL((medoid_reps_kernel<KV, D>), grid, dim3(threads), 0, st, p);
    } else if (p.rep_kind == SANTA_REP_RANDOM) {
        hipLaunchKernelGGL((random_reps_kernel<KV, D>), grid, dim3(64), 0, st, p);
    } else {
        hipLaunchKernelGGL((build_reps_kernel<KV, D>), grid, dim3(kBlock), 0, st, p);
    }
}

}  // namespace

santa_status launch_build_reps(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(p.prev_lens ? p.update_teams : p.P, p.Hkv, p.B);
    if (p.dtype == SANTA_BF16) {
        if (p.d == 64) launch_reps_kind<bf16_t, 64>(p, grid, st);
        else launch_reps_kind<bf16_t, 128>(p, grid, st);
    } else {
        if (p.d == 64) launch_reps_kind<float, 64>(p, grid, st);
        else launch_reps_kind<float, 128>(p, grid, st);
    }
    return launched();
}

}  // namespace santa
