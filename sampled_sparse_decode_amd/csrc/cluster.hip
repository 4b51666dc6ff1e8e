// Hash-partitioned teams (gfx950): the cache is packed with each sequence's
// tokens, per KV head, in the order of a sign-hash partition, so that team t
// (page t of the sequence) holds tokens of similar direction.
//
// [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
// section 三 step 1 (keys are clustered into teams) and section 八 pitfall 3
// (the partition may be sequential, hash or cluster and should be a choice).
//
// Token i of (sequence b, KV head g) gets the code whose bit j, most
// significant first, is [k_i . r_j > 0] for the caller's directions r_j; the
// dot product is a float64 sum in channel order of exact products (a
// bfloat16 or float32 key times a float32 direction). Tokens are stably
// sorted by code; sorted position s lands in team s / T, slot s % T. The
// attention over a sequence does not depend on its token order, so every
// other kernel runs unchanged on the packed cache.
//
// Three launches: codes (thread per token), a stable counting sort (block
// per sequence and KV head), and the permuted pack (block per team tile).
#include "device_common.h"

namespace santa {
namespace {

using namespace dev;

// Plain source row of logical token i of sequence b, KV head g.
template <typename KV>
__device__ __forceinline__ const KV *src_row(const ClusterParams &c, const KV *base, int b, int g, int i) {
    const int64_t page = clamp_page(c.page_table[size_t(b) * c.P + i / c.T], c.num_pages);
    return base + ((size_t(page) * c.Hkv + g) * c.T + (i % c.T)) * size_t(c.d);
}

// 1. Code of every token; -1 for positions at or past the sequence's end.
template <typename KV, int D>
__global__ __launch_bounds__(kBlock) void hash_codes_kernel(ClusterParams c) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    __shared__ __attribute__((aligned(16))) double dir_s[kMaxHashBits][D];
    const int g = blockIdx.y, b = blockIdx.z;
    for (int e = threadIdx.x; e < c.bits * D; e += kBlock)
        dir_s[e / D][e % D] = double(c.directions[(size_t(g) * c.bits + e / D) * D + e % D]);
    __syncthreads();
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= c.P * c.T) return;
    const int L = clamp_len(c.seq_lens[b], c.P * c.T);
    int32_t *codes = c.codes + (size_t(b) * c.Hkv + g) * size_t(c.P) * c.T;
    if (i >= L) {
        codes[i] = -1;
        return;
    }
    const KV *row = src_row(c, static_cast<const KV *>(c.k_src), b, g, i);
    uint4 raw[D / VPC];                            // the whole row in one round trip
#pragma unroll
    for (int q = 0; q < D / VPC; ++q) raw[q] = ld16(row + q * VPC);
    double dot[kMaxHashBits];
#pragma unroll
    for (int j = 0; j < kMaxHashBits; ++j) dot[j] = 0.0;
#pragma unroll
    for (int q = 0; q < D / VPC; ++q) {
        float f[8];
        unpack(raw[q], f, KV{});
#pragma unroll
        for (int j = 0; j < kMaxHashBits; ++j) {
            if (j < c.bits) {
#pragma unroll
                for (int e = 0; e < VPC; e += 2) {       // channel order; products exact: fma = add
                    const double2 r = *reinterpret_cast<const double2 *>(&dir_s[j][q * VPC + e]);
                    dot[j] = fma(double(f[e]), r.x, dot[j]);
                    dot[j] = fma(double(f[e + 1]), r.y, dot[j]);
                }
            }
        }
    }
    int code = 0;
#pragma unroll
    for (int j = 0; j < kMaxHashBits; ++j)
        if (j < c.bits) code = 2 * code + (dot[j] > 0.0 ? 1 : 0);
    codes[i] = code;
}

// 2. Stable counting sort by code of one (sequence, KV head): token_of[s] =
//    the token at sorted position s. Wavefront w owns a contiguous range of
//    tokens; hist[w][code] first counts its range, then becomes its cursor
//    (the sorted position of the next token of that code in the range).
//    Inside a range, groups of 64 tokens are taken in order; a lane's rank
//    among the earlier lanes of its group with the same code comes from
//    ballots over the code bits, so equal codes keep token order.
constexpr int kSortThreads = 1024;
constexpr int kSortWaves = kSortThreads / 64;

__global__ __launch_bounds__(kSortThreads) void hash_rank_kernel(ClusterParams c) {
    __shared__ int32_t hist[kSortWaves][1 << kMaxHashBits];
    __shared__ int32_t wsum[kSortWaves];
    const int g = blockIdx.x % c.Hkv, b = blockIdx.x / c.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = 1 << c.bits, cap = c.P * c.T;
    const int L = clamp_len(c.seq_lens[b], cap);
    const size_t head = (size_t(b) * c.Hkv + g) * size_t(cap);
    const int32_t *codes = c.codes + head;
    int32_t *token_of = c.token_of + head;

    for (int e = tid; e < kSortWaves * nb; e += kSortThreads) hist[e / nb][e % nb] = 0;
    for (int s = L + tid; s < cap; s += kSortThreads) token_of[s] = -1;
    __syncthreads();
    const int per = (L + kSortWaves - 1) / kSortWaves;
    const int lo = min(L, wave * per), hi = min(L, lo + per);
    // Codes are loaded kBatch groups of 64 at a time, so a pass waits for
    // memory once per batch rather than once per group.
    constexpr int kBatch = 16;
    for (int i0 = lo; i0 < hi; i0 += 64 * kBatch) {
        int cb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + 64 * u + lane;
            cb[u] = i < hi ? codes[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (cb[u] >= 0) atomicAdd(&hist[wave][cb[u] & (nb - 1)], 1);
    }
    __syncthreads();

    // Exclusive scan of the code totals (thread = code), then the cursors.
    int total = 0;
    if (tid < nb)
        for (int w = 0; w < kSortWaves; ++w) total += hist[w][tid];
    int incl = total;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = incl - total;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    if (tid < nb) {
        for (int w = 0; w < kSortWaves; ++w) {
            const int n = hist[w][tid];
            hist[w][tid] = base;
            base += n;
        }
    }
    __syncthreads();

    const uint64_t below = (uint64_t(1) << lane) - 1;
    for (int b0 = lo; b0 < hi; b0 += 64 * kBatch) {
        int cb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = b0 + 64 * u + lane;
            cb[u] = i < hi ? codes[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = b0 + 64 * u + lane;
            const bool valid = i < hi;
            const int code = valid ? (cb[u] & (nb - 1)) : 0;
            uint64_t same = __ballot(valid);
            for (int j = 0; j < c.bits; ++j) {
                const bool bit = (code >> j) & 1;
                const uint64_t ones = __ballot(valid && bit);
                same &= bit ? ones : ~ones;
            }
            const int rank = __popcll(same & below);
            const int cursor = valid ? hist[wave][code] : 0;
            if (valid && cursor + rank < cap) token_of[cursor + rank] = i;
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == 0) hist[wave][code] = cursor + __popcll(same);   // the group's first lane
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// 3. Team tile t of (sequence b, KV head g) from the plain source rows of
//    the tokens at sorted positions tT .. tT + T - 1 (zeros past the end),
//    written in the cache's tile order, one chunk of C tokens at a time.
//    Key pieces are 16-byte runs of one source row, copied directly; the
//    chunk's value rows are first staged in LDS with whole-row loads (rows
//    padded by one 4-byte bank), then written channel-major.
template <typename KV, int D>
__global__ __launch_bounds__(kBlock) void pack_hashed_kernel(ClusterParams c) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    constexpr int RP = D + 4 / int(sizeof(KV));          // padded LDS row
    __shared__ int32_t src_s[256];
    __shared__ __attribute__((aligned(16))) KV v_s[32][RP];
    const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int cap = c.P * c.T;
    const int L = clamp_len(c.seq_lens[b], cap);
    if (t >= (L + c.T - 1) / c.T) return;
    const int32_t *token_of = c.token_of + (size_t(b) * c.Hkv + g) * size_t(cap) + size_t(t) * c.T;
    for (int s = threadIdx.x; s < c.T; s += kBlock) {
        const int i = token_of[s];
        src_s[s] = (i >= 0 && i < L) ? i : -1;
    }
    __syncthreads();
    const int64_t page = clamp_page(c.page_table[size_t(b) * c.P + t], c.num_pages);
    const size_t tile = (size_t(page) * c.Hkv + g) * size_t(c.T) * D;
    KV *kd = static_cast<KV *>(c.k_dst) + tile;
    KV *vd = static_cast<KV *>(c.v_dst) + tile;
    const KV *ks = static_cast<const KV *>(c.k_src);
    const KV *vs = static_cast<const KV *>(c.v_src);
    const int C = chunk_tokens(c.T);
    constexpr int RPC = D / VPC;                          // 16-byte pieces per row
    for (int chunk = 0; chunk < c.T / C; ++chunk) {
        KV *kc = kd + size_t(chunk) * C * D;
        KV *vc = vd + size_t(chunk) * C * D;
        for (int q = threadIdx.x; q < C * RPC; q += kBlock) {
            const int s = q / RPC, col = (q % RPC) * VPC;
            const int i = src_s[chunk * C + s];
            const uint4 kx = i >= 0 ? ld16(src_row(c, ks, b, g, i) + col) : make_uint4(0, 0, 0, 0);
            const uint4 vx = i >= 0 ? ld16(src_row(c, vs, b, g, i) + col) : make_uint4(0, 0, 0, 0);
            // keys: slab col / 32, token s, channels col % 32 ..
            *reinterpret_cast<uint4 *>(kc + (col >> 5) * (C * 32) + s * 32 + (col & 31)) = kx;
            const KV *vxe = reinterpret_cast<const KV *>(&vx);
#pragma unroll
            for (int u = 0; u < VPC; ++u) v_s[s][col + u] = vxe[u];
        }
        __syncthreads();
        for (int q = threadIdx.x; q < C * RPC; q += kBlock) {
            const int ch = q / (C / VPC), s0 = (q % (C / VPC)) * VPC;
            KV x[VPC];
#pragma unroll
            for (int u = 0; u < VPC; ++u) x[u] = v_s[s0 + u][ch];
            *reinterpret_cast<uint4 *>(vc + ch * C + s0) = *reinterpret_cast<const uint4 *>(x);
        }
        __syncthreads();
    }
}

}  // namespace

santa_status launch_pack_hashed(const ClusterParams &c, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 cgrid((c.P * c.T + kBlock - 1) / kBlock, c.Hkv, c.B);
    if (c.dtype == SANTA_BF16) {
        if (c.d == 64) hipLaunchKernelGGL((hash_codes_kernel<bf16_t, 64>), cgrid, dim3(kBlock), 0, st, c);
        else hipLaunchKernelGGL((hash_codes_kernel<bf16_t, 128>), cgrid, dim3(kBlock), 0, st, c);
    } else {
        if (c.d == 64) hipLaunchKernelGGL((hash_codes_kernel<float, 64>), cgrid, dim3(kBlock), 0, st, c);
        else hipLaunchKernelGGL((hash_codes_kernel<float, 128>), cgrid, dim3(kBlock), 0, st, c);
    }
    santa_status s = launched();
    if (s != SANTA_OK) return s;
    hipLaunchKernelGGL(hash_rank_kernel, dim3(c.B * c.Hkv), dim3(kSortThreads), 0, st, c);
    s = launched();
    if (s != SANTA_OK) return s;
    const dim3 pgrid(c.P, c.Hkv, c.B);
    if (c.dtype == SANTA_BF16) {
        if (c.d == 64) hipLaunchKernelGGL((pack_hashed_kernel<bf16_t, 64>), pgrid, dim3(kBlock), 0, st, c);
        else hipLaunchKernelGGL((pack_hashed_kernel<bf16_t, 128>), pgrid, dim3(kBlock), 0, st, c);
    } else {
        if (c.d == 64) hipLaunchKernelGGL((pack_hashed_kernel<float, 64>), pgrid, dim3(kBlock), 0, st, c);
        else hipLaunchKernelGGL((pack_hashed_kernel<float, 128>), pgrid, dim3(kBlock), 0, st, c);
    }
    return launched();
}

}  // namespace santa
