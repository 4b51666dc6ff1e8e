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
    if (c.starts && tid < nb) {
        int32_t *st = c.starts + (size_t(b) * c.Hkv + g) * (nb + 1);
        st[tid] = base;
        if (tid == nb - 1) st[nb] = L;
    }
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

// ---------------------------------------------------------------------------
// k-means-partitioned teams: the codes are cluster ids from Lloyd iterations
// on the keys of each (sequence, KV head); the stable sort and the permuted
// pack above then lay the teams out as for the hash partition.
//
// [EXP] section 三 step 1 (teams are clusters of keys) and section 八
// pitfall 3 (the clustering is a choice). Lloyd's iteration (assign every
// key to its nearest centroid, move each centroid to the mean of its keys)
// is the textbook k-means; the steps the pages leave open are fixed as
// follows. C_b = min(L_b, clusters, or K_b when clusters is 0) clusters start
// at the keys of tokens floor(c L_b / C_b). Nearest means the largest
// k . mu_c - |mu_c|^2 / 2 (the same order as the smallest distance), both
// terms float64 sums in channel order of separately rounded products, ties
// to the lowest c. A non-empty cluster moves to the float64 mean of its keys
// summed in token order from +0.0; an empty one stays. `iters` assignments,
// with a move between consecutive ones. Every sum and product is rounded as
// written (contraction off), so the partition is reproducible bit for bit.

__device__ __forceinline__ int kmeans_clusters(const ClusterParams &c, int L) {
    const int K = (L + c.T - 1) / c.T;
    const int want = c.clusters > 0 ? c.clusters : K;
    return min(L, min(want, c.cmax));
}

// Centroid k of (b, g) from one channel per thread (D threads): stored, and
// its squared norm summed in channel order by thread 0.
template <int D>
__device__ __forceinline__ void store_centroid(const ClusterParams &c, int b, int g, int k, double m,
                                               double *m_s) {
#pragma clang fp contract(off)
    const size_t row = (size_t(b) * c.Hkv + g) * size_t(c.cmax) + k;
    c.mu[row * D + threadIdx.x] = m;
    m_s[threadIdx.x] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        double h = 0.0;
        for (int ch = 0; ch < D; ++ch) h = h + m_s[ch] * m_s[ch];
        c.half[row] = h;
    }
}

// 1. Start: centroid k = the key of token floor(k L / C).
template <typename KV, int D>
__global__ __launch_bounds__(D) void kmeans_init_kernel(ClusterParams c) {
    __shared__ double m_s[D];
    const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = clamp_len(c.seq_lens[b], c.P * c.T);
    const int C = kmeans_clusters(c, L);
    if (k >= C) return;
    const int i = int((int64_t(k) * L) / C);
    const KV *row = src_row(c, static_cast<const KV *>(c.k_src), b, g, i);
    store_centroid<D>(c, b, g, k, double(to_f32(row[threadIdx.x])), m_s);
}

// 2. Assign (thread per token): the cluster with the largest
//    k . mu - |mu|^2 / 2, lowest index on ties; -1 past the sequence's end.
//    The block's keys are staged channel-major in LDS, and the centroids
//    kCentroidGroup at a time (also channel-major, so one channel's values
//    for the group are contiguous broadcast reads); the channel loop is a
//    runtime loop, which keeps the live values to a few channels.
constexpr int kAssignThreads = 128;
constexpr int kCentroidGroup = 16;

template <typename KV, int D>
__global__ __launch_bounds__(kAssignThreads) void kmeans_assign_kernel(ClusterParams c) {
#pragma clang fp contract(off)
    constexpr int VPC = KVTraits<KV>::kPerChunk;
    __shared__ __attribute__((aligned(16))) double mu_s[D][kCentroidGroup];
    __shared__ double h_s[kCentroidGroup];
    __shared__ KV k_s[D][kAssignThreads];
    const int g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int cap = c.P * c.T;
    const int L = clamp_len(c.seq_lens[b], cap);
    const int i = blockIdx.x * kAssignThreads + tid;
    int32_t *codes = c.codes + (size_t(b) * c.Hkv + g) * size_t(cap);
    if (blockIdx.x * kAssignThreads >= L) {              // the whole block is past the end
        if (i < cap) codes[i] = -1;
        return;
    }
    const bool active = i < L;
    const int C = kmeans_clusters(c, L);
    if (active) {
        const KV *row = src_row(c, static_cast<const KV *>(c.k_src), b, g, i);
#pragma unroll
        for (int q = 0; q < D / VPC; ++q) {
            const uint4 v = ld16(row + q * VPC);
            const KV *ve = reinterpret_cast<const KV *>(&v);
#pragma unroll
            for (int u = 0; u < VPC; ++u) k_s[q * VPC + u][tid] = ve[u];
        }
    } else {
        for (int ch = 0; ch < D; ++ch) k_s[ch][tid] = KV(0);
    }
    const size_t head = (size_t(b) * c.Hkv + g) * size_t(c.cmax);
    const double *mu = c.mu + head * D;
    const double *half = c.half + head;
    double best = -INFINITY;
    int bi = 0;
    for (int c0 = 0; c0 < C; c0 += kCentroidGroup) {
        const int n = min(kCentroidGroup, C - c0);
        __syncthreads();                                 // also orders the key staging
        for (int e = tid; e < kCentroidGroup * D; e += kAssignThreads)
            mu_s[e % D][e / D] = e / D < n ? mu[size_t(c0) * D + e] : 0.0;
        if (tid < kCentroidGroup) h_s[tid] = tid < n ? half[c0 + tid] : 0.0;
        __syncthreads();
        double dot[kCentroidGroup];
#pragma unroll
        for (int u = 0; u < kCentroidGroup; ++u) dot[u] = 0.0;
#pragma unroll 2
        for (int ch = 0; ch < D; ++ch) {
            const double x = double(to_f32(k_s[ch][tid]));
#pragma unroll
            for (int u = 0; u < kCentroidGroup; ++u) dot[u] = dot[u] + x * mu_s[ch][u];
        }
#pragma unroll
        for (int u = 0; u < kCentroidGroup; ++u) {
            if (u < n) {
                const double score = dot[u] - h_s[u] * 0.5;
                if (score > best) {
                    best = score;
                    bi = c0 + u;
                }
            }
        }
    }
    if (i < cap) codes[i] = active ? bi : -1;
}

// 3. Move (block per cluster, thread per channel): the members are the
//    cluster's run of the stable sort, so they come in token order.
template <typename KV, int D>
__global__ __launch_bounds__(D) void kmeans_update_kernel(ClusterParams c) {
#pragma clang fp contract(off)
    __shared__ double m_s[D];
    const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int cap = c.P * c.T;
    const int L = clamp_len(c.seq_lens[b], cap);
    const int C = kmeans_clusters(c, L);
    if (k >= C) return;
    const int nb = 1 << c.bits;
    const int32_t *st = c.starts + (size_t(b) * c.Hkv + g) * size_t(nb + 1);
    const int s0 = clamp_len(st[k], L), s1 = clamp_len(st[k + 1], L);
    if (s1 <= s0) return;                                // empty: the centroid stays
    const int32_t *token_of = c.token_of + (size_t(b) * c.Hkv + g) * size_t(cap);
    const KV *ks = static_cast<const KV *>(c.k_src);
    constexpr int kRows = 8;                             // member rows in flight
    double acc = 0.0;
    for (int s = s0; s < s1; s += kRows) {
        float x[kRows];
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            x[u] = 0.0f;
            if (s + u < s1) {
                int t = token_of[s + u];
                t = t < 0 ? 0 : (t >= L ? L - 1 : t);
                x[u] = to_f32(src_row(c, ks, b, g, t)[threadIdx.x]);
            }
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u)
            if (s + u < s1) acc = acc + double(x[u]);
    }
    store_centroid<D>(c, b, g, k, acc / double(s1 - s0), m_s);
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

namespace {

template <typename KV, int D>
santa_status run_kmeans(const ClusterParams &c, int32_t iters, hipStream_t st) {
    const dim3 cgrid(c.cmax, c.Hkv, c.B);
    const dim3 agrid((c.P * c.T + kAssignThreads - 1) / kAssignThreads, c.Hkv, c.B);
    hipLaunchKernelGGL((kmeans_init_kernel<KV, D>), cgrid, dim3(D), 0, st, c);
    santa_status s = launched();
    for (int it = 0; it < iters && s == SANTA_OK; ++it) {
        hipLaunchKernelGGL((kmeans_assign_kernel<KV, D>), agrid, dim3(kAssignThreads), 0, st, c);
        if ((s = launched()) != SANTA_OK) break;
        hipLaunchKernelGGL(hash_rank_kernel, dim3(c.B * c.Hkv), dim3(kSortThreads), 0, st, c);
        if ((s = launched()) != SANTA_OK) break;
        if (it + 1 < iters) {
            hipLaunchKernelGGL((kmeans_update_kernel<KV, D>), cgrid, dim3(D), 0, st, c);
            s = launched();
        }
    }
    if (s != SANTA_OK) return s;
    hipLaunchKernelGGL((pack_hashed_kernel<KV, D>), dim3(c.P, c.Hkv, c.B), dim3(kBlock), 0, st, c);
    return launched();
}

}  // namespace

santa_status launch_pack_kmeans(const ClusterParams &c, int32_t iters, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (c.dtype == SANTA_BF16)
        return c.d == 64 ? run_kmeans<bf16_t, 64>(c, iters, st) : run_kmeans<bf16_t, 128>(c, iters, st);
    return c.d == 64 ? run_kmeans<float, 64>(c, iters, st) : run_kmeans<float, 128>(c, iters, st);
}

}  // namespace santa
