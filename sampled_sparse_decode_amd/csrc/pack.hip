// Writes KV pages, or appended tokens, into the cache's tile layout (gfx950).
//
// Source pages are [num_pages][Hkv][T][d] for both keys and values (the
// order a prefill or an append produces). Destination tiles use the chunked
// layout the decode kernels read: chunks of C = min(T, 32) tokens, keys as
// 32-channel slabs [C][32], values channel-major [d][C]. A pure permutation:
// every element is copied bit for bit.
#include "device_common.h"

namespace santa {
namespace {

using namespace dev;

// One block per (page, KV head) tile; each thread writes 16-byte pieces of
// the destination tile.
template <typename KV>
__global__ __launch_bounds__(kBlock) void pack_pages_kernel(PackParams pp) {
    constexpr int VPC = KVTraits<KV>::kPerChunk;     // elements per 16 bytes
    const size_t tile = size_t(blockIdx.x) * pp.T * pp.d;
    const KV *ks = static_cast<const KV *>(pp.k_src) + tile;
    const KV *vs = static_cast<const KV *>(pp.v_src) + tile;
    KV *kd = static_cast<KV *>(pp.k_dst) + tile;
    KV *vd = static_cast<KV *>(pp.v_dst) + tile;
    const int C = chunk_tokens(pp.T);
    const int pieces = pp.T * pp.d / VPC;
    for (int j = threadIdx.x; j < pieces; j += kBlock) {
        const int e = j * VPC;
        const int chunk = e / (C * pp.d), r = e - chunk * (C * pp.d);
        {   // keys: VPC consecutive channels of one token
            const int slab = r / (C * 32), r2 = r - slab * (C * 32);
            const int tok = chunk * C + r2 / 32, ch = slab * 32 + (r2 & 31);
            *reinterpret_cast<uint4 *>(kd + e) = ld16(ks + size_t(tok) * pp.d + ch);
        }
        {   // values: VPC consecutive tokens of one channel
            const int ch = r / C, tok0 = chunk * C + (r - ch * C);
            KV x[VPC];
#pragma unroll
            for (int i = 0; i < VPC; ++i) x[i] = vs[size_t(tok0 + i) * pp.d + ch];
            *reinterpret_cast<uint4 *>(vd + e) = *reinterpret_cast<const uint4 *>(x);
        }
    }
}

// One thread per (sequence, new token, KV head, channel): the token's
// position is prev_len + i; its key and value channel go to their tile-order
// offsets in the page the table names. Tokens past the sequence's new length
// or the table, and pages outside the cache, are skipped.
template <typename KV>
__global__ __launch_bounds__(kBlock) void append_kv_kernel(AppendParams ap) {
    const int64_t gid = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t rows = int64_t(ap.B) * ap.max_new * ap.Hkv;
    if (gid >= rows * ap.d) return;
    const int64_t row = gid / ap.d;
    const int ch = int(gid - row * ap.d);
    const int g = int(row % ap.Hkv);
    const int64_t bi = row / ap.Hkv;
    const int i = int(bi % ap.max_new), b = int(bi / ap.max_new);
    const int prev = ap.prev_lens[b], now = ap.seq_lens[b];
    if (prev < 0 || i >= now - prev) return;
    const int64_t pos = int64_t(prev) + i;
    if (pos >= int64_t(ap.P) * ap.T) return;
    const int32_t page = ap.page_table[size_t(b) * ap.P + size_t(pos / ap.T)];
    if (page < 0 || int64_t(page) >= ap.num_pages) return;
    const int tok = int(pos % ap.T);
    const size_t tile = (size_t(page) * ap.Hkv + g) * size_t(ap.T) * ap.d;
    const size_t src = size_t(row) * ap.d + ch;
    static_cast<KV *>(ap.k_pages)[tile + k_offset(tok, ch, ap.T, ap.d)] = static_cast<const KV *>(ap.k_new)[src];
    static_cast<KV *>(ap.v_pages)[tile + v_offset(tok, ch, ap.T, ap.d)] = static_cast<const KV *>(ap.v_new)[src];
}

}  // namespace

santa_status launch_append_kv(const AppendParams &ap, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t threads = int64_t(ap.B) * ap.max_new * ap.Hkv * ap.d;
    const dim3 grid(unsigned((threads + kBlock - 1) / kBlock));
    if (ap.dtype == SANTA_BF16) hipLaunchKernelGGL((append_kv_kernel<bf16_t>), grid, dim3(kBlock), 0, st, ap);
    else hipLaunchKernelGGL((append_kv_kernel<float>), grid, dim3(kBlock), 0, st, ap);
    return launched();
}

santa_status launch_pack_pages(const PackParams &pp, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(unsigned(pp.tiles));
    if (pp.dtype == SANTA_BF16) hipLaunchKernelGGL((pack_pages_kernel<bf16_t>), grid, dim3(kBlock), 0, st, pp);
    else hipLaunchKernelGGL((pack_pages_kernel<float>), grid, dim3(kBlock), 0, st, pp);
    return launched();
}

}  // namespace santa
