// Split-K gather over drawn teams and the cross-split combine (gfx950).
//
// Sources:
//   [ABS] "SANTA++: Sampling Attention through Representative Keys",
//         arXiv 2609.35629, abstract: only the drawn teams' tokens are
//         scored, and a drawn team's terms count 1/pi times (pi: its chance
//         of being drawn), which keeps the sums unbiased.
//   [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
//         section 三 steps 4-5 (exact scores inside drawn teams, the 1/pi
//         weights).
//
// Every gather block works for one (sequence b, KV head g) group: it streams
// the K and V chunks of teams some query head of g drew (dense mode: every
// team, every head, weight 0 in log space) from HBM exactly once, scores them
// for the heads that drew them, and runs an online softmax in which the team
// weight w is folded into the logit (s_j + log w): numerator and denominator
// both carry w, and nothing overflows however large 1/pi gets. It writes one
// partial (max, sum, weighted value sum) per head of g at its split slot; the
// combine merges a head's partials in slot order.
//
// Two block shapes:
//   bf16 caches  balanced blocks (gather_balanced_kernel, matrix cores): the
//                group's drawn chunks, listed by union rank, cut into even
//                contiguous ranges, one per block.
//   fp32 caches  team-range blocks (gather_f32_kernel, float64 scores): block
//                s owns teams [s tps, (s + 1) tps) (tps divides 32, so their
//                bits sit in one bitmap word), or with union ranks the drawn
//                teams of ranks [s tps, (s + 1) tps).
//
// Cache layout: each (page, KV head) tile is cut into chunks of 32 tokens;
// keys are stored as 32-channel slabs [32 tokens][32 channels] and values
// channel-major [d][32 tokens] inside a chunk. Every 16-byte load of a
// matrix-core operand then sits in a run of whole 128-byte lines that the
// same instruction reads completely.
#include "selection.h"

namespace santa {
namespace {

using namespace dev;

constexpr int kGM = kMaxGroup;     // head slots per KV head (16)

// Per-block team list of the fp32 gather, filled by load_team_list or
// load_ranked_team_list.
struct TeamList {
    int64_t page[kMaxTeamsPerSplit];
    int32_t n[kMaxTeamsPerSplit];          // valid tokens of the team
    float lnw[kMaxTeamsPerSplit][kGM];     // log weight per head slot, -inf if the head did not draw it
    int32_t raw_page[kMaxTeamsPerSplit];
    float raw_lnw[kMaxTeamsPerSplit][kGM];
    uint32_t mask[kMaxTeamsPerSplit];      // heads that drew each team slot
    uint32_t hword[kGM];                   // bitmap word of each head covering the block's teams
    int32_t slot[kMaxTeamsPerSplit];       // team slot of each kept team
    int32_t len;                           // clamped sequence length
    int32_t nteams;
    // union-rank mode
    uint32_t hbits[kGM][kMaxWords];        // every team bitmap word of the group's heads
    uint32_t uword[kMaxWords];             // their union
    int32_t upre[kMaxWords + 1];           // exclusive prefix of the union popcounts
    int32_t team[kMaxTeamsPerSplit];
};

// Builds the block's team list in LDS with a single round trip to memory:
// the sequence length, the teams' page ids, the heads' bitmap word and log
// weights are all loaded before any is used. Returns the number of kept teams
// (uniform over the block).
__device__ int load_team_list(const Params &p, TeamList &tl, int s, int g, int b) {
    const int tid = threadIdx.x;
    const int G = p.G;
    const int hbase = b * p.Hq + g * G;
    const bool dense = p.mode == kModeDense;
    const int i = tid / kGM, h = tid % kGM;          // team slot, head slot
    const int t = s * p.tps + i;
    const bool in = i < p.tps && t < p.P;
    int32_t pg = 0;
    float lw = kNegInfF;
    uint32_t word = 0u;
    if (in && h == 0) pg = p.page_table[size_t(b) * p.P + t];
    if (!dense) {
        if (in && h < G) lw = p.lnw[size_t(hbase + h) * p.P + t];
        if (i == 0 && h < G) word = p.bitmaps[size_t(hbase + h) * p.words + (s * p.tps) / 32];
    }
    const int Lraw = p.seq_lens[b];
    if (in) {
        tl.raw_lnw[i][h] = lw;
        if (h == 0) tl.raw_page[i] = pg;
    }
    if (i == 0) tl.hword[h] = word;
    if (tid == 0) tl.len = clamp_len(Lraw, p.P * p.T);
    __syncthreads();
    const int L = tl.len;
    const int K = (L + p.T - 1) / p.T;
    if (tid < p.tps) {
        const int tt = s * p.tps + tid;
        uint32_t mask = 0u;
        if (tt < K) {
            if (dense) {
                mask = (1u << G) - 1u;
            } else {
                for (int k = 0; k < G; ++k) mask |= ((tl.hword[k] >> (tt & 31)) & 1u) << k;
            }
        }
        tl.mask[tid] = mask;
    }
    __syncthreads();
    if (tid == 0) {
        int n = 0;
        for (int j = 0; j < p.tps; ++j)
            if (tl.mask[j]) tl.slot[n++] = j;
        tl.nteams = n;
    }
    __syncthreads();
    const int nt = tl.nteams;
    if (i < nt) {
        const int j = tl.slot[i];
        const int tt = s * p.tps + j;
        if (h == 0) {
            tl.page[i] = clamp_page(tl.raw_page[j], p.num_pages);
            tl.n[i] = min(p.T, L - tt * p.T);
        }
        const bool drew = (tl.mask[j] >> h) & 1u;
        tl.lnw[i][h] = drew ? (dense ? 0.0f : tl.raw_lnw[j][h]) : kNegInfF;
    }
    __syncthreads();
    return nt;
}

// In union-rank mode every slot below the grid width holds a fresh (max, sum)
// pair: a head with no team in the block gets an empty one (max -inf), which
// the combine skips.
__device__ __forceinline__ void write_empty_partial(const Params &p, int head, int s) {
    reinterpret_cast<float2 *>(p.part_ml)[size_t(head) * p.slots + s] = make_float2(kNegInfF, 0.0f);
}

// Union-rank team list (multi-team SANTA++ blocks): block s takes the teams
// of union ranks [s * tps, (s + 1) * tps) of the group, so every block but the
// last gets exactly tps drawn teams. Two round trips: the group's bitmaps and
// the sequence length, then the teams' page ids and log weights.
__device__ int load_ranked_team_list(const Params &p, TeamList &tl, int s, int g, int b) {
    const int tid = threadIdx.x;
    const int G = p.G;
    const int hbase = b * p.Hq + g * G;
    for (int idx = tid; idx < G * p.words; idx += kBlock) {
        const int h = idx / p.words, w = idx - h * p.words;
        tl.hbits[h][w] = p.bitmaps[size_t(hbase + h) * p.words + w];
    }
    const int Lraw = p.seq_lens[b];
    if (tid == 0) tl.len = clamp_len(Lraw, p.P * p.T);
    __syncthreads();
    if (tid < 64) {
        uint32_t u = 0u;
        if (tid < p.words)
            for (int h = 0; h < G; ++h) u |= tl.hbits[h][tid];
        const int cnt = __popc(u);
        int incl = cnt;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (tid >= off) incl += y;
        }
        if (tid < p.words) {
            tl.uword[tid] = u;
            tl.upre[tid] = incl - cnt;
        }
        if (tid == 63) {
            tl.upre[p.words] = incl;
            tl.nteams = max(0, min(p.tps, incl - s * p.tps));
        }
    }
    __syncthreads();
    const int nt = tl.nteams;
    if (nt == 0) return 0;
    if (tid < nt) {
        const int r = s * p.tps + tid;
        int lo = 0, hi = p.words - 1;             // last word whose prefix is <= r
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tl.upre[mid] <= r) lo = mid; else hi = mid - 1;
        }
        uint32_t u = tl.uword[lo];
        for (int k = r - tl.upre[lo]; k > 0; --k) u &= u - 1u;
        const int bit = __ffs(u) - 1;
        uint32_t mask = 0u;
        for (int h = 0; h < G; ++h) mask |= ((tl.hbits[h][lo] >> bit) & 1u) << h;
        tl.team[tid] = lo * 32 + bit;
        tl.mask[tid] = mask;
    }
    __syncthreads();
    const int i = tid / kGM, h = tid % kGM;
    if (i < nt) {
        const int t = tl.team[i];
        if (h == 0) {
            tl.page[i] = clamp_page(p.page_table[size_t(b) * p.P + t], p.num_pages);
            tl.n[i] = min(p.T, tl.len - t * p.T);
        }
        const bool drew = (tl.mask[i] >> h) & 1u;
        tl.lnw[i][h] = drew ? p.lnw[size_t(hbase + h) * p.P + t] : kNegInfF;
    }
    __syncthreads();
    return nt;
}

// ---------------------------------------------------------------------------
// bf16 gather on the matrix cores.
//
// A wavefront processes 32-token chunks of the block's teams. For a chunk it
// computes the score tile S^T (32 tokens x 16 head slots) as K Q^T with
// v_mfma_f32_16x16x32_bf16 (fp32 accumulation of exact bf16 products); rows of
// the two 16-row tiles are arranged so that lane l ends up holding, for head
// (l mod 16), the scores of the 8 consecutive tokens 8 (l div 16) + 0..7.
// That is exactly the A operand of the P V product for those tokens, and the
// matching B operand is one 16-byte load of the channel-major V page. P is
// split into a bfloat16 high part and a bfloat16 remainder so the product
// keeps ~16 significant bits of P.
// ---------------------------------------------------------------------------
template <int D>
struct MfmaChunk {
    static constexpr int KS = D / 32;     // k-steps of K Q^T
    static constexpr int NT = D / 16;     // channel tiles of P V
    uint4 k[2][KS];
    uint4 v[NT];
};

// K/V tiles are read once per call, with non-temporal loads (measured on
// MI355X: gather 14.3 -> 13.2 us at 32K batch 1, 61.7 -> 55.9 us at batch 8,
// 111 -> 105 us at 128K; the dense gather 181 -> 155 us at 128K).
// Loads are unconditional: rows past the team's end are clamped to its last
// valid row (K; those scores are masked) or to its first 8 tokens (V; zeroed
// by keep_first), so every address stays inside the page and the wavefront
// issues all of its loads back to back.
// Chunk (tokens tb .. tb + 31 of a team with n valid tokens; C = min(T, 32)
// of them stored): K slab ks holds [C][32] elements, V is [D][C]. For a tile
// of 16 keys the four 64-byte runs of a slab that one instruction reads are
// whole lines.
template <int D>
__device__ __forceinline__ void mfma_load_chunk_at(const Params &p, int64_t page, int n, int tb, int g,
                                                   int i16, int g4, MfmaChunk<D> &c) {
    const int C = chunk_tokens(p.T);
    const size_t base = (size_t(page) * p.Hkv + g) * size_t(p.T) * D + size_t(tb) * D;
    const bf16_t *kc = static_cast<const bf16_t *>(p.k_pages) + base;
    const bf16_t *vc = static_cast<const bf16_t *>(p.v_pages) + base;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tok = 8 * (i16 >> 2) + 4 * t + (i16 & 3);     // in-chunk token of this lane's row
        const bf16_t *row = kc + min(tok, max(n - 1 - tb, 0)) * 32 + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < MfmaChunk<D>::KS; ++ks) c.k[t][ks] = ld16_stream(row + ks * (C * 32));
    }
    const int tok0 = 8 * g4;
    const bf16_t *col = vc + i16 * C + (tb + tok0 < n ? tok0 : 0);
#pragma unroll
    for (int nt = 0; nt < MfmaChunk<D>::NT; ++nt) c.v[nt] = ld16_stream(col + (16 * nt) * C);
}

// Zero the bf16 elements e >= keep of a 16-byte operand (ragged team tails).
__device__ __forceinline__ uint4 keep_first(uint4 v, int keep) {
    if (keep >= 8) return v;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e0 = 2 * i;
        const uint32_t lo = (e0 < keep) ? 0x0000ffffu : 0u;
        const uint32_t hi = (e0 + 1 < keep) ? 0xffff0000u : 0u;
        w[i] &= (lo | hi);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Scores, online-softmax update and P V for one chunk; lw is the log weight
// of head i16 for the chunk's team (-inf: the head did not draw it).
template <int D>
__device__ __forceinline__ void mfma_compute_chunk_at(const Params &p, int n, int tb, float lw,
                                                      int i16, int g4, const bf16_t (*q_lds)[D + 8],
                                                      const MfmaChunk<D> &c, float &m, float &lsum,
                                                      f32x4 (&o)[D / 16]) {
    const float scale = float(p.scale);

    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < MfmaChunk<D>::KS; ++ks)
            st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, c.k[t][ks]),
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&q_lds[i16][32 * ks + 8 * g4])), st[t],
                0, 0, 0);
    }
    // Lane holds head i16, tokens tb + 8 g4 + j, j = 4 t + e.
    float sc[8];
    float cmax = kNegInfF;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int tok = tb + 8 * g4 + j;
        const float x = st[j >> 2][j & 3] * scale + lw;
        sc[j] = (tok < n && lw != kNegInfF) ? x : kNegInfF;
        cmax = fmaxf(cmax, sc[j]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_old = m;
    const float mnew = fmaxf(m, cmax);
    const float corr = (m == kNegInfF) ? 0.0f : __expf(m - mnew);
    float pj[8];
    float psum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        pj[j] = (sc[j] == kNegInfF) ? 0.0f : __expf(sc[j] - mnew);
        psum += pj[j];
    }
    lsum = lsum * corr + psum;
    m = mnew;
    // Rows of o are heads 4 g4 + e; their correction factors live in lanes
    // 4 g4 + e. Skipped when no head's running max moved (or o is still zero).
    if (__ballot(m_old != kNegInfF && corr != 1.0f) != 0ull) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ce = __shfl(corr, 4 * g4 + e, 64);
#pragma unroll
            for (int nt = 0; nt < MfmaChunk<D>::NT; ++nt) o[nt][e] *= ce;
        }
    }
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        hb[j] = f32_to_bf16_rne(pj[j]);
        lb[j] = f32_to_bf16_rne(pj[j] - __uint_as_float(hb[j] << 16));
    }
    const uint4 phu = make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                                 hb[6] | (hb[7] << 16));
    const uint4 plu = make_uint4(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16), lb[4] | (lb[5] << 16),
                                 lb[6] | (lb[7] << 16));
    const bf16x8 ph = __builtin_bit_cast(bf16x8, phu);
    const bf16x8 pl = __builtin_bit_cast(bf16x8, plu);
    const int keep = n - (tb + 8 * g4);
#pragma unroll
    for (int nt = 0; nt < MfmaChunk<D>::NT; ++nt) {
        const bf16x8 vv = __builtin_bit_cast(bf16x8, keep_first(c.v[nt], keep));
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vv, o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vv, o[nt], 0, 0, 0);
    }
}

// Cross-wavefront merge of the online-softmax states and the store of the
// block's partial at slot s of every head of the group.
template <int D, int NW = kWaves>
struct MfmaReduce {
    float m[NW][kGM];
    float l[NW][kGM];
    float o[NW][kGM][D];
    float fac[kGM][NW];
    float hm[kGM], hl[kGM];
};

template <int D, int NW = kWaves>
__device__ __forceinline__ void mfma_store_partial(const Params &p, MfmaReduce<D, NW> &rd, float m, float lsum,
                                                   const f32x4 (&o)[D / 16], int hbase, int s) {
    constexpr int NTH = NW * 64;
    constexpr int NT = D / 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int G = p.G;
    __syncthreads();                              // rd may alias the chunk loop's LDS
    // Wavefront partials: sums over the four lane groups of a head.
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (g4 == 0) {
        rd.m[wave][i16] = m;
        rd.l[wave][i16] = lsum;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) rd.o[wave][4 * g4 + e][16 * nt + i16] = o[nt][e];
    __syncthreads();

    // Merge the wavefronts in a fixed order; the per-(head, wavefront) scale
    // factors are computed once.
    if (tid < G) {
        const int h = tid;
        float mx = rd.m[0][h];
        for (int w = 1; w < NW; ++w) mx = fmaxf(mx, rd.m[w][h]);
        float l = 0.0f;
        for (int w = 0; w < NW; ++w) {
            const float f = (rd.m[w][h] == kNegInfF) ? 0.0f : expf(rd.m[w][h] - mx);
            rd.fac[h][w] = f;
            l += f * rd.l[w][h];
        }
        rd.hm[h] = mx;
        rd.hl[h] = l;
    }
    __syncthreads();
    float2 *part_ml = reinterpret_cast<float2 *>(p.part_ml);
    for (int idx = tid; idx < G * D; idx += NTH) {
        const int h = idx / D, c = idx - h * D;
        const size_t slot = size_t(hbase + h) * p.slots + s;
        if (rd.hm[h] == kNegInfF) {                 // no team of this block for the head
            if (p.ranked && c == 0) write_empty_partial(p, hbase + h, s);
            continue;
        }
        float a = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) a += rd.fac[h][w] * rd.o[w][h][c];
        p.part_acc[slot * D + c] = a;
        if (c == 0) part_ml[slot] = make_float2(rd.hm[h], rd.hl[h]);
    }
}

// Q^T operand rows (head slots >= G are zero), kept in LDS and read per
// chunk; rows padded by 16 bytes so the 16 head rows hit different banks.
template <int D>
__device__ __forceinline__ void fill_q_lds(const Params &p, bf16_t (*q_lds)[D + 8], int hbase) {
    const int tid = threadIdx.x;
    const int h = tid >> 4, cc = tid & 15;                // 16 heads x 16 pieces of 16 bytes
    if (cc * 8 < D) {
        const uint4 v = (h < p.G) ? ld16(static_cast<const bf16_t *>(p.q) + size_t(hbase + h) * D + cc * 8)
                                  : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(&q_lds[h][cc * 8]) = v;
    }
}

// ---------------------------------------------------------------------------
// Balanced gather (bf16): the chunks of a (sequence, KV head) group are
// listed in order, chunk c being 32-token piece (c mod cpt) of the union team
// of rank c / cpt (union of the teams the group's query heads drew; every
// team in dense mode), and block j of nb = gridDim.x takes the contiguous
// range [j C / nb, (j + 1) C / nb) of the C chunks, so every block of a group
// gets the same number of chunks to within one. Round trip 1 brings the
// group's bitmaps and the sequence's page-table row; a chunk's log weights
// are loaded with its K/V tiles (round trip 2), so no load waits on another
// beyond these two. Each block merges and stores one partial per head.
// ---------------------------------------------------------------------------
constexpr int kWin = 64;

template <int MAXT = kMaxTeams, int MAXG = kGM>
struct GroupChunksT {
    uint32_t hbits[MAXG][MAXT / 32];       // team bitmaps of the group's heads
    uint32_t uword[MAXT / 32];             // their union
    int32_t upre[MAXT / 32 + 1];           // exclusive prefix of the union popcounts
    int32_t len;                           // clamped sequence length
    int32_t pt[MAXT];                      // the sequence's page-table row
    int64_t page[kWin];
    int32_t n[kWin];                       // valid tokens of the chunk's team
    int32_t tb[kWin];                      // first token of the chunk within its team
    int32_t team[kWin];
    uint32_t mask[kWin];                   // heads that drew the chunk's team
};
using GroupChunks = GroupChunksT<>;

// Round trip 1 and the union: words, popcount prefix; returns the union size.
__device__ __forceinline__ void group_load(const Params &p, GroupChunks &gc, int g, int b) {
    const int tid = threadIdx.x;
    const int G = p.G;
    const bool dense = p.mode == kModeDense;
    const int hbase = b * p.Hq + g * G;
    const int Lraw = p.seq_lens[b];
    for (int t = tid; t < p.P; t += kBlock) gc.pt[t] = p.page_table[size_t(b) * p.P + t];
    if (!dense)
        for (int idx = tid; idx < G * p.words; idx += kBlock) {
            const int h = idx / p.words, w = idx - h * p.words;
            gc.hbits[h][w] = p.bitmaps[size_t(hbase + h) * p.words + w];
        }
    if (tid == 0) gc.len = clamp_len(Lraw, p.P * p.T);
    __syncthreads();
}

// The union words and their popcount prefix from the loaded group data;
// returns the union size.
template <class GC>
__device__ __forceinline__ int group_scan(const Params &p, GC &gc) {
    const int tid = threadIdx.x;
    const int G = p.G;
    const bool dense = p.mode == kModeDense;
    if (tid < 64) {
        const int K = (gc.len + p.T - 1) / p.T;
        uint32_t u = 0u;
        if (tid < p.words) {
            if (dense) {
                const int lo = tid * 32;
                u = (K >= lo + 32) ? 0xffffffffu : (K > lo ? ((1u << (K - lo)) - 1u) : 0u);
            } else {
                for (int h = 0; h < G; ++h) u |= gc.hbits[h][tid];
            }
        }
        const int cnt = __popc(u);
        int incl = cnt;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (tid >= off) incl += y;
        }
        if (tid < p.words) {
            gc.uword[tid] = u;
            gc.upre[tid] = incl - cnt;
        }
        if (tid == 63) gc.upre[p.words] = incl;
    }
    __syncthreads();
    return gc.upre[p.words];
}

__device__ int group_union(const Params &p, GroupChunks &gc, int g, int b) {
    group_load(p, gc, g, b);
    return group_scan(p, gc);
}

// Chunks c0 .. c0 + cnt - 1 (cnt <= kWin) of the group: team, heads, page,
// size, from LDS only.
template <class GC>
__device__ void chunk_window(const Params &p, GC &gc, int cpt, int c0, int cnt) {
    const int tid = threadIdx.x;
    const int G = p.G;
    if (tid < cnt) {
        const int ci = c0 + tid;
        const int r = ci / cpt, c = ci - r * cpt;
        int lo = 0, hi = p.words - 1;             // last word whose prefix is <= r
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (gc.upre[mid] <= r) lo = mid; else hi = mid - 1;
        }
        uint32_t u = gc.uword[lo];
        for (int k = r - gc.upre[lo]; k > 0; --k) u &= u - 1u;
        const int bit = __ffs(u) - 1;
        const int t = lo * 32 + bit;
        uint32_t mask = 0u;
        if (p.mode == kModeDense) mask = (1u << G) - 1u;
        else
            for (int h = 0; h < G; ++h) mask |= ((gc.hbits[h][lo] >> bit) & 1u) << h;
        gc.team[tid] = t;
        gc.mask[tid] = mask;
        gc.tb[tid] = c * 32;
        gc.page[tid] = clamp_page(gc.pt[t], p.num_pages);
        gc.n[tid] = min(p.T, gc.len - t * p.T);
    }
    __syncthreads();
}

// MODE (kModeSanta or kModeDense, equal to p.mode) is a template argument
// so the two uses show up as separate kernels in a profile.
template <int D, int MODE>
__global__ __launch_bounds__(kBlock, 3) void gather_balanced_kernel(Params p) {
    constexpr int NT = D / 16;
    struct Stream {
        GroupChunks gc;
        __attribute__((aligned(16))) bf16_t q_lds[kGM][D + 8];
    };
    __shared__ union {
        Stream st;
        MfmaReduce<D> rd;                         // used once the chunk loop is done
    } lds;
    GroupChunks &gc = lds.st.gc;

    const int j = blockIdx.x, nb = gridDim.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int hbase = b * p.Hq + g * p.G;
    constexpr bool dense = MODE == kModeDense;

    fill_q_lds<D>(p, lds.st.q_lds, hbase);
    const int U = group_union(p, gc, g, b);
    const int cpt = p.T >= 32 ? p.T / 32 : 1;
    const int total = U * cpt;
    const int c0 = int((long long)total * j / nb), c1 = int((long long)total * (j + 1) / nb);

    float m = kNegInfF, lsum = 0.0f;
    f32x4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float *lnw_h = p.lnw + size_t(hbase + i16) * p.P;
    for (int w0 = c0; w0 < c1; w0 += kWin) {
        const int cnt = min(kWin, c1 - w0);
        chunk_window(p, gc, cpt, w0, cnt);
        for (int q = wave; q < cnt; q += kWaves) {
            const bool drew = (gc.mask[q] >> i16) & 1u;
            const float lw_raw = (drew && !dense) ? lnw_h[gc.team[q]] : 0.0f;
            MfmaChunk<D> ck;
            mfma_load_chunk_at<D>(p, gc.page[q], gc.n[q], gc.tb[q], g, i16, g4, ck);
            const float lw = drew ? lw_raw : kNegInfF;
            mfma_compute_chunk_at<D>(p, gc.n[q], gc.tb[q], lw, i16, g4, lds.st.q_lds, ck, m, lsum, o);
        }
        __syncthreads();                          // the window is reused
    }
    mfma_store_partial<D>(p, lds.rd, m, lsum, o, hbase, j);
}

// ---------------------------------------------------------------------------
// SANTA++ gather over a group's union (bf16) on NW wavefronts per block: the
// block reads the team bitmaps and log weights the selection kernel left in
// the workspace and streams the group's union chunks in even contiguous
// ranges, one per block, exactly as the balanced gather above.
// Blocks are placed by XCD: consecutive (group, range) slots go to the same
// XCD (block i runs on XCD i mod 8), so the blocks of one group share the
// group's metadata in one or two L2 caches.
// ---------------------------------------------------------------------------
template <int D, int NW>
struct UnionGatherLds {
    struct Live {
        GroupChunksT<kMaxTeams, kGM> gc;
        __attribute__((aligned(16))) bf16_t q_lds[kGM][D + 8];
    };
    union {
        Live live;
        MfmaReduce<D, NW> rd;                     // used once the chunk loop is done
    };
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void santa_gather_kernel(Params p) {
    constexpr int NT = D / 16;
    constexpr int NTH = NW * 64;
    __shared__ UnionGatherLds<D, NW> lds;
    auto &gc = lds.live.gc;

    // Block -> (group, range) slot: XCD x = i mod 8 takes slots
    // [x n8, (x + 1) n8) of the n8 = gridDim.x / 8 per XCD.
    const int nb = p.max_splits;
    const int nreal = p.B * p.Hkv * nb;
    const int slot = int(blockIdx.x & 7) * int(gridDim.x >> 3) + int(blockIdx.x >> 3);
    if (slot >= nreal) return;
    const int grp = slot / nb, j = slot - grp * nb;
    const int b = grp / p.Hkv, g = grp - b * p.Hkv;
    const int hbase = b * p.Hq + g * p.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;

    // Round trip 1: length, queries, the page-table row and the heads'
    // bitmaps, all requested before any is used.
    const int Lraw = p.seq_lens[b];
    const int qh = tid >> 4, qc = tid & 15;                 // 16 head slots x 16 pieces of 16 bytes
    uint4 qv = make_uint4(0, 0, 0, 0);
    if (tid < 256 && qc * 8 < D && qh < p.G)
        qv = ld16(static_cast<const bf16_t *>(p.q) + size_t(hbase + qh) * D + qc * 8);
    constexpr int PTN = kMaxTeams / NTH, BWN = kGM * kMaxWords / NTH;
    int32_t ptv[PTN];
    uint32_t bwv[BWN];
#pragma unroll
    for (int k = 0; k < PTN; ++k) {
        const int t = tid + k * NTH;
        ptv[k] = t < p.P ? p.page_table[size_t(b) * p.P + t] : 0;
    }
#pragma unroll
    for (int k = 0; k < BWN; ++k) {
        const int idx = tid + k * NTH;
        const int h = idx / p.words, w = idx - h * p.words;
        bwv[k] = idx < p.G * p.words ? p.bitmaps[size_t(hbase + h) * p.words + w] : 0u;
    }
#pragma unroll
    for (int k = 0; k < PTN; ++k)
        if (tid + k * NTH < p.P) gc.pt[tid + k * NTH] = ptv[k];
#pragma unroll
    for (int k = 0; k < BWN; ++k) {
        const int idx = tid + k * NTH;
        if (idx < p.G * p.words) gc.hbits[idx / p.words][idx % p.words] = bwv[k];
    }
    if (tid < 256 && qc * 8 < D) *reinterpret_cast<uint4 *>(&lds.live.q_lds[qh][qc * 8]) = qv;
    if (tid == 0) gc.len = clamp_len(Lraw, p.P * p.T);
    __syncthreads();

    const int U = group_scan(p, gc);
    const int cpt = p.T >= 32 ? p.T / 32 : 1;
    const int total = U * cpt;
    const int c0 = int((long long)total * j / nb), c1 = int((long long)total * (j + 1) / nb);

    float m = kNegInfF, lsum = 0.0f;
    f32x4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float *lnw_h = p.lnw + size_t(hbase + i16) * p.P;
    for (int w0 = c0; w0 < c1; w0 += kWin) {
        const int cnt = min(kWin, c1 - w0);
        chunk_window(p, gc, cpt, w0, cnt);
        for (int q = wave; q < cnt; q += NW) {
            const bool drew = (gc.mask[q] >> i16) & 1u;
            const float lw_raw = drew ? lnw_h[gc.team[q]] : 0.0f;
            MfmaChunk<D> ck;
            mfma_load_chunk_at<D>(p, gc.page[q], gc.n[q], gc.tb[q], g, i16, g4, ck);
            const float lw = drew ? lw_raw : kNegInfF;
            mfma_compute_chunk_at<D>(p, gc.n[q], gc.tb[q], lw, i16, g4, lds.live.q_lds, ck, m, lsum, o);
        }
        __syncthreads();                          // the window is reused
    }
    mfma_store_partial<D, NW>(p, lds.rd, m, lsum, o, hbase, j);
}

// ---------------------------------------------------------------------------
// Per-head SANTA++ gather (bf16), for calls with few query heads: block
// (b, h, j) takes the j-th of S even ranges of head h's drawn chunks (the
// 32-token pieces of the teams head h drew, in team order) and runs the
// weighted online softmax for that head alone on the vector ALUs.
//   FUSED  the block first selects head h's teams itself (selection.h, the
//          same arithmetic as the selection kernel), so a decode call is this
//          kernel and the combine;
//   else   it reads the head's bitmap and log weights from the workspace
//          (santa_attend_selected after santa_select_teams).
// A team that several heads of a group drew is read by each of them; the
// blocks of one (group, range) are placed on the same XCD (consecutive
// slots, block i on XCD i mod 8) so that such repeated reads of a tile meet
// in that XCD's L2. Keys are loaded as whole 1 KB pieces of a 32-channel
// slab (four lanes per token, eight channels each, summed over the quad by
// DPP); values as whole 1 KB pieces of the channel-major value block (each
// lane eight tokens of one channel).
// ---------------------------------------------------------------------------
constexpr int kHeadWaves = 8;                     // wavefronts per per-head block
constexpr int kHeadMaxTeams = 512;                // page-table rows a per-head block handles

template <int D, int C>
struct HeadChunk {
    static constexpr int KL = (C / 16) * (D / 32); // 16-byte key loads per lane
    static constexpr int CH = 1024 / (2 * C);      // value channels per 1 KB load
    static constexpr int LPC = C / 8;              // lanes sharing one value channel
    static constexpr int VL = D / CH;              // 16-byte value loads per lane
    uint4 k[KL];
    uint4 v[VL];
};

template <int D>
struct HeadLds {
    double q64[D];
    double s[kHeadMaxTeams];                      // scores, then exp(s - m)
    double c[kHeadMaxTeams];                      // cumulative sums
    double pts[kHeadMaxTeams];                    // draw points (M < K <= kHeadMaxTeams when drawing)
    int32_t pt[kHeadMaxTeams];                    // page-table row
    uint32_t bits[kHeadMaxTeams / 32];
    int32_t spre[kHeadMaxTeams / 32 + 1];
    float lnw[kHeadMaxTeams];                     // log weight of each drawn team, by team (fused)
    float ipi[kHeadMaxTeams];                     // 1 / pi of each drawn team, by team (fused, sets requested)
    __attribute__((aligned(16))) float qf[D];     // the query in float32, for the token scores
    float pw[kHeadWaves][2][32];                  // a chunk's probabilities, per wavefront and buffer
    float mw[kHeadWaves], lw[kHeadWaves];        // per-wavefront maxima (scores, then logits) and sums
    float accw[kHeadWaves][D];
};

// One chunk of the head's list: its team, first token, valid tokens and
// tile offset (uniform over the wavefront).
struct HeadChunkDesc {
    int t, tb, n;
    size_t base;
};

template <int D, int C, bool FUSED>
__global__ __launch_bounds__(kHeadWaves * 64, 1) void santa_head_kernel(Params p) {
    constexpr int NW = kHeadWaves, NTH = NW * 64;
    using HC = HeadChunk<D, C>;
    using Pt = sel::Part<bf16_t, D>;
    constexpr int ROWS = NTH / sel::kParts;      // representative rows per scoring pass
    constexpr int PASSES = kHeadMaxTeams / ROWS;
    __shared__ HeadLds<D> lds;

    // Block -> slot ((group, range), head in group): the G heads of one
    // (group, range) sit on consecutive slots, hence on one XCD.
    const int S = p.max_splits;
    const int nreal = p.B * p.Hq * S;
    const int slot = int(blockIdx.x & 7) * int(gridDim.x >> 3) + int(blockIdx.x >> 3);
    if (slot >= nreal) return;
    const int gi = slot % p.G, rest = slot / p.G;
    const int j = rest % S, grp = rest / S;
    const int b = grp / p.Hkv, g = grp - b * p.Hkv;
    const int h = g * p.G + gi, bh = b * p.Hq + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Round trip 1: length, query, page-table row, and (fused) this
    // thread's part of every representative row it scores, or the head's
    // bitmap words.
    const int Lraw = p.seq_lens[b];
    const bf16_t *qg = static_cast<const bf16_t *>(p.q) + size_t(bh) * D;
    uint4 qv = make_uint4(0, 0, 0, 0);
    if (tid < D / 8) qv = ld16(qg + tid * 8);
    const int32_t ptv = tid < p.P ? p.page_table[size_t(b) * p.P + tid] : 0;
    const int row0 = tid / sel::kParts, part = tid % sel::kParts;
    uint4 raw[FUSED ? PASSES : 1][Pt::LOADS];
    uint32_t bw = 0u;
    const sel::TailArgs ta{0, p.M, p.scheme, p.seed_lo, p.seed_hi, p.offset, h, b};
    if constexpr (FUSED) {
        const bf16_t *reps = static_cast<const bf16_t *>(p.reps) + size_t(b) * p.P * p.Hkv * D;
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            const int row = row0 + ps * ROWS;
            if (row < p.P) sel::load_part<bf16_t, D>(reps + (size_t(row) * p.Hkv + g) * D, part, raw[ps]);
        }
        // Draw points while the rows are in flight (M < P <= kHeadMaxTeams
        // whenever they are used).
        if (p.M < p.P) sel::draw_points(ta, lds.pts, tid, NTH);
    } else {
        if (tid < p.words) bw = p.bitmaps[size_t(bh) * p.words + tid];
    }
    if (tid < D / 8) {
        float f[8];
        unpack(qv, f, bf16_t{});
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lds.q64[tid * 8 + e] = double(f[e]);
            lds.qf[tid * 8 + e] = f[e];
        }
    }
    if (tid < p.P) lds.pt[tid] = ptv;
    const int len = clamp_len(Lraw, p.P * p.T);
    const int K = (len + p.T - 1) / p.T;
    if constexpr (!FUSED) {
        if (tid < p.words) lds.bits[tid] = bw;
    }
    __syncthreads();

    if constexpr (FUSED) {
        // Scores (selection.h order; the query part stays in registers).
        double qp[Pt::N];
#pragma unroll
        for (int i = 0; i < Pt::N; ++i) qp[i] = lds.q64[part * Pt::N + i];
        float mx = -INFINITY;                                 // largest float32-rounded score of the thread's rows
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
            if (ps * ROWS >= K) break;                        // uniform
            const int t = row0 + ps * ROWS;
            const double sc = sel::row_score(sel::part_dot_raw<bf16_t, D>(raw[ps], qp), p.scale);
            if (part == 0 && t < K) {
                lds.s[t] = sc;
                mx = fmaxf(mx, float(sc));
            }
        }
        mx = sel::wave_max(mx);
        if (lane == 0) lds.mw[wave] = mx;
        __syncthreads();
        sel::team_exps(lds.s, K, lds.mw, NW, tid, NTH);
        __syncthreads();
    }

    // The head's drawn teams in order: rank rk is the team of the rk-th set
    // bit, found from the popcount prefix spre of the bitmap words.
    const int words = (K + 31) >> 5;
    const int cpt = p.T >= 32 ? p.T / 32 : 1;             // chunks per team
    const bool full = p.M >= K;
    auto team_of = [&](int rk) {
        int lo = 0, hi = words - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (lds.spre[mid] <= rk) lo = mid; else hi = mid - 1;
        }
        uint32_t u = lds.bits[lo];
        for (int k = rk - lds.spre[lo]; k > 0; --k) u &= u - 1u;
        return lo * 32 + __ffs(u) - 1;
    };
    // This block's chunks [c0, c1) of the head's ndrawn * cpt, and the ranks
    // of their teams.
    const bool out_sets = FUSED && p.sampled != nullptr;
    // Wavefront 0: the draws (fused; each drawing lane also stores its
    // team's weights), then the popcount prefix.
    if (wave == 0) {
        if constexpr (FUSED) {
            sel::TailArgs a = ta;
            a.K = K;
            sel::head_tail(lds.s, lds.c, lds.bits, lds.pts, a, lds.lnw, out_sets ? lds.ipi : nullptr);
        }
        const int cnt = lane < words ? __popc(lds.bits[lane]) : 0;
        const int ic = sel::wave_incl_scan(cnt);
        if (lane < words) lds.spre[lane] = ic - cnt;
        if (lane == 63) lds.spre[words] = ic;
    }
    __syncthreads();
    // This block's chunks [c0, c1) of the head's ndrawn * cpt (total * S <
    // 2^31: ndrawn <= 512, cpt <= 8, S <= 512).
    const int ndrawn = lds.spre[words];
    const int total = ndrawn * cpt;
    const int c0 = total * j / S, c1 = total * (j + 1) / S;
    if (out_sets && j == S - 1)
        for (int r = ndrawn + tid; r < p.M; r += NTH) {
            p.sampled[size_t(bh) * p.M + r] = -1;
            p.inv_pi[size_t(bh) * p.M + r] = 0.0f;
        }

    const float scale = float(p.scale);
    const float *lnw_g = p.lnw + size_t(bh) * p.P;
    const bf16_t *kbase = static_cast<const bf16_t *>(p.k_pages);
    const bf16_t *vbase = static_cast<const bf16_t *>(p.v_pages);

    // Chunk ci of the list: the (ci / cpt)-th drawn team, piece ci mod cpt.
    auto describe = [&](int ci) {
        const int rk = ci / cpt, piece = ci - rk * cpt;
        HeadChunkDesc d;
        d.t = team_of(rk);
        d.tb = piece * 32;
        d.n = min(p.T, len - d.t * p.T);
        d.base = (size_t(clamp_page(lds.pt[d.t], p.num_pages)) * p.Hkv + g) * size_t(p.T) * D + size_t(d.tb) * D;
        return d;
    };
    auto load = [&](const HeadChunkDesc &d, HC &ck) {
        const bf16_t *kc = kbase + d.base;
        const bf16_t *vc = vbase + d.base;
#pragma unroll
        for (int kk = 0; kk < HC::KL; ++kk) {
            const int r = kk / (D / 32), sl = kk % (D / 32);
            ck.k[kk] = ld16_stream(kc + sl * (C * 32) + (r * 16 + (lane >> 2)) * 32 + (lane & 3) * 8);
        }
#pragma unroll
        for (int vv = 0; vv < HC::VL; ++vv)
            ck.v[vv] = ld16_stream(vc + (vv * HC::CH + lane / HC::LPC) * C + (lane % HC::LPC) * 8);
    };
    // Log weight of the chunk's team (the selection kernel computes the same
    // value for the unfused call); a fused call also writes the team's entry
    // of the sorted set, from the block holding the team's first chunk.
    auto weight = [&](int ci, const HeadChunkDesc &d) {
        if constexpr (FUSED) {
            if (out_sets && d.tb == 0 && lane == 0) {
                p.sampled[size_t(bh) * p.M + ci / cpt] = d.t;
                p.inv_pi[size_t(bh) * p.M + ci / cpt] = full ? 1.0f : lds.ipi[d.t];
            }
            return full ? 0.0f : lds.lnw[d.t];
        } else {
            return lnw_g[d.t];
        }
    };

    float m = kNegInfF, lsum = 0.0f;
    float acc[HC::VL];
#pragma unroll
    for (int r = 0; r < HC::VL; ++r) acc[r] = 0.0f;
    // Scores, weighted online softmax and P V for one loaded chunk.
    auto compute = [&](const HeadChunkDesc &d, float lwt, const HC &ck, int buf) {
        float sc[C / 16];
        float cmax = kNegInfF;
#pragma unroll
        for (int r = 0; r < C / 16; ++r) {
            float a = 0.0f;
#pragma unroll
            for (int sl = 0; sl < D / 32; ++sl) {
                // the lane's query slice: channels 32 sl + 8 (lane % 4) + e
                const float4 q0 = *reinterpret_cast<const float4 *>(&lds.qf[sl * 32 + (lane & 3) * 8]);
                const float4 q1 = *reinterpret_cast<const float4 *>(&lds.qf[sl * 32 + (lane & 3) * 8 + 4]);
                const float qs[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                float f[8];
                unpack(ck.k[r * (D / 32) + sl], f, bf16_t{});
#pragma unroll
                for (int e = 0; e < 8; ++e) a = fmaf(f[e], qs[e], a);
            }
            a += __int_as_float(sel::dpp_i<sel::kQuadXor1, 0xF>(__float_as_int(a), 0));
            a += __int_as_float(sel::dpp_i<sel::kQuadXor2, 0xF>(__float_as_int(a), 0));
            const int tok = d.tb + r * 16 + (lane >> 2);
            sc[r] = tok < d.n ? a * scale + lwt : kNegInfF;
            cmax = fmaxf(cmax, sc[r]);
        }
        cmax = sel::wave_max(cmax);
        const float mnew = fmaxf(m, cmax);
        const float corr = (m == kNegInfF) ? 0.0f : __expf(m - mnew);
        float psum = 0.0f;
#pragma unroll
        for (int r = 0; r < C / 16; ++r) {
            const float pr = sc[r] == kNegInfF ? 0.0f : __expf(sc[r] - mnew);
            if ((lane & 3) == 0) {
                lds.pw[wave][buf][r * 16 + (lane >> 2)] = pr;
                psum += pr;
            }
        }
        psum = sel::wave_sum(psum);
        lsum = lsum * corr + psum;
        m = mnew;
        __builtin_amdgcn_wave_barrier();
        // Values: channel vv * CH + lane / LPC, tokens 8 (lane % LPC) + e.
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = lds.pw[wave][buf][(lane % HC::LPC) * 8 + e];
        const int keep = d.n - (d.tb + (lane % HC::LPC) * 8);      // valid tokens among this lane's 8
#pragma unroll
        for (int vv = 0; vv < HC::VL; ++vv) {
            float f[8];
            unpack(ck.v[vv], f, bf16_t{});
            float a = acc[vv] * corr;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaf(pe[e], e < keep ? f[e] : 0.0f, a);
            acc[vv] = a;
        }
    };

    // Two chunks in flight per wavefront: both are requested, then computed
    // in order.
    for (int ci = c0 + wave; ci < c1; ci += 2 * NW) {
        const int cj = ci + NW;
        const bool two = cj < c1;                                   // uniform
        HC ca, cb;
        const HeadChunkDesc da = describe(ci);
        load(da, ca);
        HeadChunkDesc db = da;
        if (two) {
            db = describe(cj);
            load(db, cb);
        }
        const float lwa = weight(ci, da);
        const float lwb = two ? weight(cj, db) : 0.0f;
        compute(da, lwa, ca, 0);
        if (two) compute(db, lwb, cb, 1);
        __builtin_amdgcn_wave_barrier();
    }

    // Wavefront partials: sum the LPC lanes of each channel, then merge the
    // wavefronts in order and store the block's partial.
#pragma unroll
    for (int vv = 0; vv < HC::VL; ++vv) {
        float a = acc[vv];
        a += __int_as_float(sel::dpp_i<sel::kQuadXor1, 0xF>(__float_as_int(a), 0));
        if (HC::LPC == 4) a += __int_as_float(sel::dpp_i<sel::kQuadXor2, 0xF>(__float_as_int(a), 0));
        if (lane % HC::LPC == 0) lds.accw[wave][vv * HC::CH + lane / HC::LPC] = a;
    }
    if (lane == 0) {
        lds.mw[wave] = m;
        lds.lw[wave] = lsum;
    }
    __syncthreads();
    if (tid < D) {
        float mx = kNegInfF;
        for (int w = 0; w < NW; ++w) mx = fmaxf(mx, lds.mw[w]);
        const size_t sl = size_t(bh) * p.slots + j;
        if (mx == kNegInfF) {
            if (tid == 0) write_empty_partial(p, bh, j);
        } else {
            float a = 0.0f, l = 0.0f;
            for (int w = 0; w < NW; ++w) {
                const float f = lds.mw[w] == kNegInfF ? 0.0f : expf(lds.mw[w] - mx);
                a += f * lds.accw[w][tid];
                l += f * lds.lw[w];
            }
            p.part_acc[sl * D + tid] = a;
            if (tid == 0) reinterpret_cast<float2 *>(p.part_ml)[sl] = make_float2(mx, l);
        }
    }
}

// ---------------------------------------------------------------------------
// Dense gather for batch >= 2 (bf16), with a plan chosen per launch from the
// sequence lengths (round trip 1, beside the per-group plan's own metadata).
//   Even lengths: the per-group plan of gather_balanced_kernel — block j
//     takes range j mod nb of the nb = max_splits even ranges of group
//     j / nb — whose metadata round trip is the first one, so it costs
//     nothing extra.
//   Ragged lengths (some group above 5/4 of the mean number of teams): one
//     even split of the chunks of all groups, in group order, over the grid,
//     so that long sequences do not finish last on a few blocks. A block
//     walks the groups its range [j C / nbe, (j + 1) C / nbe) overlaps
//     (usually one or two), each with a metadata round trip, the chunk loop
//     and a partial store; group X's partial from block j goes to slot
//     j - J(X), J(X) the block holding X's first chunk.
// Block 0 writes every group's slot count for the combine. (SANTA++ keeps
// the per-group plan: its union sizes are even enough that one split over
// all groups measured slower, its extra round trips outweighing the balance.)
// ---------------------------------------------------------------------------
constexpr int kRaggedNum = 5, kRaggedDen = 4;   // ragged: largest group > 5/4 of the mean

// The block whose range holds chunk c (ranges [j C / nbe, (j + 1) C / nbe)).
__device__ __forceinline__ int spread_block_of(int c, int total, int nbe) {
    return int(((int64_t(c) + 1) * nbe - 1) / total);
}

template <int D>
union DenseLds {
    struct {
        GroupChunks gc;
        __attribute__((aligned(16))) bf16_t q_lds[kGM][D + 8];
    } st;
    MfmaReduce<D> rd;                             // used by each partial store
};

// Chunks [lo, hi) of the group whose metadata is in lds (dense: every head
// takes every chunk with weight 1), merged into one partial at slot s.
template <int D>
__device__ __forceinline__ void dense_stream_range(const Params &p, DenseLds<D> &lds, int g, int hbase, int lo,
                                                   int hi, int s) {
    constexpr int NT = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i16 = lane & 15, g4 = lane >> 4;
    const int cpt = p.T >= 32 ? p.T / 32 : 1;
    GroupChunks &gc = lds.st.gc;
    float m = kNegInfF, lsum = 0.0f;
    f32x4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w0 = lo; w0 < hi; w0 += kWin) {
        const int cnt = min(kWin, hi - w0);
        chunk_window(p, gc, cpt, w0, cnt);
        for (int q = wave; q < cnt; q += kWaves) {
            const bool drew = (gc.mask[q] >> i16) & 1u;
            MfmaChunk<D> ck;
            mfma_load_chunk_at<D>(p, gc.page[q], gc.n[q], gc.tb[q], g, i16, g4, ck);
            mfma_compute_chunk_at<D>(p, gc.n[q], gc.tb[q], drew ? 0.0f : kNegInfF, i16, g4, lds.st.q_lds, ck, m,
                                     lsum, o);
        }
        __syncthreads();                          // the window is reused
    }
    mfma_store_partial<D>(p, lds.rd, m, lsum, o, hbase, s);
}

template <int D>
__global__ __launch_bounds__(kBlock, 3) void gather_dense_spread_kernel(Params p) {
    __shared__ DenseLds<D> lds;
    __shared__ int32_t ucnt[kMaxSpreadGroups];          // teams of each group
    __shared__ int32_t ustart[kMaxSpreadGroups + 1];    // first chunk of each group; [ngroups] = all chunks
    __shared__ int32_t ragged_s;
    GroupChunks &gc = lds.st.gc;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ngroups = p.B * p.Hkv;
    const int cpt = p.T >= 32 ? p.T / 32 : 1;
    const int j = blockIdx.x, nb = p.max_splits;
    const int xe = min(j / nb, ngroups - 1);             // the block's group in the per-group plan
    const int be = xe / p.Hkv, ge = xe - be * p.Hkv;

    // Round trip 1: every group's team count, and the per-group plan's
    // query rows, page-table row and length.
    for (int x = tid; x < ngroups; x += kBlock) {
        const int L = clamp_len(p.seq_lens[x / p.Hkv], p.P * p.T);
        ucnt[x] = (L + p.T - 1) / p.T;
    }
    fill_q_lds<D>(p, lds.st.q_lds, be * p.Hq + ge * p.G);
    group_load(p, gc, ge, be);                           // ends with a barrier
    if (wave == 0) {
        // Exclusive prefix of chunk counts (four consecutive groups per lane)
        // and the largest group.
        constexpr int PER = kMaxSpreadGroups / 64;
        int v[PER], sum = 0, mx = 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int x = lane * PER + k;
            v[k] = x < ngroups ? ucnt[x] * cpt : 0;
            sum += v[k];
            mx = max(mx, v[k]);
        }
        int incl = sum;
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (lane >= off) incl += y;
        }
        for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
        int run = incl - sum;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int x = lane * PER + k;
            if (x < ngroups) ustart[x] = run;
            run += v[k];
        }
        if (lane == 63) {
            ustart[ngroups] = incl;
            ragged_s = int64_t(mx) * ngroups * kRaggedDen > int64_t(incl) * kRaggedNum;
        }
    }
    __syncthreads();
    const int total = ustart[ngroups];
    const bool ragged = ragged_s != 0;
    const int nbe = min(min(int(gridDim.x), p.slots), total);   // a group's slots stay below p.slots
    if (j == 0)
        for (int x = tid; x < ngroups; x += kBlock)
            p.grp_slots[x] = !ragged ? nb
                             : ucnt[x] == 0 ? 0
                                            : spread_block_of(ustart[x + 1] - 1, total, nbe) -
                                                  spread_block_of(ustart[x], total, nbe) + 1;

    if (!ragged) {
        if (j / nb >= ngroups) return;                   // no such block in the per-group grid
        const int U = group_scan(p, gc);
        const int jl = j - xe * nb, all = U * cpt;
        dense_stream_range<D>(p, lds, ge, be * p.Hq + ge * p.G, int(int64_t(all) * jl / nb),
                              int(int64_t(all) * (jl + 1) / nb), jl);
        return;
    }
    if (j >= nbe) return;
    const int c0 = int(int64_t(total) * j / nbe), c1 = int(int64_t(total) * (j + 1) / nbe);
    int x = 0;                                           // the last group starting at or before c0
    {
        int lo = 0, hi = ngroups - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ustart[mid] <= c0) lo = mid; else hi = mid - 1;
        }
        x = lo;
    }
    for (; x < ngroups && ustart[x] < c1; ++x) {
        if (ustart[x + 1] == ustart[x]) continue;          // no chunk in this group
        const int b = x / p.Hkv, g = x - b * p.Hkv;
        const int hbase = b * p.Hq + g * p.G;
        __syncthreads();                                     // LDS is free again (previous store, plan reads)
        fill_q_lds<D>(p, lds.st.q_lds, hbase);
        const int U = group_union(p, gc, g, b);
        const int lo = max(c0, ustart[x]) - ustart[x];
        const int hi = min(min(c1, ustart[x + 1]) - ustart[x], U * cpt);
        dense_stream_range<D>(p, lds, g, hbase, lo, hi, j - spread_block_of(ustart[x], total, nbe));
    }
}

// ---------------------------------------------------------------------------
// float32 gather: scores in float64 (products of two float32 values are exact
// in float64), one team at a time with block-wide steps. Used for float32
// caches, where the 1e-5 output tolerance needs more than float32 scores.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kBlock) void gather_f32_kernel(Params p) {
    constexpr int PARTS = kBlock / D;                   // token subsets per channel
    constexpr int kMaxT = 256;
    __shared__ TeamList tl;
    __shared__ float q_s[kGM][D];
    __shared__ double m_s[kGM], l_s[kGM], corr_s[kGM];
    // Scores / weights of the current team, reused at the end for the
    // per-part value sums (both 32 KiB).
    __shared__ double buf[kGM * kMaxT];
    static_assert(PARTS * kGM * D <= kGM * kMaxT, "reduction buffer fits the score buffer");

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int G = p.G;
    const int hbase = b * p.Hq + g * G;
    const float *qg = static_cast<const float *>(p.q) + size_t(hbase) * D;
    for (int i = tid; i < kGM * D; i += kBlock) q_s[i / D][i % D] = (i / D < G) ? qg[i] : 0.0f;
    if (tid < kGM) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.0;
    }
    const int nteams = p.ranked ? load_ranked_team_list(p, tl, s, g, b) : load_team_list(p, tl, s, g, b);
    if (nteams == 0) {
        if (p.ranked && tid < G) write_empty_partial(p, hbase + tid, s);
        return;
    }

    double (*sc)[kMaxT] = reinterpret_cast<double (*)[kMaxT]>(buf);
    const int c = tid % D, part = tid / D;
    double acc[kGM];
#pragma unroll
    for (int h = 0; h < kGM; ++h) acc[h] = 0.0;

    for (int ti = 0; ti < nteams; ++ti) {
        const int n = tl.n[ti];
        const size_t tile = (size_t(tl.page[ti]) * p.Hkv + g) * size_t(p.T) * D;
        const float *kt = static_cast<const float *>(p.k_pages) + tile;
        const float *vt = static_cast<const float *>(p.v_pages) + tile;
        for (int idx = tid; idx < n * G; idx += kBlock) {
            const int j = idx / G, h = idx - j * G;
            const float lw = tl.lnw[ti][h];
            if (lw == kNegInfF) {
                sc[h][j] = -INFINITY;
                continue;
            }
            double dot = 0.0;
            for (int c0 = 0; c0 < D; c0 += 4) {
                const uint4 r = ld16(kt + k_offset(j, c0, p.T, D));
                dot = fma(double(__uint_as_float(r.x)), double(q_s[h][c0 + 0]), dot);
                dot = fma(double(__uint_as_float(r.y)), double(q_s[h][c0 + 1]), dot);
                dot = fma(double(__uint_as_float(r.z)), double(q_s[h][c0 + 2]), dot);
                dot = fma(double(__uint_as_float(r.w)), double(q_s[h][c0 + 3]), dot);
            }
            sc[h][j] = dot * p.scale + double(lw);
        }
        __syncthreads();
        if (tid < G) {
            const int h = tid;
            if (tl.lnw[ti][h] == kNegInfF) {
                corr_s[h] = 1.0;
            } else {
                double tm = -INFINITY;
                for (int j = 0; j < n; ++j) tm = fmax(tm, sc[h][j]);
                const double mn = fmax(m_s[h], tm);
                corr_s[h] = (m_s[h] == -INFINITY) ? 0.0 : exp(m_s[h] - mn);
                m_s[h] = mn;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < n * G; idx += kBlock) {
            const int j = idx / G, h = idx - j * G;
            sc[h][j] = (tl.lnw[ti][h] == kNegInfF) ? 0.0 : exp(sc[h][j] - m_s[h]);
        }
        __syncthreads();
        if (tid < G) {
            double sum = 0.0;
            for (int j = 0; j < n; ++j) sum += sc[tid][j];
            l_s[tid] = l_s[tid] * corr_s[tid] + sum;
        }
#pragma unroll
        for (int h = 0; h < kGM; ++h)
            if (h < G) acc[h] *= corr_s[h];
        for (int j = part; j < n; j += PARTS) {
            const double v = double(vt[v_offset(j, c, p.T, D)]);
#pragma unroll
            for (int h = 0; h < kGM; ++h)
                if (h < G) acc[h] = fma(sc[h][j], v, acc[h]);
        }
        __syncthreads();
    }
    double (*red)[kGM][D] = reinterpret_cast<double (*)[kGM][D]>(buf);
#pragma unroll
    for (int h = 0; h < kGM; ++h)
        if (h < G) red[part][h][c] = acc[h];
    __syncthreads();
    float2 *part_ml = reinterpret_cast<float2 *>(p.part_ml);
    for (int idx = tid; idx < G * D; idx += kBlock) {
        const int h = idx / D, cc = idx - h * D;
        const size_t slot = size_t(hbase + h) * p.slots + s;
        if (m_s[h] == -INFINITY) {             // the head drew no team of this split
            if (p.ranked && cc == 0) write_empty_partial(p, hbase + h, s);
            continue;
        }
        double a = 0.0;
        for (int pp = 0; pp < PARTS; ++pp) a += red[pp][h][cc];
        // Store relative to the float32-rounded max the partial is labelled with.
        const float mstore = float(m_s[h]);
        const double f = exp(m_s[h] - double(mstore));
        p.part_acc[slot * D + cc] = float(a * f);
        if (cc == 0) part_ml[slot] = make_float2(mstore, float(l_s[h] * f));
    }
}

// ---------------------------------------------------------------------------
// combine: one 256-thread block per (sequence, query head). The head's bitmap
// says which split slots hold its partials; they are merged in slot order:
//   out = sum_s e^{m_s - m*} acc_s / sum_s e^{m_s - m*} l_s,
//   lse = m* + log(sum_s e^{m_s - m*} l_s).
// Two round trips: (sequence length, bitmap, every slot's (max, sum)), then
// the value sums of the slots that hold partials, as float4, all at once.
// ---------------------------------------------------------------------------
constexpr int kCombine = 256;
constexpr int kFew = 8;                            // value quads per thread of the one-round-trip combine

template <int D>
__global__ __launch_bounds__(kCombine) void combine_kernel(Params p) {
    constexpr int Q4 = D / 4;                      // float4 quads per row
    constexpr int SUB = kCombine / Q4;             // split subsets (8 at d = 128, 16 at d = 64)
    constexpr int PER = kMaxTeams / kCombine;      // slots per thread at most
    constexpr int W = kCombine / 64;
    constexpr int BATCH = 8;
    __shared__ uint32_t hw_s[kMaxWords];
    __shared__ int32_t list_s[kMaxTeams];
    __shared__ float f_s[kMaxTeams];
    __shared__ float redf[W];
    __shared__ int32_t redi[W];
    __shared__ float4 acc_s[SUB][Q4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x;
    const int b = bh / p.Hq;
    const bool dense = p.mode == kModeDense;
    const float2 *ml = reinterpret_cast<const float2 *>(p.part_ml) + size_t(bh) * p.slots;
    const float4 *pacc = reinterpret_cast<const float4 *>(p.part_acc + size_t(bh) * p.slots * D);
    const int c4 = tid % Q4, sb = tid / Q4;
    // Slots of this head's group: written by the spread gather, else every
    // slot below max_splits.
    const int nsp = p.spread ? p.grp_slots[b * p.Hkv + (bh - b * p.Hq) / p.G] : p.max_splits;

    if (p.max_splits <= kFew * SUB) {
        // Few slots (every balanced split at batch >= 1 up to 64 / 128 slots):
        // one round trip. Every slot's (max, sum) and this thread's quads of
        // every slot's value sum are loaded at once; slots that hold no
        // partial of this call get weight 0 and their values are never used.
        __shared__ float2 ml_s[kFew * SUB];
        // Every load into registers first (one round trip), then into LDS.
        const int Lraw = p.seq_lens[b];
        uint32_t hwv = 0u;
        if (!dense && !p.ranked && tid < p.words) hwv = p.bitmaps[size_t(bh) * p.words + tid];
        float2 mlv = make_float2(kNegInfF, 0.0f);
        if (tid < p.max_splits) mlv = ml[tid];
        float4 x[kFew];
#pragma unroll
        for (int u = 0; u < kFew; ++u) {
            const int sp = sb + u * SUB;
            x[u] = (sp < p.max_splits) ? pacc[size_t(sp) * Q4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (!dense && !p.ranked && tid < p.words) hw_s[tid] = hwv;
        if (tid < p.max_splits) ml_s[tid] = mlv;
        __syncthreads();
        if (nsp <= p.max_splits) {                // uniform; else the slot count needs the general path
            // Every wavefront forms m* and l itself (DPP, the same order in
            // each), so no wavefront waits for another before its sums.
            const int L = clamp_len(Lraw, p.P * p.T);
            const int K = (L + p.T - 1) / p.T;
            const int nslots = (K + p.tps - 1) / p.tps;
            const uint32_t low = (p.tps >= 32) ? 0xffffffffu : ((1u << p.tps) - 1u);
            auto holds = [&](int sp) {            // slot sp holds a partial of this head
                if (sp >= nsp) return false;
                if (p.ranked) return ml_s[sp].x != kNegInfF;
                if (sp >= nslots) return false;
                if (dense) return true;
                const int t0 = sp * p.tps;
                return ((hw_s[t0 >> 5] >> (t0 & 31)) & low) != 0u;
            };
            float mv[2];
            bool ok[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int sp = lane + 64 * i;
                ok[i] = holds(sp);
                mv[i] = ok[i] ? ml_s[sp].x : kNegInfF;
            }
            const float mstar = sel::wave_max(fmaxf(mv[0], mv[1]));
            if (mstar == kNegInfF) {                  // no partial: empty sequence
                for (int c = tid; c < D; c += kCombine) p.out[size_t(bh) * D + c] = 0.0f;
                if (tid == 0 && p.lse) p.lse[bh] = kNegInfF;
                return;
            }
            float lpart = 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (ok[i]) lpart += expf(mv[i] - mstar) * ml_s[lane + 64 * i].y;
            const float l = sel::wave_sum(lpart);
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < kFew; ++u) {
                const int sp = sb + u * SUB;
                if (sp < p.max_splits && holds(sp)) {
                    const float f = expf(ml_s[sp].x - mstar);
                    a.x += f * x[u].x; a.y += f * x[u].y; a.z += f * x[u].z; a.w += f * x[u].w;
                }
            }
            acc_s[sb][c4] = a;
            __syncthreads();
            if (tid < Q4) {
                float4 sum = acc_s[0][tid];
                for (int i = 1; i < SUB; ++i) {
                    const float4 y = acc_s[i][tid];
                    sum.x += y.x; sum.y += y.y; sum.z += y.z; sum.w += y.w;
                }
                const float inv = 1.0f / l;
                reinterpret_cast<float4 *>(p.out + size_t(bh) * D)[tid] =
                    make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
                if (tid == 0 && p.lse) p.lse[bh] = mstar + logf(l);
            }
            return;
        }
    }

    // Round trip 1. Slot (max, sum) values are read for every slot that can
    // exist (all inside the workspace); stale ones are ignored below.
    const int Lraw = p.seq_lens[b];
    if (!dense && !p.ranked && tid < p.words) hw_s[tid] = p.bitmaps[size_t(bh) * p.words + tid];
    const int nslots_max = p.spread ? nsp : p.max_splits;
    float2 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int sp = tid * PER + i;
        v[i] = (sp < nslots_max) ? ml[sp] : make_float2(kNegInfF, 0.0f);
    }
    __syncthreads();
    const int L = clamp_len(Lraw, p.P * p.T);
    const int K = (L + p.T - 1) / p.T;
    const int nslots = (K + p.tps - 1) / p.tps;
    const uint32_t low = (p.tps >= 32) ? 0xffffffffu : ((1u << p.tps) - 1u);

    // Slots holding this head's partials (thread tid owns slots tid*PER ...),
    // their running max, and their positions in the compact list.
    int cnt = 0;
    float mloc = kNegInfF;
    bool has[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int sp = tid * PER + i;
        bool hv;
        if (p.ranked) {
            hv = sp < nslots_max && v[i].x != kNegInfF;
        } else {
            hv = sp < nslots;
            if (hv && !dense) {
                const int t0 = sp * p.tps;
                hv = ((hw_s[t0 >> 5] >> (t0 & 31)) & low) != 0u;
            }
        }
        has[i] = hv;
        cnt += hv ? 1 : 0;
        if (hv) mloc = fmaxf(mloc, v[i].x);
    }
    int incl = cnt;
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off, 64));
    if (lane == 63) redi[wave] = incl;
    if (lane == 0) redf[wave] = mloc;
    __syncthreads();
    int base = 0, total = 0;
    float mstar = kNegInfF;
    for (int w = 0; w < W; ++w) {
        if (w < wave) base += redi[w];
        total += redi[w];
        mstar = fmaxf(mstar, redf[w]);
    }
    if (total == 0) {
        for (int c = tid; c < D; c += kCombine) p.out[size_t(bh) * D + c] = 0.0f;
        if (tid == 0 && p.lse) p.lse[bh] = kNegInfF;
        return;
    }
    int pos = base + incl - cnt;
    float lpart = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (!has[i]) continue;
        const float f = expf(v[i].x - mstar);
        list_s[pos] = tid * PER + i;
        f_s[pos] = f;
        lpart += f * v[i].y;
        ++pos;
    }
    for (int off = 32; off > 0; off >>= 1) lpart += __shfl_xor(lpart, off, 64);
    __syncthreads();
    if (lane == 0) redf[wave] = lpart;

    // Round trip 2: value sums, thread (quad c4, subset sb) takes list
    // entries sb, sb + SUB, ... in batches whose loads are all issued first.
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = sb; k0 < total; k0 += BATCH * SUB) {
        float4 x[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int k = k0 + u * SUB;
            x[u] = (k < total) ? pacc[size_t(list_s[k]) * Q4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int k = k0 + u * SUB;
            const float f = (k < total) ? f_s[k] : 0.0f;
            a.x += f * x[u].x; a.y += f * x[u].y; a.z += f * x[u].z; a.w += f * x[u].w;
        }
    }
    acc_s[sb][c4] = a;
    __syncthreads();
    float l = 0.0f;
    for (int w = 0; w < W; ++w) l += redf[w];
    if (tid < Q4) {
        float4 sum = acc_s[0][tid];
        for (int i = 1; i < SUB; ++i) {
            const float4 y = acc_s[i][tid];
            sum.x += y.x; sum.y += y.y; sum.z += y.z; sum.w += y.w;
        }
        const float inv = 1.0f / l;
        reinterpret_cast<float4 *>(p.out + size_t(bh) * D)[tid] =
            make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
        if (tid == 0 && p.lse) p.lse[bh] = mstar + logf(l);
    }
}

}  // namespace

santa_status launch_gather(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(p.max_splits, p.Hkv, p.B);
    if (p.dtype == SANTA_BF16 && p.balanced && p.spread && p.mode == kModeDense) {
        const dim3 sgrid(p.max_splits * p.Hkv * p.B);
        if (p.d == 64) hipLaunchKernelGGL((gather_dense_spread_kernel<64>), sgrid, dim3(kBlock), 0, st, p);
        else hipLaunchKernelGGL((gather_dense_spread_kernel<128>), sgrid, dim3(kBlock), 0, st, p);
    } else if (p.dtype == SANTA_BF16 && p.balanced) {
        if (p.mode == kModeDense) {
            if (p.d == 64) hipLaunchKernelGGL((gather_balanced_kernel<64, kModeDense>), grid, dim3(kBlock), 0, st, p);
            else hipLaunchKernelGGL((gather_balanced_kernel<128, kModeDense>), grid, dim3(kBlock), 0, st, p);
        } else {
            if (p.per_head) {
                // One block per (head, range) slot, rounded up to whole XCD rounds.
                const int64_t nh = int64_t(p.B) * p.Hq * p.max_splits;
                const dim3 hgrid(unsigned((nh + 7) / 8 * 8)), hblock(kHeadWaves * 64);
                const bool c16 = p.T < 32;
#define SANTA_HEAD_LAUNCH(DD, CC)                                                                               \
    if (p.fused) hipLaunchKernelGGL((santa_head_kernel<DD, CC, true>), hgrid, hblock, 0, st, p);                \
    else hipLaunchKernelGGL((santa_head_kernel<DD, CC, false>), hgrid, hblock, 0, st, p);
                if (p.d == 64) {
                    if (c16) { SANTA_HEAD_LAUNCH(64, 16) } else { SANTA_HEAD_LAUNCH(64, 32) }
                } else {
                    if (c16) { SANTA_HEAD_LAUNCH(128, 16) } else { SANTA_HEAD_LAUNCH(128, 32) }
                }
#undef SANTA_HEAD_LAUNCH
                return launched();
            }
            // One block per (group, range) slot, rounded up to whole XCD rounds.
            const int64_t n = int64_t(p.B) * p.Hkv * p.max_splits;
            const dim3 sgrid(unsigned((n + 7) / 8 * 8)), block(kSantaWaves * 64);
            if (p.d == 64) hipLaunchKernelGGL((santa_gather_kernel<64, kSantaWaves>), sgrid, block, 0, st, p);
            else hipLaunchKernelGGL((santa_gather_kernel<128, kSantaWaves>), sgrid, block, 0, st, p);
        }
    } else if (p.dtype == SANTA_BF16) {
        return SANTA_ERR_UNSUPPORTED;             // bf16 caches always take balanced blocks
    } else {
        if (p.d == 64) hipLaunchKernelGGL((gather_f32_kernel<64>), grid, dim3(kBlock), 0, st, p);
        else hipLaunchKernelGGL((gather_f32_kernel<128>), grid, dim3(kBlock), 0, st, p);
    }
    return launched();
}

santa_status launch_combine(const Params &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.d == 64) hipLaunchKernelGGL((combine_kernel<64>), dim3(p.B * p.Hq), dim3(kCombine), 0, st, p);
    else hipLaunchKernelGGL((combine_kernel<128>), dim3(p.B * p.Hq), dim3(kCombine), 0, st, p);
    return launched();
}

}  // namespace santa
