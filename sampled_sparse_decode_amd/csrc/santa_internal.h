// Internal interface between the host entry points (santa_api.cpp) and the
// HIP kernels (reps.hip, select.hip, gather.hip, pack.hip, cluster.hip).
// Not installed; not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/santa.h"

namespace santa {

constexpr int kMaxTeams = 2048;        // max_pages_per_seq limit (LDS-resident scan)
constexpr int kMaxWords = kMaxTeams / 32;
constexpr int kMaxGroup = 16;          // query heads per KV head
constexpr int kMaxTeamsPerSplit = 16;
constexpr int kSantaWaves = 8;         // wavefronts per SANTA++ union-gather block (bfloat16)
constexpr int kPerHeadMaxTeams = 512;  // per-head gather: page-table rows at most
constexpr int kPerHeadMaxHeads = 64;   // per-head gather: (sequence, query head) pairs per call at most
constexpr int kVsMaxTokens = 16384;    // value samples: drawn tokens per head at most (min(M, P) * T)
constexpr int kVsMaxSamples = 256;     // value samples per head at most
constexpr int kVsChunk = 512;          // value samples: drawn tokens per logit block (a multiple of every T)
constexpr int kVsMaxChunks = kVsMaxTokens / kVsChunk;

enum Mode : int32_t { kModeSanta = 0, kModeDense = 1 };

// Byte offsets of the workspace sections (all 256-byte aligned).
struct WorkspaceLayout {
    size_t bitmaps;     // uint32 [B][Hq][words]      team bitmap of each query head
    size_t lnw;         // float  [B][Hq][P]          log weight of each drawn team
    size_t part_ml;     // float2 [B][Hq][slots]      split partial (max, sum)
    size_t part_acc;    // float  [B][Hq][slots][d]   split partial weighted value sums
    size_t grp_slots;   // int32  [B][Hkv]            partial slots of each group (spread gather)
    size_t total;
    int32_t words;      // ceil(P / 32)
    int32_t max_splits; // P
    int32_t slots;      // partial slots per head: P (float32), max(P, kSpreadBlocks) (bfloat16)
};

// Dense gather of a ragged batch (bfloat16, batch >= 2): one even split of all
// groups' chunks over the grid, at most max(P, kSpreadBlocks) blocks meeting a
// group; used while the groups fit its plan.
constexpr int kSpreadBlocks = 256;
constexpr int kMaxSpreadGroups = 256;

WorkspaceLayout workspace_layout(const santa_kv &kv);
// Value samples: the selection's sections, then the running sums, chunk
// pairs and piece ends over the (unused) partial sections; returns the bytes
// and the three offsets.
size_t value_workspace_layout(const santa_kv &kv, int32_t M, size_t *cs_off, size_t *sum_off, size_t *piece_off,
                              int32_t *chunks);
// The same sections with `slots` partial slots per head (the splits one
// launch uses), for a workspace sized to a single call.
WorkspaceLayout workspace_layout(const santa_kv &kv, int32_t slots);

// Device scratch of santa_decode_attention_noalloc (noalloc.hip): the
// address of the file-scope array on the device of `stream` (the current
// device for the NULL stream), looked up once per device.
constexpr size_t kNoallocScratchBytes = SANTA_NOALLOC_SCRATCH_BYTES;
santa_status noalloc_scratch(void *stream, void **ptr);

// Everything a kernel launch needs, passed by value.
struct Params {
    const void *k_pages;
    const void *v_pages;
    const void *q;
    const void *reps;
    const int32_t *page_table;
    const int32_t *seq_lens;
    int64_t num_pages;
    int32_t dtype;
    int32_t B, Hq, Hkv, G, d, T, P, words;
    int32_t M;
    uint32_t seed_lo, seed_hi, offset;
    int32_t mode;           // Mode
    int32_t tps;            // union teams per split-K block
    int32_t max_splits;     // gather grid.x
    int32_t ranked;         // 1: every split slot < max_splits gets a (max, sum) pair, -inf if empty
    int32_t balanced;       // 1 (bf16 only): block j takes the j-th of max_splits even ranges of union chunks
    int32_t spread;         // 1 (bf16 dense, batch >= 2): per-launch plan, per group or over all groups
    int32_t slots;          // partial slots per head (stride of part_ml / part_acc)
    int32_t *grp_slots;     // spread: [B][Hkv] partial slots written for each group
    double scale;           // 1 / sqrt(d)
    uint32_t *bitmaps;
    float *lnw;
    float *part_ml;         // float2 pairs
    float *part_acc;
    float *out;
    float *lse;
    int32_t *sampled;
    float *inv_pi;
    const int32_t *given_teams;
    const float *given_w;
    void *reps_out;
    const int32_t *prev_lens;   // build_reps update mode: lengths before the append (NULL: rebuild all)
    int32_t update_teams;       // update mode: teams refreshed per sequence at most
    int32_t rep_kind;           // santa_rep_kind of build_reps launches (seed_lo/hi key the random kind)
    int32_t scheme;             // santa_draw_scheme of select launches
    int32_t per_head;           // 1 (bf16): blocks per (head, range), each head streaming its own teams
    int32_t fused;              // per-head blocks select their head's teams themselves (one-launch decode)
    int32_t vs_samples;         // value samples per head (santa_decode_attention_value_sampled)
    int32_t vs_scheme;          // santa_draw_scheme of the value samples
    int32_t *vs_positions;      // [B][Hq][vs_samples] sampled token positions, or NULL
    int32_t vs_chunks;          // logit blocks per head: ceil(min(M, P) T / kVsChunk)
    double *vs_cs;              // [B][Hq][vs_chunks * kVsChunk] running sums inside each chunk
    double *vs_sum;             // [B][Hq][vs_chunks] (max, sum) pairs of the chunks
    double *vs_piece;           // [B][Hq][vs_chunks][kVsChunk / 16] running sum at each 16-token piece's end
};

constexpr uint32_t kRepKeyXor = 0x52455053u;   // random representatives: key word 0 = seed lo ^ this

// Arguments of the append kernel (santa_append_kv).
struct AppendParams {
    const void *k_new;
    const void *v_new;
    void *k_pages;
    void *v_pages;
    const int32_t *page_table;
    const int32_t *seq_lens;     // new lengths
    const int32_t *prev_lens;    // lengths before the append
    int64_t num_pages;
    int32_t dtype, B, P, Hkv, T, d, max_new;
};

// santa_pack_pages arguments.
struct PackParams {
    const void *k_src;
    const void *v_src;
    void *k_dst;
    void *v_dst;
    int64_t tiles;          // num_pages * Hkv
    int32_t dtype, T, d;
};

// santa_pack_pages_hashed arguments.
constexpr int kMaxHashBits = 10;
struct ClusterParams {
    const void *k_src;          // plain pages [num_pages][Hkv][T][d]
    const void *v_src;
    void *k_dst;                // tile-order pages [num_pages][Hkv][T * d]
    void *v_dst;
    const float *directions;    // [Hkv][bits][d]
    const int32_t *page_table;
    const int32_t *seq_lens;
    int32_t *codes;             // [B][Hkv][P * T]
    int32_t *token_of;          // [B][Hkv][P * T]
    int64_t num_pages;
    int32_t dtype, B, Hkv, P, T, d, bits;
    // k-means partition (workspace sections; NULL for the hash partition)
    double *mu;                 // [B][Hkv][cmax][d] centroids
    double *half;               // [B][Hkv][cmax] |mu|^2 / 2 terms (the sums, halved at use)
    int32_t *starts;            // [B][Hkv][2^bits + 1] first sorted position of each code
    int32_t clusters;           // requested clusters per sequence (0: one per team)
    int32_t cmax;               // allocated clusters per (sequence, KV head)
};

constexpr int kMaxClusters = 1 << 10;      // codes must fit the counting sort
constexpr int kMaxKmeansIters = 1000;

// Host-side argument checks; no HIP calls.
santa_status validate_kv(const santa_kv *kv);

// Kernel launches. Each returns SANTA_OK or SANTA_ERR_HIP.
santa_status launch_build_reps(const Params &p, void *stream);
santa_status launch_select(const Params &p, void *stream);
santa_status launch_given(const Params &p, void *stream);
santa_status launch_gather(const Params &p, void *stream);
santa_status launch_combine(const Params &p, void *stream);
santa_status launch_value_sample(const Params &p, void *stream);
santa_status launch_pack_pages(const PackParams &pp, void *stream);
santa_status launch_append_kv(const AppendParams &ap, void *stream);
santa_status launch_pack_hashed(const ClusterParams &c, void *stream);
santa_status launch_pack_kmeans(const ClusterParams &c, int32_t iters, void *stream);

}  // namespace santa
