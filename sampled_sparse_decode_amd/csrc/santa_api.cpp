// C-ABI entry points of libsanta: argument validation, workspace carve-up,
// split sizing and the launch sequence of each operation. Validation runs
// before any HIP call so that bad arguments return a status without touching
// the device.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "santa_internal.h"

namespace santa {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

santa_status validate_kv(const santa_kv *kv) {
    if (!kv) return SANTA_ERR_NULL;
    if (kv->dtype != SANTA_F32 && kv->dtype != SANTA_BF16) return SANTA_ERR_UNSUPPORTED;
    if (kv->batch < 1 || kv->batch > 65535) return SANTA_ERR_SHAPE;
    if (kv->num_q_heads < 1 || kv->num_kv_heads < 1) return SANTA_ERR_SHAPE;
    if (kv->num_q_heads % kv->num_kv_heads != 0) return SANTA_ERR_SHAPE;
    if (kv->num_q_heads / kv->num_kv_heads > kMaxGroup) return SANTA_ERR_UNSUPPORTED;
    if (kv->head_dim != 64 && kv->head_dim != 128) return SANTA_ERR_UNSUPPORTED;
    const int T = kv->page_size;
    if (T != 16 && T != 32 && T != 64 && T != 128 && T != 256) return SANTA_ERR_UNSUPPORTED;
    if (kv->max_pages_per_seq < 1 || kv->max_pages_per_seq > kMaxTeams) return SANTA_ERR_SHAPE;
    if (kv->reserved != 0) return SANTA_ERR_SHAPE;
    if (kv->num_pages < 1) return SANTA_ERR_SHAPE;
    if (!kv->k_pages || !kv->v_pages || !kv->page_table || !kv->seq_lens) return SANTA_ERR_NULL;
    return SANTA_OK;
}

WorkspaceLayout workspace_layout(const santa_kv &kv) {
    return workspace_layout(kv, kv.dtype == SANTA_BF16 ? std::max<int32_t>(kv.max_pages_per_seq, kSpreadBlocks)
                                                       : kv.max_pages_per_seq);
}

WorkspaceLayout workspace_layout(const santa_kv &kv, int32_t slots) {
    WorkspaceLayout w{};
    const size_t B = kv.batch, Hq = kv.num_q_heads, P = kv.max_pages_per_seq, d = kv.head_dim;
    w.words = (kv.max_pages_per_seq + 31) / 32;
    w.max_splits = kv.max_pages_per_seq;
    w.slots = slots;
    const size_t S = size_t(w.slots);
    size_t off = 0;
    w.bitmaps = off;   off = align256(off + B * Hq * size_t(w.words) * 4);
    w.lnw = off;       off = align256(off + B * Hq * P * 4);
    w.part_ml = off;   off = align256(off + B * Hq * S * 8);
    w.part_acc = off;  off = align256(off + B * Hq * S * d * 4);
    w.grp_slots = off; off = align256(off + size_t(kv.batch) * kv.num_kv_heads * 4);
    w.total = off;
    return w;
}

// Teams per split-K block of the float32 path: a power of two (so a block's
// teams share one bitmap word), at most 16, giving about `target` blocks.
static int32_t teams_per_split(int64_t team_slots, int64_t target) {
    int32_t tps = 1;
    while (tps < kMaxTeamsPerSplit && int64_t(tps) * 2 * target <= team_slots) tps *= 2;
    return tps;
}

size_t value_workspace_layout(const santa_kv &kv, int32_t M, size_t *cs_off, size_t *sum_off, size_t *piece_off,
                              int32_t *chunks) {
    const WorkspaceLayout w = workspace_layout(kv);
    const int64_t tokens = int64_t(std::min(M, kv.max_pages_per_seq)) * kv.page_size;
    const int64_t nc = (tokens + kVsChunk - 1) / kVsChunk;
    const size_t heads = size_t(kv.batch) * kv.num_q_heads;
    *chunks = int32_t(nc);
    *cs_off = w.part_ml;
    *sum_off = align256(*cs_off + heads * size_t(nc) * kVsChunk * 8);
    *piece_off = align256(*sum_off + heads * size_t(nc) * 16);
    return std::max(w.total, align256(*piece_off + heads * size_t(nc) * (kVsChunk / 16) * 8));
}

// Split shapes. bfloat16 caches use balanced blocks: each (sequence, KV
// head) group gets nb blocks that split the group's chunks (32-token pieces
// of its drawn teams, or of every team for dense) into even contiguous
// ranges, about kBalancedBlocks blocks in all: one per CU streamed best on
// MI355X at 32K-128K contexts, batch 1-8 (more blocks only add prologues).
// float32 caches use team ranges (one round trip before the K/V loads;
// blocks of undrawn teams exit early) or, with several teams per block,
// union ranks: a group holds at most U = min(P, G M) distinct drawn teams and
// block s takes those of ranks [s tps, (s + 1) tps).
constexpr int64_t kBalancedBlocks = 256;

static void balanced_split(Params *p) {
    const int64_t groups = int64_t(p->B) * p->Hkv;
    p->balanced = 1;
    p->ranked = 1;
    p->tps = 1;
    p->spread = 0;
    p->max_splits = int32_t(std::min<int64_t>(p->P, std::max<int64_t>(1, (kBalancedBlocks + groups - 1) / groups)));
}

// Few query heads per call (bfloat16): one block per (head, range) of the
// head's own drawn chunks, S ranges per head so that about kBalancedBlocks
// blocks run. Used when the call has at most kPerHeadMaxHeads (sequence,
// query head) pairs: the per-head blocks then need only one head's
// selection each and the launch fills the chip.
static bool per_head_shape(const Params &p) {
    return p.dtype == SANTA_BF16 && p.P <= kPerHeadMaxTeams && int64_t(p.B) * p.Hq <= kPerHeadMaxHeads;
}

static void per_head_split(Params *p) {
    const int64_t heads = int64_t(p->B) * p->Hq;
    p->balanced = 1;
    p->per_head = 1;
    p->ranked = 1;
    p->tps = 1;
    p->spread = 0;
    p->max_splits = int32_t(std::min<int64_t>(p->P, std::max<int64_t>(1, kBalancedBlocks / heads)));
}

static void santa_split(Params *p) {
    const int64_t groups = int64_t(p->B) * p->Hkv;
    p->balanced = 0;
    p->per_head = 0;
    if (per_head_shape(*p)) {
        per_head_split(p);
        return;
    }
    if (p->dtype == SANTA_BF16) {
        balanced_split(p);
        return;
    }
    p->tps = teams_per_split(groups * p->P, 2048);
    p->ranked = 0;
    if (p->tps == 1) {
        p->max_splits = p->P;
        return;
    }
    const int64_t U = std::min<int64_t>(p->P, int64_t(p->G) * p->M);
    p->ranked = 1;
    p->tps = teams_per_split(groups * U, 1024);
    p->max_splits = int32_t((U + p->tps - 1) / p->tps);
}

static Params base_params(const santa_kv &kv, const void *q, float *out, float *lse, void *workspace,
                          const WorkspaceLayout &w) {
    Params p{};
    p.dtype = kv.dtype;
    p.k_pages = kv.k_pages;
    p.v_pages = kv.v_pages;
    p.q = q;
    p.page_table = kv.page_table;
    p.seq_lens = kv.seq_lens;
    p.num_pages = kv.num_pages;
    p.B = kv.batch;
    p.Hq = kv.num_q_heads;
    p.Hkv = kv.num_kv_heads;
    p.G = kv.num_q_heads / kv.num_kv_heads;
    p.d = kv.head_dim;
    p.T = kv.page_size;
    p.P = kv.max_pages_per_seq;
    p.words = w.words;
    p.slots = w.slots;
    p.scale = 1.0 / std::sqrt(double(kv.head_dim));
    char *ws = static_cast<char *>(workspace);
    if (ws) {
        p.bitmaps = reinterpret_cast<uint32_t *>(ws + w.bitmaps);
        p.lnw = reinterpret_cast<float *>(ws + w.lnw);
        p.part_ml = reinterpret_cast<float *>(ws + w.part_ml);
        p.part_acc = reinterpret_cast<float *>(ws + w.part_acc);
        p.grp_slots = reinterpret_cast<int32_t *>(ws + w.grp_slots);
    }
    p.out = out;
    p.lse = lse;
    return p;
}

static Params base_params(const santa_kv &kv, const void *q, float *out, float *lse, void *workspace) {
    return base_params(kv, q, out, lse, workspace, workspace_layout(kv));
}

static santa_status check_workspace(const santa_kv &kv, void *workspace, size_t bytes) {
    if (!workspace) return SANTA_ERR_WORKSPACE;
    if (bytes < workspace_layout(kv).total) return SANTA_ERR_WORKSPACE;
    return SANTA_OK;
}

// Split-K gather then the cross-split combine, shared by all three attention
// entry points once the per-head team bitmaps and weights are in place.
static santa_status run_gather_combine(Params &p, void *stream) {
    santa_status st = launch_gather(p, stream);
    if (st != SANTA_OK) return st;
    return launch_combine(p, stream);
}

// Selection, gather and combine of one decode call on a filled-in Params:
// with per-head blocks, one gather launch that selects for itself; else the
// selection kernel first. Either gives the same bits as santa_select_teams
// followed by santa_attend_selected (same split shape, same arithmetic).
static santa_status run_decode(Params &p, void *stream) {
    if (p.per_head) {
        p.fused = 1;
        return run_gather_combine(p, stream);
    }
    santa_status st = launch_select(p, stream);
    if (st != SANTA_OK) return st;
    return run_gather_combine(p, stream);
}

}  // namespace santa

using namespace santa;

extern "C" {

santa_status santa_workspace_size(const santa_kv *kv, int32_t M, size_t *bytes) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!bytes) return SANTA_ERR_NULL;
    if (M < 1) return SANTA_ERR_SHAPE;
    *bytes = workspace_layout(*kv).total;
    return SANTA_OK;
}

santa_status santa_build_reps(const santa_kv *kv, void *reps, void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!reps) return SANTA_ERR_NULL;
    Params p = base_params(*kv, nullptr, nullptr, nullptr, nullptr);
    p.reps_out = reps;
    return launch_build_reps(p, stream);
}

santa_status santa_update_reps(const santa_kv *kv, void *reps, const int32_t *prev_seq_lens,
                               int32_t max_new_tokens, void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!reps || !prev_seq_lens) return SANTA_ERR_NULL;
    if (max_new_tokens < 0) return SANTA_ERR_SHAPE;
    if (max_new_tokens == 0) return SANTA_OK;
    Params p = base_params(*kv, nullptr, nullptr, nullptr, nullptr);
    p.reps_out = reps;
    p.prev_lens = prev_seq_lens;
    // Tokens [prev, prev + n) touch at most ceil(n / T) + 1 teams from the
    // one holding token prev; never more than the table holds.
    const int64_t teams = (int64_t(max_new_tokens) + kv->page_size - 1) / kv->page_size + 1;
    p.update_teams = int32_t(std::min<int64_t>(teams, kv->max_pages_per_seq));
    return launch_build_reps(p, stream);
}

santa_status santa_append_kv(const santa_kv *kv, const int32_t *prev_seq_lens, const void *k_new,
                             const void *v_new, int32_t max_new_tokens, void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!prev_seq_lens || !k_new || !v_new) return SANTA_ERR_NULL;
    if (max_new_tokens < 0) return SANTA_ERR_SHAPE;
    if (max_new_tokens == 0) return SANTA_OK;
    const int64_t threads = int64_t(kv->batch) * max_new_tokens * kv->num_kv_heads * kv->head_dim;
    if (threads >= (int64_t(1) << 31)) return SANTA_ERR_SHAPE;     // one thread per element, 32-bit grid
    AppendParams ap{k_new, v_new, const_cast<void *>(kv->k_pages), const_cast<void *>(kv->v_pages),
                    kv->page_table, kv->seq_lens, prev_seq_lens, kv->num_pages, kv->dtype, kv->batch,
                    kv->max_pages_per_seq, kv->num_kv_heads, kv->page_size, kv->head_dim, max_new_tokens};
    return launch_append_kv(ap, stream);
}

santa_status santa_build_reps_ex(const santa_kv *kv, void *reps, int32_t kind, uint64_t seed,
                                 const int32_t *prev_seq_lens, int32_t max_new_tokens, void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!reps) return SANTA_ERR_NULL;
    if (kind != SANTA_REP_MEAN && kind != SANTA_REP_MEDOID && kind != SANTA_REP_RANDOM) return SANTA_ERR_SHAPE;
    Params p = base_params(*kv, nullptr, nullptr, nullptr, nullptr);
    p.reps_out = reps;
    p.rep_kind = kind;
    p.seed_lo = uint32_t(seed);
    p.seed_hi = uint32_t(seed >> 32);
    if (prev_seq_lens) {
        if (max_new_tokens < 0) return SANTA_ERR_SHAPE;
        if (max_new_tokens == 0) return SANTA_OK;
        p.prev_lens = prev_seq_lens;
        const int64_t teams = (int64_t(max_new_tokens) + kv->page_size - 1) / kv->page_size + 1;
        p.update_teams = int32_t(std::min<int64_t>(teams, kv->max_pages_per_seq));
    }
    return launch_build_reps(p, stream);
}

static santa_status santa_params(const santa_kv *kv, const void *q, int32_t M, float *out, float *lse,
                                 void *workspace, size_t workspace_bytes, Params *p) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!q) return SANTA_ERR_NULL;
    if (M < 1) return SANTA_ERR_SHAPE;
    st = check_workspace(*kv, workspace, workspace_bytes);
    if (st != SANTA_OK) return st;
    *p = base_params(*kv, q, out, lse, workspace);
    p->M = M;
    p->mode = kModeSanta;
    santa_split(p);
    return SANTA_OK;
}

santa_status santa_select_teams_ex(const santa_kv *kv, const void *q, const void *reps,
                                   int32_t M, uint64_t seed, uint32_t offset, int32_t scheme,
                                   int32_t *sampled, float *inv_pi,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    Params p;
    santa_status st = santa_params(kv, q, M, nullptr, nullptr, workspace, workspace_bytes, &p);
    if (st != SANTA_OK) return st;
    if (!reps) return SANTA_ERR_NULL;
    if (scheme != SANTA_DRAW_IID && scheme != SANTA_DRAW_SYSTEMATIC && scheme != SANTA_DRAW_STRATIFIED)
        return SANTA_ERR_SHAPE;
    p.scheme = scheme;
    if ((sampled == nullptr) != (inv_pi == nullptr)) return SANTA_ERR_NULL;
    p.reps = reps;
    p.seed_lo = uint32_t(seed & 0xffffffffu);
    p.seed_hi = uint32_t(seed >> 32);
    p.offset = offset;
    p.sampled = sampled;
    p.inv_pi = inv_pi;
    return launch_select(p, stream);
}

santa_status santa_value_sampled_workspace_size(const santa_kv *kv, int32_t M, size_t *bytes) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!bytes) return SANTA_ERR_NULL;
    if (M < 1) return SANTA_ERR_SHAPE;
    if (int64_t(std::min(M, kv->max_pages_per_seq)) * kv->page_size > kVsMaxTokens) return SANTA_ERR_UNSUPPORTED;
    size_t cs_off, sum_off, piece_off;
    int32_t chunks;
    *bytes = value_workspace_layout(*kv, M, &cs_off, &sum_off, &piece_off, &chunks);
    return SANTA_OK;
}

santa_status santa_decode_attention_value_sampled(const santa_kv *kv, const void *q, const void *reps,
                                                 int32_t M, int32_t scheme, int32_t S, int32_t value_scheme,
                                                 uint64_t seed, uint32_t offset, float *out, float *lse,
                                                 int32_t *sampled, float *inv_pi, int32_t *positions,
                                                 void *workspace, size_t workspace_bytes, void *stream) {
    Params p;
    santa_status st = santa_params(kv, q, M, out, lse, workspace, workspace_bytes, &p);
    if (st != SANTA_OK) return st;
    if (!reps || !out) return SANTA_ERR_NULL;
    if ((sampled == nullptr) != (inv_pi == nullptr)) return SANTA_ERR_NULL;
    for (int32_t sc : {scheme, value_scheme})
        if (sc != SANTA_DRAW_IID && sc != SANTA_DRAW_SYSTEMATIC && sc != SANTA_DRAW_STRATIFIED) return SANTA_ERR_SHAPE;
    if (S < 1 || S > kVsMaxSamples) return SANTA_ERR_SHAPE;
    if (int64_t(std::min(M, kv->max_pages_per_seq)) * kv->page_size > kVsMaxTokens) return SANTA_ERR_UNSUPPORTED;
    size_t cs_off, sum_off, piece_off;
    if (workspace_bytes < value_workspace_layout(*kv, M, &cs_off, &sum_off, &piece_off, &p.vs_chunks))
        return SANTA_ERR_WORKSPACE;
    p.vs_cs = reinterpret_cast<double *>(static_cast<char *>(workspace) + cs_off);
    p.vs_sum = reinterpret_cast<double *>(static_cast<char *>(workspace) + sum_off);
    p.vs_piece = reinterpret_cast<double *>(static_cast<char *>(workspace) + piece_off);
    p.scheme = scheme;
    p.reps = reps;
    p.seed_lo = uint32_t(seed & 0xffffffffu);
    p.seed_hi = uint32_t(seed >> 32);
    p.offset = offset;
    p.sampled = sampled;
    p.inv_pi = inv_pi;
    p.vs_samples = S;
    p.vs_scheme = value_scheme;
    p.vs_positions = positions;
    st = launch_select(p, stream);
    if (st != SANTA_OK) return st;
    return launch_value_sample(p, stream);
}

santa_status santa_select_teams(const santa_kv *kv, const void *q, const void *reps,
                                int32_t M, uint64_t seed, uint32_t offset,
                                int32_t *sampled, float *inv_pi,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return santa_select_teams_ex(kv, q, reps, M, seed, offset, SANTA_DRAW_IID, sampled, inv_pi,
                                 workspace, workspace_bytes, stream);
}

santa_status santa_attend_selected(const santa_kv *kv, const void *q, int32_t M,
                                   float *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    Params p;
    santa_status st = santa_params(kv, q, M, out, lse, workspace, workspace_bytes, &p);
    if (st != SANTA_OK) return st;
    if (!out) return SANTA_ERR_NULL;
    return run_gather_combine(p, stream);
}

santa_status santa_decode_attention_ex(const santa_kv *kv, const void *q, const void *reps,
                                       int32_t M, uint64_t seed, uint32_t offset, int32_t scheme,
                                       float *out, float *lse, int32_t *sampled, float *inv_pi,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    Params p;
    santa_status st = santa_params(kv, q, M, out, lse, workspace, workspace_bytes, &p);
    if (st != SANTA_OK) return st;
    if (!reps || !out) return SANTA_ERR_NULL;
    if (scheme != SANTA_DRAW_IID && scheme != SANTA_DRAW_SYSTEMATIC && scheme != SANTA_DRAW_STRATIFIED)
        return SANTA_ERR_SHAPE;
    if ((sampled == nullptr) != (inv_pi == nullptr)) return SANTA_ERR_NULL;
    p.scheme = scheme;
    p.reps = reps;
    p.seed_lo = uint32_t(seed & 0xffffffffu);
    p.seed_hi = uint32_t(seed >> 32);
    p.offset = offset;
    p.sampled = sampled;
    p.inv_pi = inv_pi;
    return run_decode(p, stream);
}

santa_status santa_decode_attention_noalloc(const santa_kv *kv, const void *q, const void *reps,
                                            int32_t M, uint64_t seed, uint32_t offset,
                                            float *out, float *lse, int32_t *sampled, float *inv_pi,
                                            void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!q || !reps || !out) return SANTA_ERR_NULL;
    if (M < 1) return SANTA_ERR_SHAPE;
    if ((sampled == nullptr) != (inv_pi == nullptr)) return SANTA_ERR_NULL;
    // The split shape of this call, then a workspace with exactly its slots.
    Params p = base_params(*kv, q, out, lse, nullptr);
    p.M = M;
    p.mode = kModeSanta;
    santa_split(&p);
    const WorkspaceLayout w = workspace_layout(*kv, p.max_splits);
    if (w.total > kNoallocScratchBytes) return SANTA_ERR_WORKSPACE;
    void *scratch = nullptr;
    st = noalloc_scratch(stream, &scratch);
    if (st != SANTA_OK) return st;
    Params r = base_params(*kv, q, out, lse, scratch, w);
    r.M = M;
    r.mode = kModeSanta;
    santa_split(&r);
    r.scheme = SANTA_DRAW_IID;
    r.reps = reps;
    r.seed_lo = uint32_t(seed & 0xffffffffu);
    r.seed_hi = uint32_t(seed >> 32);
    r.offset = offset;
    r.sampled = sampled;
    r.inv_pi = inv_pi;
    return run_decode(r, stream);
}

santa_status santa_decode_attention(const santa_kv *kv, const void *q, const void *reps,
                                    int32_t M, uint64_t seed, uint32_t offset,
                                    float *out, float *lse, int32_t *sampled, float *inv_pi,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    return santa_decode_attention_ex(kv, q, reps, M, seed, offset, SANTA_DRAW_IID, out, lse, sampled, inv_pi,
                                     workspace, workspace_bytes, stream);
}

santa_status dense_decode_attention(const santa_kv *kv, const void *q, float *out, float *lse,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!q || !out) return SANTA_ERR_NULL;
    st = check_workspace(*kv, workspace, workspace_bytes);
    if (st != SANTA_OK) return st;
    Params p = base_params(*kv, q, out, lse, workspace);
    p.mode = kModeDense;
    if (p.dtype == SANTA_BF16) {
        balanced_split(&p);
        // Batch >= 2: the kernel picks a split over all groups when the
        // lengths are ragged (they are known only on the device).
        if (p.B >= 2 && int64_t(p.B) * p.Hkv <= kMaxSpreadGroups) p.spread = 1;
    } else {
        p.tps = teams_per_split(int64_t(p.B) * p.Hkv * p.P, 512);
        while (p.tps < kMaxTeamsPerSplit && (p.P + p.tps - 1) / p.tps > 128) p.tps *= 2;
        p.max_splits = (p.P + p.tps - 1) / p.tps;
    }
    return run_gather_combine(p, stream);
}

santa_status santa_attention_given_teams(const santa_kv *kv, const void *q, int32_t M,
                                         const int32_t *teams, const float *weights,
                                         float *out, float *lse,
                                         void *workspace, size_t workspace_bytes, void *stream) {
    Params p;
    santa_status st = santa_params(kv, q, M, out, lse, workspace, workspace_bytes, &p);
    if (st != SANTA_OK) return st;
    if (!teams || !weights || !out) return SANTA_ERR_NULL;
    p.given_teams = teams;
    p.given_w = weights;
    st = launch_given(p, stream);
    if (st != SANTA_OK) return st;
    return run_gather_combine(p, stream);
}

santa_status santa_pack_pages(int32_t dtype, int64_t num_pages, int32_t num_kv_heads,
                              int32_t page_size, int32_t head_dim,
                              const void *k_src, const void *v_src, void *k_dst, void *v_dst,
                              void *stream) {
    if (dtype != SANTA_F32 && dtype != SANTA_BF16) return SANTA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return SANTA_ERR_UNSUPPORTED;
    const int T = page_size;
    if (T != 16 && T != 32 && T != 64 && T != 128 && T != 256) return SANTA_ERR_UNSUPPORTED;
    if (num_kv_heads < 1 || num_pages < 0) return SANTA_ERR_SHAPE;
    if (num_pages > (int64_t(1) << 31) / num_kv_heads) return SANTA_ERR_SHAPE;
    const int64_t tiles = num_pages * num_kv_heads;
    if (tiles >= (int64_t(1) << 31)) return SANTA_ERR_SHAPE;
    if (tiles == 0) return SANTA_OK;
    if (!k_src || !v_src || !k_dst || !v_dst) return SANTA_ERR_NULL;
    const uintptr_t bytes = uintptr_t(tiles) * uintptr_t(T) * uintptr_t(head_dim) * (dtype == SANTA_BF16 ? 2u : 4u);
    const uintptr_t lo[4] = {uintptr_t(k_src), uintptr_t(v_src), uintptr_t(k_dst), uintptr_t(v_dst)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if ((i >= 2 || j >= 2) && lo[i] < lo[j] + bytes && lo[j] < lo[i] + bytes) return SANTA_ERR_SHAPE;
    PackParams pp{k_src, v_src, k_dst, v_dst, tiles, dtype, T, head_dim};
    return launch_pack_pages(pp, stream);
}

santa_status santa_pack_pages_hashed(const santa_kv *kv, const void *k_src, const void *v_src,
                                     const float *directions, int32_t bits,
                                     int32_t *codes, int32_t *token_of, void *stream) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (!k_src || !v_src || !directions || !codes || !token_of) return SANTA_ERR_NULL;
    if (bits < 1 || bits > kMaxHashBits) return SANTA_ERR_SHAPE;
    const int64_t positions = int64_t(kv->batch) * kv->num_kv_heads * kv->max_pages_per_seq * kv->page_size;
    if (positions >= (int64_t(1) << 31)) return SANTA_ERR_SHAPE;
    // Source and destination pages must be distinct buffers.
    const uintptr_t bytes = uintptr_t(kv->num_pages) * uintptr_t(kv->num_kv_heads) * uintptr_t(kv->page_size) *
                            uintptr_t(kv->head_dim) * (kv->dtype == SANTA_BF16 ? 2u : 4u);
    const uintptr_t lo[4] = {uintptr_t(k_src), uintptr_t(v_src), uintptr_t(kv->k_pages), uintptr_t(kv->v_pages)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if ((i >= 2 || j >= 2) && lo[i] < lo[j] + bytes && lo[j] < lo[i] + bytes) return SANTA_ERR_SHAPE;
    ClusterParams c{};
    c.k_src = k_src;
    c.v_src = v_src;
    c.k_dst = const_cast<void *>(kv->k_pages);
    c.v_dst = const_cast<void *>(kv->v_pages);
    c.directions = directions;
    c.page_table = kv->page_table;
    c.seq_lens = kv->seq_lens;
    c.codes = codes;
    c.token_of = token_of;
    c.num_pages = kv->num_pages;
    c.dtype = kv->dtype;
    c.B = kv->batch;
    c.Hkv = kv->num_kv_heads;
    c.P = kv->max_pages_per_seq;
    c.T = kv->page_size;
    c.d = kv->head_dim;
    c.bits = bits;
    return launch_pack_hashed(c, stream);
}

}  // extern "C"

namespace {

struct KmeansLayout {
    int32_t cmax = 0, bits = 0;
    size_t mu = 0, half = 0, starts = 0, total = 0;
};

// Clusters allocated per (sequence, KV head) and the workspace sections.
santa_status kmeans_layout(const santa_kv *kv, int32_t clusters, KmeansLayout *out) {
    santa_status st = validate_kv(kv);
    if (st != SANTA_OK) return st;
    if (clusters < 0) return SANTA_ERR_SHAPE;
    const int64_t cap = int64_t(kv->max_pages_per_seq) * kv->page_size;
    if (int64_t(kv->batch) * kv->num_kv_heads * cap >= (int64_t(1) << 31)) return SANTA_ERR_SHAPE;
    const int64_t cmax = clusters > 0 ? std::min<int64_t>(clusters, cap) : kv->max_pages_per_seq;
    if (cmax > kMaxClusters) return SANTA_ERR_SHAPE;
    KmeansLayout w;
    w.cmax = int32_t(std::max<int64_t>(cmax, 1));
    while ((int64_t(1) << w.bits) < w.cmax) ++w.bits;
    const size_t heads = size_t(kv->batch) * kv->num_kv_heads;
    size_t off = 0;
    w.mu = off;     off = align256(off + heads * w.cmax * size_t(kv->head_dim) * 8);
    w.half = off;   off = align256(off + heads * w.cmax * 8);
    w.starts = off; off = align256(off + heads * ((size_t(1) << w.bits) + 1) * 4);
    w.total = off;
    *out = w;
    return SANTA_OK;
}

}  // namespace

extern "C" {

santa_status santa_kmeans_workspace_size(const santa_kv *kv, int32_t clusters, size_t *bytes) {
    if (!bytes) return SANTA_ERR_NULL;
    KmeansLayout w;
    const santa_status st = kmeans_layout(kv, clusters, &w);
    if (st == SANTA_OK) *bytes = w.total;
    return st;
}

santa_status santa_pack_pages_kmeans(const santa_kv *kv, const void *k_src, const void *v_src,
                                     int32_t clusters, int32_t iters, int32_t *codes,
                                     int32_t *token_of, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    KmeansLayout w;
    santa_status st = kmeans_layout(kv, clusters, &w);
    if (st != SANTA_OK) return st;
    if (!k_src || !v_src || !codes || !token_of) return SANTA_ERR_NULL;
    if (iters < 1 || iters > kMaxKmeansIters) return SANTA_ERR_SHAPE;
    if (!workspace || workspace_bytes < w.total || uintptr_t(workspace) % 8 != 0) return SANTA_ERR_WORKSPACE;
    const uintptr_t bytes = uintptr_t(kv->num_pages) * uintptr_t(kv->num_kv_heads) * uintptr_t(kv->page_size) *
                            uintptr_t(kv->head_dim) * (kv->dtype == SANTA_BF16 ? 2u : 4u);
    const uintptr_t lo[4] = {uintptr_t(k_src), uintptr_t(v_src), uintptr_t(kv->k_pages), uintptr_t(kv->v_pages)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if ((i >= 2 || j >= 2) && lo[i] < lo[j] + bytes && lo[j] < lo[i] + bytes) return SANTA_ERR_SHAPE;
    char *ws = static_cast<char *>(workspace);
    ClusterParams c{};
    c.k_src = k_src;
    c.v_src = v_src;
    c.k_dst = const_cast<void *>(kv->k_pages);
    c.v_dst = const_cast<void *>(kv->v_pages);
    c.page_table = kv->page_table;
    c.seq_lens = kv->seq_lens;
    c.codes = codes;
    c.token_of = token_of;
    c.num_pages = kv->num_pages;
    c.dtype = kv->dtype;
    c.B = kv->batch;
    c.Hkv = kv->num_kv_heads;
    c.P = kv->max_pages_per_seq;
    c.T = kv->page_size;
    c.d = kv->head_dim;
    c.bits = w.bits;
    c.mu = reinterpret_cast<double *>(ws + w.mu);
    c.half = reinterpret_cast<double *>(ws + w.half);
    c.starts = reinterpret_cast<int32_t *>(ws + w.starts);
    c.clusters = clusters;
    c.cmax = w.cmax;
    return launch_pack_kmeans(c, iters, stream);
}

const char *santa_status_string(int32_t status) {
    switch (status) {
        case SANTA_OK: return "ok";
        case SANTA_ERR_NULL: return "a required pointer is NULL";
        case SANTA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case SANTA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, page_size or group size";
        case SANTA_ERR_WORKSPACE: return "workspace missing or too small";
        case SANTA_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

int32_t santa_version(void) { return 260; }

}  // extern "C"
