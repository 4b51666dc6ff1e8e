/*
 * libsanta — SANTA++ sampled-team decode attention for AMD MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [ABS] "SANTA++: Sampling Attention through Representative Keys",
 *         arXiv 2609.35629, abstract.
 *   [EXP] "SANTA++：用代表性 Key 采样把 KV cache 读带宽砍掉 80%" (explainer),
 *         section 三 (core method) and its sub-sections 3.1-3.2.
 *
 * What the library computes, for one decode step of one attention layer
 * ([ABS]; [EXP] section 三): for every new query (one per sequence and query
 * head), a dot product with each team's summary key and a softmax give team
 * probabilities p; M draws from p pick the teams whose tokens are read and
 * scored exactly; a drawn team's terms count 1/pi times, pi = 1 - (1 - p)^M
 * its chance of being drawn, so the weighted sums stand in, without bias, for
 * the sums over every cached token. A dense decode over every cached token,
 * built from the same kernels, is exported as the baseline.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array argument is a device (HBM) pointer, owned by the
 *           caller, 16-byte aligned, densely packed in the layout stated.
 *           The library allocates nothing and keeps no state between calls;
 *           calls are re-entrant and may run concurrently on different
 *           streams if their output and workspace buffers differ. (The one
 *           exception, santa_decode_attention_noalloc, brings its own
 *           workspace: a device array per GPU, shared by its calls.)
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *           stream). All work is enqueued on it and the call returns before
 *           it runs; buffers must stay valid until the stream reaches it.
 * Errors.   Arguments are checked on the host before any HIP call; a bad
 *           argument returns a status and enqueues nothing. A launch failure
 *           returns SANTA_ERR_HIP. Values that live in device memory
 *           (seq_lens, page_table, teams) are not visible to the host: the
 *           kernels clamp sequence lengths to [0, page_size * max_pages_per_seq]
 *           and page ids to [0, num_pages - 1] so they never read out of
 *           bounds, but results for such inputs are meaningless.
 * Results.  Deterministic: the same inputs, seed and offset give bitwise
 *           identical outputs (no floating-point atomics; partial results
 *           are merged in a fixed order).
 *
 * Paged KV layout (all entry points)
 * ----------------------------------
 *   k_pages, v_pages  [num_pages][num_kv_heads][tile], dtype; a tile holds
 *                     the page_size * head_dim keys (values) of one page and
 *                     KV head in the chunked order below
 *   tile order        chunks of C = min(page_size, 32) tokens, C * head_dim
 *                     elements each, in token order. Inside chunk c (tokens
 *                     c*C .. c*C + C - 1):
 *                       keys:   head_dim / 32 slabs, slab s = [C][32]: key of
 *                               token c*C + i, channel 32 s + j at element
 *                               c*C*d + s*C*32 + i*32 + j
 *                       values: channel-major [d][C]: value of token c*C + i,
 *                               channel ch at element c*C*d + ch*C + i
 *                     (d = head_dim). With this order every 16-byte load of
 *                     the decode kernels' matrix-core operands lies in a run
 *                     of whole 128-byte lines that one instruction reads
 *                     entirely. santa_pack_pages writes pages in this order
 *                     from plain [page][KV head][token][channel] arrays.
 *   page_table        [batch][max_pages_per_seq] int32: physical page of
 *                     logical team t of sequence b
 *   seq_lens          [batch] int32: cached tokens L_b of sequence b
 * A team is one page: team t of sequence b is tokens [t*T, min((t+1)*T, L_b))
 * stored in physical page page_table[b][t] (T = page_size). The pages leave
 * the team partition open ([EXP] 3.2); contiguous runs, one per page, are
 * the default; santa_pack_pages_hashed and santa_pack_pages_kmeans write
 * each sequence's tokens in a hash- or k-means-partition order so that the
 * same pages hold clustered teams.
 * Sequence b has K_b = ceil(L_b / T) teams.
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef SANTA_H
#define SANTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum santa_status {
    SANTA_OK = 0,
    SANTA_ERR_NULL = 1,         /* a required pointer is NULL                      */
    SANTA_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes              */
    SANTA_ERR_UNSUPPORTED = 3,  /* valid but not built (dtype, head_dim, page_size) */
    SANTA_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required          */
    SANTA_ERR_HIP = 5           /* a HIP launch failed                              */
} santa_status;

typedef enum santa_dtype {
    SANTA_F32 = 0,              /* IEEE binary32                                    */
    SANTA_BF16 = 1              /* bfloat16 (top 16 bits of a binary32)             */
} santa_dtype;

/* Supported sizes: dtype in {SANTA_F32, SANTA_BF16}; head_dim in {64, 128};
 * page_size in {16, 32, 64, 128, 256}; num_q_heads % num_kv_heads == 0 with
 * num_q_heads / num_kv_heads <= 16; 1 <= max_pages_per_seq <= 2048;
 * 1 <= batch <= 65535; num_pages >= 1. */
typedef struct santa_kv {
    int32_t dtype;              /* santa_dtype of k_pages, v_pages, q and reps       */
    int32_t batch;              /* B                                                 */
    int32_t num_q_heads;        /* Hq                                                */
    int32_t num_kv_heads;       /* Hkv                                               */
    int32_t head_dim;           /* d                                                 */
    int32_t page_size;          /* T: tokens per page = tokens per team              */
    int32_t max_pages_per_seq;  /* row length of page_table                          */
    int32_t reserved;           /* must be 0                                         */
    int64_t num_pages;          /* physical pages in k_pages / v_pages               */
    const void *k_pages;        /* [num_pages][Hkv][T * d] dtype, tile order          */
    const void *v_pages;        /* [num_pages][Hkv][T * d] dtype, tile order          */
    const int32_t *page_table;  /* [B][max_pages_per_seq]                            */
    const int32_t *seq_lens;    /* [B], each in [0, T * max_pages_per_seq]           */
} santa_kv;

/* Bytes of device workspace that santa_decode_attention,
 * santa_attention_given_teams and dense_decode_attention need for this cache
 * shape. The workspace holds per-head team bitmaps and weights and the
 * split-K partial results; its contents need no initialisation. After
 * santa_select_teams(_ex) it holds the drawn sets that santa_attend_selected
 * reads; after any other call its contents are meaningless. Returns SANTA_OK
 * and writes *bytes, or a validation status. */
santa_status santa_workspace_size(const santa_kv *kv, int32_t M, size_t *bytes);

/* Representative keys: reps[b][t][g][:] = the mean of the keys of team t of
 * sequence b for KV head g, rounded once (to nearest, ties to even) to the
 * cache dtype. [EXP] section 三 step 2 (one representative key per team:
 * mean, medoid or random are listed; the mean is used); [ABS] (selection
 * reads these summary keys, not the cache). The mean is the float64 sum of
 * the n valid keys divided by n (n < T only for a sequence's last team).
 *   reps  [B][max_pages_per_seq][Hkv][d] dtype, indexed by logical team so
 *         that selection reads it without a page-table lookup; written for
 *         t < K_b, other rows left untouched.
 * Run once after prefill, and for a team again after its keys change. */
santa_status santa_build_reps(const santa_kv *kv, void *reps, void *stream);

/* Representative kinds of santa_build_reps_ex ([EXP] section 三 step 2 lists
 * the mean, the medoid and a random member as choices of representative). */
typedef enum santa_rep_kind {
    SANTA_REP_MEAN = 0,         /* the rounded team mean (santa_build_reps)           */
    SANTA_REP_MEDOID = 1,       /* the member nearest, in summed distance, to all      */
    SANTA_REP_RANDOM = 2        /* a member drawn from a Philox stream of its own      */
} santa_rep_kind;

/* Representative upkeep after an append ([EXP] section 三 step 2: one
 * representative per team, here kept equal to the team mean as tokens
 * arrive). For each sequence b, recomputes reps[b][t] for the teams that
 * received tokens since the lengths were prev_seq_lens[b], i.e. teams
 * floor(prev_seq_lens[b] / T) .. K_b - 1 (at most ceil(max_new_tokens / T) + 1
 * of them), with the arithmetic of santa_build_reps, so the result equals a
 * full rebuild bit for bit. The new keys must already be in the pages and
 * kv->seq_lens must hold the new lengths.
 *   reps           as for santa_build_reps; rows of other teams untouched
 *   prev_seq_lens  [B] int32, device: lengths before the append; a sequence
 *                  whose length did not grow (prev >= new) keeps every row
 *   max_new_tokens host bound on the tokens appended to any one sequence
 *                  (>= 0; 0 enqueues nothing) */
santa_status santa_update_reps(const santa_kv *kv, void *reps, const int32_t *prev_seq_lens,
                               int32_t max_new_tokens, void *stream);

/* Appended tokens into the cache ([EXP] section 三 step 2: the cache grows
 * by a token per decode step, and the team holding it must stay consistent
 * with its representative). For each sequence b, the tokens at positions
 * prev_seq_lens[b] .. kv->seq_lens[b] - 1 are copied, exactly, from row
 * i = position - prev_seq_lens[b] of k_new / v_new into page
 * page_table[b][position / T], token position mod T, every channel at its
 * tile-order offset (the layout santa_pack_pages writes). A serving step is
 * then: write the new lengths into kv->seq_lens, santa_append_kv,
 * santa_update_reps with the old lengths, decode.
 *   kv              kv->seq_lens holds the new lengths; the pages are written
 *                   through kv->k_pages / kv->v_pages
 *   prev_seq_lens   [B] int32, device: lengths before the append; a sequence
 *                   whose length did not grow writes nothing
 *   k_new, v_new    [B][max_new_tokens][Hkv][d] dtype, device: row i of
 *                   sequence b is its i-th new token; rows at or beyond the
 *                   sequence's count are not read
 *   max_new_tokens  host bound on the tokens appended to any one sequence
 *                   (>= 0; 0 enqueues nothing); more new tokens than this in
 *                   device lengths are not written
 * Positions at or beyond T * max_pages_per_seq, and page ids outside
 * [0, num_pages), are skipped (nothing is written for them). Returns
 * SANTA_ERR_NULL for a missing pointer, SANTA_ERR_SHAPE for a negative
 * max_new_tokens or B * max_new_tokens * Hkv * d >= 2^31. */
santa_status santa_append_kv(const santa_kv *kv, const int32_t *prev_seq_lens, const void *k_new,
                             const void *v_new, int32_t max_new_tokens, void *stream);

/* Representatives of another kind ([EXP] section 三 step 2: mean, medoid or
 * random member), built for every team or refreshed after an append.
 *   kind            SANTA_REP_MEAN: exactly santa_build_reps (or, with
 *                   prev_seq_lens, santa_update_reps).
 *                   SANTA_REP_MEDOID: the member key k_i of the team's n keys
 *                   minimising sum_j ||k_i - k_j||, copied exactly. Each
 *                   distance is the correctly rounded float64 square root of
 *                   the float64 sum, in channel order, of the squared float64
 *                   channel differences; a member's n distances are added in
 *                   member order; equal sums go to the lower member index.
 *                   Costs n * n * d float64 multiply-adds per team and head.
 *                   SANTA_REP_RANDOM: member floor(x * n / 2^32), x = word 0
 *                   of Philox4x32-10 with counter (t, g, b, 0) and key
 *                   (seed lo ^ 0x52455053, seed hi), copied exactly.
 *   seed            SANTA_REP_RANDOM only; the key word change keeps this
 *                   stream apart from the team draws of the same seed
 *   prev_seq_lens   NULL: rows of every team t < K_b are written. Else the
 *                   update mode of santa_update_reps (same meaning of
 *                   prev_seq_lens and max_new_tokens), with the same result
 *                   as a full build of this kind.
 * Returns SANTA_ERR_SHAPE for another kind or a negative max_new_tokens. */
santa_status santa_build_reps_ex(const santa_kv *kv, void *reps, int32_t kind, uint64_t seed,
                                 const int32_t *prev_seq_lens, int32_t max_new_tokens, void *stream);

/* SANTA++ decode attention ([ABS]; [EXP] section 三 steps 2-7).
 * For each sequence b and query head h (KV head g):
 *   1. s_t = q . reps[b][t][g] / sqrt(d), summed in float64;
 *   2. p = softmax(s) over the K_b teams, with cumulative sums C;
 *   3. M draws with replacement by inverse CDF: draw j takes word j mod 4 of
 *      Philox4x32-10 (Salmon et al., SC'11) with counter
 *      (j / 4, h, b, offset) and key (seed & 0xffffffff, seed >> 32), maps it
 *      to u = (word + 1/2) 2^-32 and picks the first t with u * C_last < C_t;
 *      duplicates are removed. If M >= K_b every team is taken with pi = 1;
 *   4. pi_t = 1 - (1 - p_t)^M, weight w_t = 1 / pi_t ([ABS]: inverse of the
 *      inclusion probability);
 *   5. exact scores q . k_j / sqrt(d) for the tokens of the drawn teams and
 *      out = (sum_t w_t sum_j e^{s_j} v_j) / (sum_t w_t sum_j e^{s_j}),
 *      lse = log(sum_t w_t sum_j e^{s_j}).
 * Draws are independent per query head; the K/V tiles of a KV head are read
 * once for the union of its query heads' drawn teams.
 *   q        [B][Hq][d] dtype
 *   reps     [B][max_pages_per_seq][Hkv][d] dtype (from santa_build_reps)
 *   M        draws per query head, >= 1
 *   seed     Philox key; offset: Philox counter word 3 (advance it per
 *            decode step and layer so every step draws afresh)
 *   out      [B][Hq][d] float32
 *   lse      [B][Hq] float32, or NULL
 *   sampled  [B][Hq][M] int32 drawn team indices ascending, -1 padded, or NULL
 *   inv_pi   [B][Hq][M] float32 weights 1/pi of `sampled` (0 padded), or NULL
 * An empty sequence gives out = 0 and lse = -inf. */
santa_status santa_decode_attention(const santa_kv *kv, const void *q, const void *reps,
                                    int32_t M, uint64_t seed, uint32_t offset,
                                    float *out, float *lse, int32_t *sampled, float *inv_pi,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* santa_decode_attention without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments (minus workspace),
 * same draws and same results bit for bit as santa_decode_attention.
 * The workspace is a file-scope device array of SANTA_NOALLOC_SCRATCH_BYTES
 * that each GPU the library runs on holds until the process ends; this call
 * allocates nothing (no hipMalloc or hipFree, no allocating library call).
 * Sizing: a workspace with one partial slot per split-K block of this call,
 *   B*Hq*ceil(P/32)*4 + B*Hq*P*4 + B*Hq*S*8 + B*Hq*S*d*4 + B*Hkv*4 bytes,
 *   each term rounded up to 256, with S the call's split count (bfloat16:
 *   min(P, ceil(256 / (B*Hkv)))); a shape that needs more than the array
 *   returns SANTA_ERR_WORKSPACE and enqueues nothing.
 * Device: the array of the device that owns `stream` (the current device for
 *   the NULL stream); its address is looked up once per device, on the first
 *   call there.
 * Sharing: every call on one GPU uses that GPU's array, whose contents the
 *   next call overwrites (nothing in it needs initialising). Calls that
 *   overlap on one GPU (other streams, other host threads) race on it and
 *   give meaningless results; serialise them on one stream. */
#define SANTA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
santa_status santa_decode_attention_noalloc(const santa_kv *kv, const void *q, const void *reps,
                                            int32_t M, uint64_t seed, uint32_t offset,
                                            float *out, float *lse, int32_t *sampled, float *inv_pi,
                                            void *stream);

/* Where the M draws of santa_decode_attention_ex / santa_select_teams_ex
 * fall. The SANTA page ("Stochastic Sparse Attention for Memory-Bound
 * Inference", abstract) introduces stratified and systematic sampling as
 * lower-variance variants; here they place the team draws. Each scheme
 * takes draw j's uniform u_j = (word + 1/2) 2^-32 as in step 3 of
 * santa_decode_attention and sends a point through the same inverse CDF
 * (first t with point * C_last < C_t):
 *   SANTA_DRAW_IID         point u_j; pi = 1 - (1 - p)^M
 *   SANTA_DRAW_SYSTEMATIC  point (j + u_0) / M; pi = min(1, M p)
 *   SANTA_DRAW_STRATIFIED  point (j + u_j) / M; with a = M C_(t-1) / C_last
 *                          and w = M p_t, q1 = min(w, floor(a) + 1 - a) and
 *                          r = w - q1: pi = 1 if r >= 1, else w - q1 r
 *                          (= 1 - (1 - q1)(1 - r))
 * Every scheme keeps the full-coverage rule (M >= K_b: all teams, pi = 1). */
typedef enum santa_draw_scheme {
    SANTA_DRAW_IID = 0,
    SANTA_DRAW_SYSTEMATIC = 1,
    SANTA_DRAW_STRATIFIED = 2
} santa_draw_scheme;

/* santa_decode_attention and santa_select_teams with a draw scheme
 * (santa_draw_scheme); SANTA_DRAW_IID gives exactly the plain calls.
 * Returns SANTA_ERR_SHAPE for another scheme; otherwise as the plain calls. */
santa_status santa_decode_attention_ex(const santa_kv *kv, const void *q, const void *reps,
                                       int32_t M, uint64_t seed, uint32_t offset, int32_t scheme,
                                       float *out, float *lse, int32_t *sampled, float *inv_pi,
                                       void *workspace, size_t workspace_bytes, void *stream);
santa_status santa_select_teams_ex(const santa_kv *kv, const void *q, const void *reps,
                                   int32_t M, uint64_t seed, uint32_t offset, int32_t scheme,
                                   int32_t *sampled, float *inv_pi,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* The two stages of santa_decode_attention, for callers that time or
 * schedule them separately; running santa_select_teams and then
 * santa_attend_selected on the same workspace equals one
 * santa_decode_attention call.
 *   santa_select_teams:    steps 1-4; writes the per-head team bitmaps and
 *                          log-weights into `workspace` (and `sampled`,
 *                          `inv_pi` when not NULL, as above).
 *   santa_attend_selected: step 5 over the teams the last
 *                          santa_select_teams call with this workspace and
 *                          the same kv, M left in it; writes out and lse. */
santa_status santa_select_teams(const santa_kv *kv, const void *q, const void *reps,
                                int32_t M, uint64_t seed, uint32_t offset,
                                int32_t *sampled, float *inv_pi,
                                void *workspace, size_t workspace_bytes, void *stream);
santa_status santa_attend_selected(const santa_kv *kv, const void *q, int32_t M,
                                   float *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes of santa_decode_attention_value_sampled for this kv and
 * M: the selection's sections followed by the per-chunk running sums
 * (8 bytes per drawn-token slot, ceil(min(M, max_pages_per_seq) * page_size
 * / 512) * 512 slots per (sequence, query head)), the chunks' (max, total)
 * pairs and the running sum at every 16-token piece's end (at least
 * santa_workspace_size's bytes). SANTA_ERR_UNSUPPORTED when
 * min(M, max_pages_per_seq) * page_size > 16384. */
santa_status santa_value_sampled_workspace_size(const santa_kv *kv, int32_t M, size_t *bytes);

/* SANTA++ team draws, then value samples inside the drawn teams ([ABS] for
 * the teams and their 1/pi weights; "Stochastic Sparse Attention for
 * Memory-Bound Inference" (the SANTA page), abstract: token positions
 * picked with probability equal to their attention weight, and the mean of
 * their values, give an unbiased stand-in for the attention output; evenly
 * spread (stratified or systematic) picks reduce its variance). The teams,
 * their weights and the optional sorted set are those of
 * santa_select_teams_ex with `scheme`. Over the drawn tokens, in team order then token order, the
 * weighted logits are l_g = q . k_g / sqrt(d) + log w_t (float64 scores,
 * w_t as stored by the selection: the float32 -log(pi_t)); with
 * e_g = exp(l_g - max l) and C their running sums, value sample k takes the
 * first token g with point_k * C_last < C_g, point_k from Philox4x32-10 word
 * k mod 4 of counter (k / 4, h, b, offset) and key (seed lo ^ 0x56414C55,
 * seed hi), u = (x + 1/2) 2^-32, and (k + u_0) / S or (k + u_k) / S for the
 * systematic and stratified `value_scheme`. Then
 *   out[b][h] = (1 / S) sum_k v(g_k)       float32
 *   lse[b][h] = max l + log C_last          float32 (the drawn tokens' exact
 *                                           log-sum-exp, as santa_decode_attention)
 *   positions [B][Hq][S] int32 or NULL: sampled token positions t * T + j,
 *             in sample order (-1 for an empty sequence)
 * Given the drawn teams, out averages to santa_decode_attention's output
 * (the value samples add their own variance). Reads the drawn teams' keys
 * and only the value lines the samples touch. The running sums C are formed
 * per 512-token chunk of the drawn tokens and the chunk totals then added in
 * chunk order (equal to the flat sums up to rounding). Needs
 * min(M, max_pages_per_seq) * page_size <= 16384 (SANTA_ERR_UNSUPPORTED
 * otherwise), 1 <= S <= 256 (SANTA_ERR_SHAPE) and a workspace of at least
 * santa_value_sampled_workspace_size bytes (SANTA_ERR_WORKSPACE); other
 * arguments as for santa_decode_attention_ex. Three launches (selection,
 * chunk logits, samples). */
santa_status santa_decode_attention_value_sampled(const santa_kv *kv, const void *q, const void *reps,
                                                 int32_t M, int32_t scheme, int32_t S, int32_t value_scheme,
                                                 uint64_t seed, uint32_t offset, float *out, float *lse,
                                                 int32_t *sampled, float *inv_pi, int32_t *positions,
                                                 void *workspace, size_t workspace_bytes, void *stream);

/* Dense decode attention over every cached token: the baseline SANTA++ is
 * compared with ([ABS]: the dense attention baseline). Same kernels as step 5
 * above with every team taken and w = 1.
 *   q [B][Hq][d] dtype; out [B][Hq][d] float32; lse [B][Hq] float32 or NULL. */
santa_status dense_decode_attention(const santa_kv *kv, const void *q, float *out, float *lse,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Step 5 alone, over caller-chosen teams and weights (for testing the
 * estimator, or for a caller that samples teams itself).
 *   teams   [B][Hq][M] int32 team indices of each head, -1 for unused slots;
 *           indices outside [0, K_b) are ignored, repeats count once
 *   weights [B][Hq][M] float32 w > 0 for each listed team
 *   out, lse as in santa_decode_attention. */
santa_status santa_attention_given_teams(const santa_kv *kv, const void *q, int32_t M,
                                         const int32_t *teams, const float *weights,
                                         float *out, float *lse,
                                         void *workspace, size_t workspace_bytes, void *stream);

/* Writes whole pages into the cache's tile order (a pure permutation; every
 * element is copied bit for bit). Not a step of the method: it is how a
 * caller lays out pages after prefill or after filling a page.
 *   k_src, v_src  [num_pages][num_kv_heads][page_size][head_dim] dtype
 *   k_dst, v_dst  [num_pages][num_kv_heads][page_size * head_dim] dtype, in
 *                 the tile order of "Paged KV layout" above
 * dtype, page_size and head_dim as for santa_kv; num_kv_heads >= 1;
 * num_pages >= 0 (0 enqueues nothing); num_pages * num_kv_heads < 2^31. The
 * four buffers must not overlap (SANTA_ERR_SHAPE if their byte ranges do). */
santa_status santa_pack_pages(int32_t dtype, int64_t num_pages, int32_t num_kv_heads,
                              int32_t page_size, int32_t head_dim,
                              const void *k_src, const void *v_src, void *k_dst, void *v_dst,
                              void *stream);

/* Hash-partitioned teams ([EXP] section 三 step 1: keys are clustered into
 * teams; section 八 pitfall 3: the partition may be sequential, hash or
 * cluster). Writes the cache pages of every sequence with its tokens, per KV
 * head, in the order of a sign-hash partition, so that team t (page
 * page_table[b][t]) holds tokens of similar direction; all other entry
 * points then run on these teams unchanged. For sequence b and KV head g,
 * token i (i < L_b) gets code_i whose bit j, most significant first, is
 * [k_i . r_gj > 0], the dot product a float64 sum in channel order; the
 * tokens are stably sorted by code (equal codes keep token order) and the
 * token at sorted position s is written to team s / T, slot s % T. Slots
 * past L_b in the last team are zero.
 *   kv          destination cache: k_pages / v_pages are written (tile order,
 *               see "Paged KV layout"); page_table, seq_lens as usual. A
 *               page may belong to one sequence only. Pages outside the
 *               sequences' first K_b table entries are not written.
 *   k_src, v_src  the same pages in plain [num_pages][Hkv][T][d] order
 *               (distinct from the destination: SANTA_ERR_SHAPE otherwise)
 *   directions  [Hkv][bits][d] float32, device
 *   bits        1 .. 10
 *   codes       [B][Hkv][max_pages_per_seq * T] int32 out: code of token i,
 *               -1 for i >= L_b
 *   token_of    [B][Hkv][max_pages_per_seq * T] int32 out: the token at
 *               sorted position s, -1 for s >= L_b
 * Tokens appended later go to the end in arrival order (santa_update_reps
 * keeps their team's representative); packing again re-partitions. */
santa_status santa_pack_pages_hashed(const santa_kv *kv, const void *k_src, const void *v_src,
                                     const float *directions, int32_t bits,
                                     int32_t *codes, int32_t *token_of, void *stream);

/* k-means-partitioned teams ([EXP] section 三 step 1: teams are clusters of
 * keys; section 八 pitfall 3: the clustering is a choice). Like
 * santa_pack_pages_hashed, but the codes are cluster ids from Lloyd's
 * k-means on the keys of each (sequence b, KV head g):
 *   C_b = min(L_b, clusters), or min(L_b, K_b) when clusters is 0 (one
 *         cluster per team on average);
 *   start: centroid c = the key of token floor(c L_b / C_b);
 *   assign: token i goes to the c with the largest k_i . mu_c - |mu_c|^2 / 2
 *         (the nearest centroid), lowest c on ties; both terms are float64
 *         sums in channel order of separately rounded float64 products;
 *   move: each non-empty cluster's centroid becomes the float64 mean of its
 *         keys, summed in token order from +0.0 and divided once; an empty
 *         cluster's centroid stays;
 *   `iters` assignments with a move between consecutive ones; the codes are
 *         those of the last assignment.
 * Tokens are then stably sorted by code and written to the teams as for the
 * hash partition. Non-finite keys give a valid permutation but no defined
 * clustering.
 *   kv, k_src, v_src, codes, token_of   as for santa_pack_pages_hashed
 *               (codes are cluster ids in [0, C_b))
 *   clusters    0, or the clusters per sequence; clusters (or
 *               max_pages_per_seq when 0), capped at max_pages_per_seq * T,
 *               must be <= 1024
 *   iters       1 .. 1000
 *   workspace   device buffer of santa_kmeans_workspace_size bytes, 8-byte
 *               aligned; holds the centroids and sort offsets; no
 *               initialisation needed, meaningless afterwards
 * Errors: SANTA_ERR_NULL, SANTA_ERR_SHAPE (sizes, clusters, iters,
 * overlapping source and destination), SANTA_ERR_WORKSPACE, and the
 * validation statuses of the cache. Enqueues 3 * iters + 1 launches. */
santa_status santa_kmeans_workspace_size(const santa_kv *kv, int32_t clusters, size_t *bytes);
santa_status santa_pack_pages_kmeans(const santa_kv *kv, const void *k_src, const void *v_src,
                                     int32_t clusters, int32_t iters, int32_t *codes,
                                     int32_t *token_of, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* Static description of a status code. */
const char *santa_status_string(int32_t status);

/* Library ABI version (major * 100 + minor). */
int32_t santa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SANTA_H */
