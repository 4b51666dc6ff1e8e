/* Every libsanta entry point on valid arguments, for the host-only build
 * whose kernel launchers are stubs (tests/host_stubs.cpp): exercises the
 * workspace carve-up, split sizing and parameter set-up of each call under
 * the address and undefined-behaviour sanitizers. Device pointers are fake
 * values that nothing dereferences. Shapes cover bfloat16 and float32, every
 * head size and page size, GQA groups of 1 to 16, one to many sequences, and
 * the largest page table. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "santa.h"

unsigned long long santa_stub_launches(void);

static int failures = 0;

#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "line %d: %s\n", __LINE__, #cond);        \
            ++failures;                                               \
        }                                                             \
    } while (0)

static void *fp(uintptr_t k) { return (void *)((uintptr_t)0x10000u + (k << 40)); }

static void run_shape(int32_t dtype, int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t T, int32_t P,
                      int32_t M) {
    santa_kv kv;
    size_t ws = 0, kws = 0;
    memset(&kv, 0, sizeof kv);
    kv.dtype = dtype;
    kv.batch = batch;
    kv.num_q_heads = hq;
    kv.num_kv_heads = hkv;
    kv.head_dim = d;
    kv.page_size = T;
    kv.max_pages_per_seq = P;
    kv.num_pages = (int64_t)batch * P;
    kv.k_pages = fp(1);
    kv.v_pages = fp(2);
    kv.page_table = (const int32_t *)fp(3);
    kv.seq_lens = (const int32_t *)fp(4);
    EXPECT(santa_workspace_size(&kv, M, &ws) == SANTA_OK && ws > 0);
    EXPECT(santa_build_reps(&kv, fp(5), NULL) == SANTA_OK);
    EXPECT(santa_update_reps(&kv, fp(5), (const int32_t *)fp(6), 3, NULL) == SANTA_OK);
    EXPECT(santa_append_kv(&kv, (const int32_t *)fp(6), fp(7), fp(8), 3, NULL) == SANTA_OK);
    EXPECT(santa_build_reps_ex(&kv, fp(5), SANTA_REP_MEDOID, 7, NULL, 0, NULL) == SANTA_OK);
    EXPECT(santa_build_reps_ex(&kv, fp(5), SANTA_REP_RANDOM, 7, (const int32_t *)fp(6), 2, NULL) == SANTA_OK);
    EXPECT(santa_decode_attention(&kv, fp(9), fp(5), M, 1, 2, (float *)fp(10), (float *)fp(11),
                                  (int32_t *)fp(12), (float *)fp(13), fp(14), ws, NULL) == SANTA_OK);
    EXPECT(santa_decode_attention_ex(&kv, fp(9), fp(5), M, 1, 2, SANTA_DRAW_STRATIFIED, (float *)fp(10), NULL,
                                     NULL, NULL, fp(14), ws, NULL) == SANTA_OK);
    {
        const santa_status st = santa_decode_attention_noalloc(&kv, fp(9), fp(5), M, 1, 2, (float *)fp(10),
                                                               NULL, NULL, NULL, NULL);
        EXPECT(st == SANTA_OK || st == SANTA_ERR_WORKSPACE);
    }
    {
        /* value samples need every drawn token's logit on chip: at most 16384 tokens per head */
        const int64_t drawn = (int64_t)(M < P ? M : P) * T;
        const santa_status want = drawn <= 16384 ? SANTA_OK : SANTA_ERR_UNSUPPORTED;
        size_t vws = 0;
        EXPECT(santa_value_sampled_workspace_size(&kv, M, &vws) == want);
        if (want == SANTA_OK) EXPECT(vws >= ws);
        else vws = ws;
        EXPECT(santa_decode_attention_value_sampled(&kv, fp(9), fp(5), M, SANTA_DRAW_IID, 32, SANTA_DRAW_SYSTEMATIC,
                                                    1, 2, (float *)fp(10), (float *)fp(11), (int32_t *)fp(12),
                                                    (float *)fp(13), (int32_t *)fp(23), fp(14), vws, NULL) == want);
        EXPECT(santa_decode_attention_value_sampled(&kv, fp(9), fp(5), M, SANTA_DRAW_STRATIFIED, 1, SANTA_DRAW_IID,
                                                    1, 2, (float *)fp(10), NULL, NULL, NULL, NULL, fp(14), vws,
                                                    NULL) == want);
    }
    EXPECT(santa_select_teams(&kv, fp(9), fp(5), M, 1, 2, (int32_t *)fp(12), (float *)fp(13), fp(14), ws,
                              NULL) == SANTA_OK);
    EXPECT(santa_select_teams_ex(&kv, fp(9), fp(5), M, 1, 2, SANTA_DRAW_SYSTEMATIC, NULL, NULL, fp(14), ws,
                                 NULL) == SANTA_OK);
    EXPECT(santa_attend_selected(&kv, fp(9), M, (float *)fp(10), (float *)fp(11), fp(14), ws, NULL) == SANTA_OK);
    EXPECT(dense_decode_attention(&kv, fp(9), (float *)fp(10), (float *)fp(11), fp(14), ws, NULL) == SANTA_OK);
    EXPECT(santa_attention_given_teams(&kv, fp(9), M, (const int32_t *)fp(12), (const float *)fp(13),
                                       (float *)fp(10), NULL, fp(14), ws, NULL) == SANTA_OK);
    EXPECT(santa_pack_pages(dtype, kv.num_pages, hkv, T, d, fp(15), fp(16), fp(17), fp(18), NULL) == SANTA_OK);
    EXPECT(santa_pack_pages_hashed(&kv, fp(15), fp(16), (const float *)fp(19), 6, (int32_t *)fp(20),
                                   (int32_t *)fp(21), NULL) == SANTA_OK);
    {
        const int32_t clusters = P <= 1024 ? 0 : 1024;   /* one per team, at most 1024 */
        EXPECT(santa_kmeans_workspace_size(&kv, clusters, &kws) == SANTA_OK && kws > 0);
        EXPECT(santa_pack_pages_kmeans(&kv, fp(15), fp(16), clusters, 4, (int32_t *)fp(20), (int32_t *)fp(21),
                                       fp(22), kws, NULL) == SANTA_OK);
    }
}

int main(void) {
    const unsigned long long before = santa_stub_launches();
    run_shape(SANTA_BF16, 1, 28, 4, 128, 128, 256, 31);      /* per-head path */
    run_shape(SANTA_BF16, 8, 28, 4, 128, 128, 256, 32);      /* union path */
    run_shape(SANTA_BF16, 4, 28, 4, 128, 256, 512, 64);
    run_shape(SANTA_BF16, 3, 48, 3, 64, 16, 2048, 24);       /* longest page table, groups of 16 */
    run_shape(SANTA_BF16, 64, 8, 4, 64, 16, 25, 6);
    run_shape(SANTA_BF16, 1, 1, 1, 64, 32, 1, 1);            /* one team, one draw */
    run_shape(SANTA_F32, 2, 4, 2, 128, 64, 47, 9);
    run_shape(SANTA_F32, 16, 8, 2, 64, 16, 300, 50);
    run_shape(SANTA_F32, 1, 16, 1, 64, 256, 20, 40);         /* M above the team count */
    run_shape(SANTA_BF16, 1, 8, 2, 128, 128, 17, 7);         /* the smoke check's shape */
    EXPECT(santa_stub_launches() > before);
    if (failures) return 1;
    printf("launch paths ok (%llu stub launches)\n", santa_stub_launches() - before);
    return 0;
}
