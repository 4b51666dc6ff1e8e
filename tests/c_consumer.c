/* A plain C99 consumer of libsanta: includes the public header, links the
 * shared library, and exercises the calls that need no GPU (version, status
 * strings, workspace sizes, host-side argument validation). It checks that
 * the header is valid C and that the library is usable without Python.
 * Every call below returns before any kernel launch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "santa.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "line %d: %s\n", __LINE__, #cond);        \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main(void) {
    /* Non-NULL pointer values that validation never dereferences; the two
     * page arrays are far apart so they do not overlap. */
    const uintptr_t fake = 0x10000u;
    santa_kv kv;
    size_t bytes = 0;

    memset(&kv, 0, sizeof kv);
    kv.dtype = SANTA_BF16;
    kv.batch = 2;
    kv.num_q_heads = 28;
    kv.num_kv_heads = 4;
    kv.head_dim = 128;
    kv.page_size = 128;
    kv.max_pages_per_seq = 256;
    kv.num_pages = 512;
    kv.k_pages = (const void *)fake;
    kv.v_pages = (const void *)(fake + ((uintptr_t)1 << 40));
    kv.page_table = (const int32_t *)fake;
    kv.seq_lens = (const int32_t *)fake;

    EXPECT(santa_version() >= 100);
    EXPECT(strcmp(santa_status_string(SANTA_OK), "ok") == 0);
    EXPECT(santa_status_string(SANTA_ERR_WORKSPACE) != NULL);

    EXPECT(santa_workspace_size(&kv, 31, &bytes) == SANTA_OK && bytes > 0);
    EXPECT(santa_workspace_size(NULL, 31, &bytes) == SANTA_ERR_NULL);
    EXPECT(santa_kmeans_workspace_size(&kv, 0, &bytes) == SANTA_OK && bytes > 0);

    /* Validation statuses, each before any HIP call. */
    EXPECT(santa_decode_attention(&kv, NULL, (const void *)fake, 31, 0, 0, (float *)fake, NULL, NULL, NULL,
                                  (void *)fake, (size_t)1 << 40, NULL) == SANTA_ERR_NULL);
    EXPECT(santa_decode_attention(&kv, (const void *)fake, (const void *)fake, 31, 0, 0, (float *)fake, NULL,
                                  NULL, NULL, NULL, 0, NULL) == SANTA_ERR_WORKSPACE);
    kv.head_dim = 80;
    EXPECT(santa_build_reps(&kv, (void *)fake, NULL) == SANTA_ERR_UNSUPPORTED);
    kv.head_dim = 128;
    kv.num_q_heads = 30;                  /* not a multiple of num_kv_heads */
    EXPECT(dense_decode_attention(&kv, (const void *)fake, (float *)fake, NULL, (void *)fake, (size_t)1 << 40,
                                  NULL) != SANTA_OK);

    if (failures) return 1;
    printf("c consumer ok (libsanta %d)\n", santa_version());
    return 0;
}
