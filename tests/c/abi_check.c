/* Plain C99 use of include/kvdec.h against libkvdec.so: the header compiles
 * as C, the library links and runs from C, and argument checks that return
 * before any device work behave as documented (no GPU needed). */
#include <stdio.h>
#include <string.h>

#include "kvdec.h"

static int fails = 0;

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++fails;                                                  \
        }                                                             \
    } while (0)

int main(void)
{
    /* capacity padding to whole 64-row groups */
    CHECK(kvdec_padded_capacity(0) == 0);
    CHECK(kvdec_padded_capacity(1) == KVDEC_ROW_ALIGN);
    CHECK(kvdec_padded_capacity(64) == 64);
    CHECK(kvdec_padded_capacity(65) == 128);
    CHECK(kvdec_padded_capacity(2147483647) == 0);          /* padded size would overflow */

    CHECK(strcmp(kvdec_status_str(KVDEC_OK), "ok") == 0);
    CHECK(strlen(kvdec_status_str(KVDEC_E_WORKSPACE)) > 0);

    /* cache creation: invalid descriptors are refused before any device call */
    kvdec_cache* c = NULL;
    CHECK(kvdec_cache_create(NULL, NULL, NULL, &c) == KVDEC_E_INVALID && c == NULL);
    kvdec_cache_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 2;
    d.n_kv_heads = 2;
    d.head_dim = 32;                                       /* only 64 is supported */
    d.capacity = 100;
    d.dtype = KVDEC_BF16;
    int32_t lens[2] = {0, 0};
    CHECK(kvdec_cache_create(&d, lens, NULL, &c) == KVDEC_E_SHAPE && c == NULL);
    CHECK(strlen(kvdec_last_error()) > 0);
    d.head_dim = KVDEC_HEAD_DIM;
    d.window = 50;                                         /* a ring's window equals its capacity */
    CHECK(kvdec_cache_create(&d, lens, NULL, &c) == KVDEC_E_SHAPE && c == NULL);
    d.window = 0;
    CHECK(kvdec_cache_create(&d, lens, NULL, &c) == KVDEC_E_INVALID);   /* NULL device buffers */

    /* calls on a NULL handle */
    float dummy[64];
    CHECK(kvdec_attend_self(NULL, dummy, 4, 0.125f, 0, dummy, dummy, 0, NULL) == KVDEC_E_INVALID);
    CHECK(kvdec_attend_cross(NULL, dummy, 4, 0.125f, 0, dummy, dummy, 0, NULL) == KVDEC_E_INVALID);
    CHECK(kvdec_append(NULL, dummy, dummy, NULL) == KVDEC_E_INVALID);
    CHECK(kvdec_append_attend(NULL, dummy, dummy, dummy, 4, 0.125f, 0, dummy, dummy, 0, NULL) ==
          KVDEC_E_INVALID);
    CHECK(kvdec_append_attend_at(NULL, lens, dummy, dummy, dummy, 4, 0.125f, 0, dummy, dummy, 0,
                                 NULL) == KVDEC_E_INVALID);
    CHECK(kvdec_reset_lens(NULL, lens, NULL) == KVDEC_E_INVALID);
    CHECK(kvdec_get_lens(NULL, lens) == KVDEC_E_INVALID);
    CHECK(kvdec_set_replay_mode(NULL, 64) == KVDEC_E_INVALID);
    CHECK(kvdec_workspace_bytes(NULL, 4) == 0);
    kvdec_cache_destroy(NULL);

    /* paged pool: invalid descriptors */
    kvdec_paged* p = NULL;
    CHECK(kvdec_paged_create(NULL, NULL, &p) == KVDEC_E_INVALID && p == NULL);
    kvdec_paged_desc pd;
    memset(&pd, 0, sizeof pd);
    pd.batch = 1;
    pd.n_kv_heads = 1;
    pd.head_dim = KVDEC_HEAD_DIM;
    pd.dtype = KVDEC_F32;
    pd.page_rows = 24;                                     /* not a power of two */
    pd.num_pages = 4;
    pd.max_pages_per_seq = 4;
    CHECK(kvdec_paged_create(&pd, NULL, &p) == KVDEC_E_SHAPE && p == NULL);
    CHECK(kvdec_paged_free_pages(NULL) == -1);
    CHECK(kvdec_paged_workspace_bytes(NULL, 4) == 0);
    CHECK(kvdec_paged_set_replay_mode(NULL, 64, NULL) == KVDEC_E_INVALID);
    CHECK(kvdec_set_replay_horizon(NULL, 4) == KVDEC_E_INVALID);
    CHECK(kvdec_paged_set_replay_horizon(NULL, 4) == KVDEC_E_INVALID);
    CHECK(kvdec_paged_prepare(NULL, 1, NULL) == KVDEC_E_INVALID);

    printf("%d failed\n", fails);
    return fails != 0;
}
