/* Host sanitizer run of liblosa.so's argument checks and size queries: the
 * library is built with AddressSanitizer and UndefinedBehaviorSanitizer on its
 * host code, and every call below must return its status without launching
 * anything (no GPU is needed).  Any out-of-bounds access or undefined operation
 * in the host code aborts the run. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "losa.h"

static int fails = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "failed at line %d: %s\n", __LINE__, #cond); \
            ++fails;                                                  \
        }                                                             \
    } while (0)

static losa_shape base(void) {
    losa_shape s;
    memset(&s, 0, sizeof s);
    s.n_seq = 8; s.block = 32; s.n_qhead = 32; s.n_kvhead = 8; s.head_dim = 128; s.page_size = 16;
    s.budget_tokens = 256; s.n_active = 8; s.max_prefix_len = 65536; s.dtype = LOSA_BF16;
    s.kv_tokens = 8 * 65536; s.softmax_scale = 0.0f; s.flags = 0;
    return s;
}

int main(void) {
    void *p = (void *)(uintptr_t)(1u << 20);      /* never dereferenced */
    void *odd = (void *)(uintptr_t)((1u << 20) + 2);
    for (int st = -2; st < 8; ++st) EXPECT(losa_status_string(st) != NULL);
    /* size queries over valid and invalid shapes */
    for (int d = 32; d <= 160; d += 32)
        for (int b = 0; b <= 70; b += 7)
            for (int a = -1; a <= b + 1; a += 5)
                for (int budget = 0; budget <= 512; budget += 80) {
                    losa_shape s = base();
                    s.head_dim = d; s.block = b; s.n_active = a; s.budget_tokens = budget;
                    size_t m = losa_page_meta_bytes(&s), w = losa_workspace_bytes(&s);
                    int32_t cap = losa_union_capacity(&s);
                    EXPECT((m == 0) == (w == 0) && (cap < 0) == (w == 0));
                }
    losa_shape s = base();
    EXPECT(losa_workspace_bytes(&s) > 0 && losa_page_meta_bytes(&s) > 0);
    s.kv_tokens = 15; EXPECT(losa_workspace_bytes(&s) == 0);
    s = base(); s.flags = 8; EXPECT(losa_workspace_bytes(&s) == 0);
    s = base(); s.max_prefix_len = -1; EXPECT(losa_workspace_bytes(&s) == 0);
    s = base(); s.n_qhead = 33; EXPECT(losa_workspace_bytes(&s) == 0);
    EXPECT(losa_workspace_bytes(NULL) == 0 && losa_union_capacity(NULL) == -1);
    /* entry points: bad arguments are rejected before anything is enqueued */
    s = base();
    const size_t need = losa_workspace_bytes(&s);
    EXPECT(losa_build_page_meta(NULL, p, p, p, NULL, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_build_page_meta(&s, NULL, p, p, NULL, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_build_page_meta(&s, p, NULL, p, NULL, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_build_page_meta(&s, odd, p, p, NULL, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_build_page_meta(&s, p, p, p, odd, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_update_page_meta(&s, p, p, p, NULL, p, -1, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_update_page_meta(&s, p, p, p, NULL, NULL, 16, p, NULL) == LOSA_ERR_INVALID_ARG);
    EXPECT(losa_dense_first_step(&s, p, p, p, p, p, p, p, NULL, p, p, p, NULL, p, need - 1, NULL) ==
           LOSA_ERR_WORKSPACE);
    EXPECT(losa_dense_first_step(&s, p, p, p, p, p, NULL, p, NULL, p, p, p, NULL, p, need, NULL) ==
           LOSA_ERR_INVALID_ARG);
    EXPECT(losa_step(&s, p, p, p, p, p, p, p, p, p, NULL, p, p, p, NULL, p, need - 1, NULL) ==
           LOSA_ERR_WORKSPACE);
    EXPECT(losa_step(&s, p, odd, p, p, p, p, p, p, p, NULL, p, p, p, NULL, p, need, NULL) ==
           LOSA_ERR_INVALID_ARG);
    losa_debug dbg;
    memset(&dbg, 0, sizeof dbg);
    dbg.union_idx = (int32_t *)p;
    dbg.union_cap = losa_union_capacity(&s) - 1;
    EXPECT(losa_step(&s, p, p, p, p, p, p, p, p, p, NULL, p, p, p, &dbg, p, need, NULL) ==
           LOSA_ERR_INVALID_ARG);
    /* the allocation-free step: the ragged batch's scratch need exceeds the static array */
    EXPECT(losa_step_noalloc(&s, p, p, p, p, p, p, p, p, p, NULL, p, p, p, NULL, NULL) ==
           LOSA_ERR_SCRATCH);
    s.block = 65;
    EXPECT(losa_step_noalloc(&s, p, p, p, p, p, p, p, p, p, NULL, p, p, p, NULL, NULL) ==
           LOSA_ERR_UNSUPPORTED);
    printf("api sanitizer run: %d failed checks\n", fails);
    return fails != 0;
}
