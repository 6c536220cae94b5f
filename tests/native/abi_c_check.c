/* The C ABI from plain C: include/dq.h compiles as C11, and the host-only
 * calls behave as documented without a GPU (plan creation and its checks,
 * options, sizes, layout, state errors before binding).  Prints "ok" and
 * exits 0, or names the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "dq.h"

#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            printf("failed: %s (line %d)\n", #cond, __LINE__);   \
            return 1;                                            \
        }                                                        \
    } while (0)

int main(void) {
    dq_plan *p = NULL;
    CHECK(dq_plan_create(256 * 1000, 8, DQ_RING, 5.0f, NULL) == DQ_ENULL);
    CHECK(dq_plan_create(255, 8, DQ_RING, 5.0f, &p) == DQ_EINVAL && p == NULL);
    CHECK(dq_plan_create(256 * 1000, 6, DQ_BUTTERFLY, 5.0f, &p) == DQ_EINVAL);
    CHECK(dq_plan_create(256 * 1000, 8, DQ_RING, 1.5f, &p) == DQ_EBUDGET);
    CHECK(dq_plan_create(256 * 1000, 8, DQ_BUTTERFLY, 5.0f, &p) == DQ_OK && p != NULL);

    CHECK(dq_plan_set_u64(p, DQ_OPT_SEED, 42) == DQ_OK);
    CHECK(dq_plan_set_u64(p, DQ_OPT_ROUNDING, 7) == DQ_EINVAL);
    CHECK(dq_plan_set_f64(p, DQ_OPT_EPS, 0.0) == DQ_EINVAL);

    const size_t ws = dq_workspace_bytes(p);
    dq_layout lay;
    memset(&lay, 0, sizeof lay);
    CHECK(ws > 0);
    CHECK(dq_workspace_layout(p, &lay) == DQ_OK);
    CHECK(lay.total == ws && lay.sumsq >= lay.sum + 4 * 1000);
    /* worst-case region of one part of m = 8: (256 + 20) bytes per SG of ceil(1000 / 8) */
    CHECK(dq_region_bytes_max(p, 8) >= (size_t)(276 * 125));
    CHECK(dq_arena_bytes(p) > 0);
    CHECK(dq_final_part(p, 5) == 5);

    /* every stage call before a workspace is bound is refused, without device work */
    int dummy[4];
    CHECK(dq_stats(p, 0, dummy, DQ_BF16, NULL) == DQ_EWORKSPACE);
    CHECK(dq_allocate(p, NULL) == DQ_EWORKSPACE);
    CHECK(dq_reorder(p, NULL) == DQ_EWORKSPACE);
    CHECK(dq_stats(NULL, 0, dummy, DQ_BF16, NULL) == DQ_ENULL);

    CHECK(strlen(dq_status_string(DQ_ESTATE)) > 0);
    CHECK(dq_version() >= 1);
    dq_plan_destroy(p);
    dq_plan_destroy(NULL);
    printf("ok\n");
    return 0;
}
