/* A plain C99 caller of the zs3 C ABI: host-only entry points (layout,
 * planning, coordinator, errors), so it runs without a GPU.  Built and run
 * by tests/test_c_abi.py; prints "ok" and returns 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "zs3.h"

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            printf("check failed at line %d: %s\n", __LINE__, #cond);     \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

int main(void) {
    /* the toy 2-layer model: [64,32], [32], [32,16], [16] over N = 4 ranks */
    const int64_t ids[4] = {0, 1, 2, 3};
    const int64_t numel[4] = {2048, 32, 512, 16};
    zs3_layout_t L = NULL;
    int32_t world = 0, n_params = 0;
    int64_t threshold = -1, shard = 0, bytes = 0;
    int64_t ps = 0, off = 0, nm = 0, lo = 0, hi = 0;
    int32_t pers = -1;
    int32_t nb = 0, starts[8];
    int64_t order[4];
    int64_t be[8];
    int32_t ng = 0;
    int64_t chunk = 0, full = 0;

    CHECK(zs3_abi_version() == ZS3_ABI_VERSION);
    CHECK(zs3_layout_create(4, 0, 4, ids, numel, &L) == ZS3_OK && L != NULL);
    CHECK(zs3_layout_info(L, &world, &threshold, &n_params, &shard, &bytes) == ZS3_OK);
    CHECK(world == 4 && threshold == 0 && n_params == 4);
    CHECK(shard == 652 && bytes == 16 * 652);            /* 16 Psi / N with Psi = 2,608 */
    shard = bytes = 0;
    CHECK(zs3_layout_totals(L, &shard, &bytes) == ZS3_OK && shard == 652 && bytes == 10432);
    CHECK(zs3_layout_totals(NULL, &shard, &bytes) == ZS3_EINVAL);
    CHECK(zs3_layout_param(L, 2, &nm, &ps, &pers, &off) == ZS3_OK);
    CHECK(nm == 512 && ps == 128 && pers == 0 && off == 512 + 8);
    CHECK(zs3_layout_own_range(L, 0, 3, &lo, &hi) == ZS3_OK && lo == 1536 && hi == 2048);
    CHECK(zs3_bucket_sizes(L, 4, ids, &chunk, &full) == ZS3_OK && chunk == 652 && full == 2608);

    CHECK(zs3_plan_buckets(L, ZS3_GATHER_BUCKETS, 1000000, 8, &nb, starts, order) == ZS3_OK);
    CHECK(nb == 1 && starts[0] == 0 && starts[1] == 4 && order[0] == 0 && order[3] == 3);
    CHECK(zs3_plan_buckets(L, ZS3_REDUCE_BUCKETS, 600, 8, &nb, starts, order) == ZS3_OK);
    CHECK(nb == 2 && order[0] == 3 && order[3] == 0);    /* descending ds_id: {3,2,1} holds 560, then {0} */
    CHECK(zs3_plan_buckets(L, ZS3_REDUCE_BUCKETS, 600, 1, &nb, starts, order) == ZS3_EINVAL && nb == 2);
    CHECK(zs3_sub_groups(L, 600, 4, &ng, be) == ZS3_OK && ng == 2 && be[1] == 520 && be[3] == 652); /* 512+8 | 128+4 */

    /* errors: nothing thrown, a status and a message */
    {
        const int64_t dup[2] = {5, 5};
        const int64_t two[2] = {1, 1};
        zs3_layout_t bad = NULL;
        CHECK(zs3_layout_create(2, 0, 2, dup, two, &bad) == ZS3_EDUPID && bad == NULL);
        CHECK(strlen(zs3_last_error()) > 0);
        CHECK(strlen(zs3_status_str(ZS3_EDUPID)) > 0);
        CHECK(zs3_layout_param(L, 99, &nm, &ps, &pers, &off) == ZS3_ENOTFOUND);
        CHECK(zs3_layout_create(0, 0, 2, ids, numel, &bad) == ZS3_EINVAL);
    }

    /* persistence: numel < threshold stays whole */
    {
        zs3_layout_t P = NULL;
        CHECK(zs3_layout_create(4, 100, 4, ids, numel, &P) == ZS3_OK);
        CHECK(zs3_layout_param(P, 1, &nm, &ps, &pers, &off) == ZS3_OK && pers == 1 && ps == 32);
        CHECK(zs3_layout_param(P, 2, &nm, &ps, &pers, &off) == ZS3_OK && pers == 0 && ps == 128);
        zs3_layout_destroy(P);
    }

    /* the coordinator: two modules, record then complete */
    {
        const int32_t mstart[3] = {0, 2, 4};
        const int64_t mids[4] = {0, 1, 2, 3};
        zs3_coord_config cfg;
        zs3_coord_t C = NULL;
        int32_t n = 0, kinds[2], gstarts[3], mode = -1, tl = 0, inv = 0, nf = 0;
        int64_t got[4], live = -1;
        uint64_t so = 0, sp = 0;
        int step, m;
        cfg.prefetch_bucket_size = 1000000;
        cfg.max_live_parameters = 1000000;
        cfg.max_reuse_distance = 0;
        CHECK(zs3_coord_create(L, 2, mstart, mids, &cfg, &C) == ZS3_OK);
        CHECK(zs3_coord_reset_step(C, &mode) == ZS3_OK && mode == ZS3_TRACE_RECORD);
        for (step = 0; step < 2; ++step) {
            for (m = 0; m < 2; ++m) {
                CHECK(zs3_coord_fetch(C, m, &n, kinds, gstarts, got) == ZS3_OK);
                if (step == 0 || m == 0) {      /* recording, or the first module of a complete trace */
                    CHECK(n >= 1 && kinds[0] == ZS3_GATHER_CURRENT);
                }
                CHECK(zs3_coord_release(C, m, &n, got) == ZS3_OK);
            }
            CHECK(zs3_coord_reset_step(C, &mode) == ZS3_OK);
            CHECK(mode == ZS3_TRACE_COMPLETE);
        }
        CHECK(zs3_coord_info(C, &mode, &live, &tl, &inv) == ZS3_OK && tl == 2 && inv == 0 && live == 0);
        CHECK(zs3_coord_trace_signature(C, &so, &sp, &nf) == ZS3_OK && nf == 2 && so != 0 && sp != 0);
        CHECK(zs3_coord_fetch(C, 5, &n, kinds, gstarts, got) == ZS3_EINVAL);
        zs3_coord_destroy(C);
    }

    zs3_layout_destroy(L);
    zs3_layout_destroy(NULL);
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
