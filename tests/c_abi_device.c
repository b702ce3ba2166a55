/* A plain C99 caller of the zs3 device entry points with no Python or torch
 * in the process: hipMalloc'd buffers, the toy 2-layer model over N = 4
 * ranks (bf16), and three checks whose answers follow from the definitions:
 *   - partition then gather (pack + unpack) gives every parameter back;
 *   - padding of a rank's shard is written as 0;
 *   - when every rank sends the same gradient, the averaged slice equals it
 *     bit for bit (N = 4 is a power of two, so sum / N is exact).
 * Built and run by tests/test_c_abi.py on a GPU; prints "ok". */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zs3.h"

#define N 4
#define NP 4
static const int64_t ids[NP] = {0, 1, 2, 3};
static const int64_t numel[NP] = {2048, 33, 511, 16};   /* 33 and 511 leave padding on the last ranks */

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            printf("check failed at line %d: %s\n", __LINE__, #cond);     \
            ++failures;                                                    \
        }                                                                  \
    } while (0)
#define HIP(x) CHECK((x) == hipSuccess)

int main(void) {
    zs3_layout_t L = NULL;
    int64_t shard_n = 0, total = 0, chunk = 0, full_n = 0, offs[NP];
    int i, r, v;
    uint16_t* host_full[NP];
    void* dev_full[NP];
    void* shards[N];
    void* wire = NULL;
    void* gathered = NULL;
    const void* chunks[N];
    uint16_t *h = NULL, *g = NULL;

    CHECK(zs3_layout_create(N, 0, NP, ids, numel, &L) == ZS3_OK);
    CHECK(zs3_layout_info(L, NULL, NULL, NULL, &shard_n, NULL) == ZS3_OK);
    CHECK(zs3_bucket_sizes(L, NP, ids, &chunk, &full_n) == ZS3_OK && chunk == shard_n);
    for (i = 0; i < NP; ++i) total += numel[i];
    CHECK(full_n == total);

    /* full parameters: distinct bf16 bit patterns */
    for (i = 0; i < NP; ++i) {
        int64_t k;
        host_full[i] = (uint16_t*)malloc((size_t)numel[i] * 2);
        for (k = 0; k < numel[i]; ++k) host_full[i][k] = (uint16_t)(0x3C00 + ((i * 4099 + k * 7) & 0x3FF));
        HIP(hipMalloc(&dev_full[i], (size_t)numel[i] * 2));
        HIP(hipMemcpy(dev_full[i], host_full[i], (size_t)numel[i] * 2, hipMemcpyHostToDevice));
    }
    HIP(hipMalloc(&wire, (size_t)(N * chunk) * 2));
    HIP(hipMalloc(&gathered, (size_t)full_n * 2));
    h = (uint16_t*)malloc((size_t)shard_n * 2);
    g = (uint16_t*)malloc((size_t)full_n * 2);

    /* (1) partition every rank, check each shard against the definition */
    for (r = 0; r < N; ++r) {
        HIP(hipMalloc(&shards[r], (size_t)shard_n * 2));
        HIP(hipMemset(shards[r], 0xFF, (size_t)shard_n * 2));
        CHECK(zs3_partition(L, r, ZS3_BF16, NP, ids, (const void* const*)dev_full, shards[r], NULL) == ZS3_OK);
        HIP(hipDeviceSynchronize());
        HIP(hipMemcpy(h, shards[r], (size_t)shard_n * 2, hipMemcpyDeviceToHost));
        for (i = 0; i < NP; ++i) {
            int64_t ps = 0, off = 0, k;
            int32_t pers = 0;
            CHECK(zs3_layout_param(L, ids[i], NULL, &ps, &pers, &off) == ZS3_OK);
            for (k = 0; k < ps; ++k) {
                const int64_t j = r * ps + k;
                const uint16_t want = j < numel[i] ? host_full[i][j] : 0;
                if (h[off + k] != want) {
                    CHECK(h[off + k] == want);
                    break;
                }
            }
        }
    }

    /* (2) every rank packs its chunk into the wire; rank 0 unpacks */
    for (r = 0; r < N; ++r) {
        void* own = (char*)wire + (size_t)(r * chunk) * 2;
        CHECK(zs3_gather_coalesced(L, r, ZS3_BF16, ZS3_PACK, NP, ids, shards[r], own, NULL, NULL, NULL, NULL) == ZS3_OK);
        chunks[r] = own;
    }
    CHECK(zs3_gather_coalesced(L, 0, ZS3_BF16, ZS3_UNPACK, NP, ids, NULL, NULL, chunks, gathered, offs, NULL) == ZS3_OK);
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(g, gathered, (size_t)full_n * 2, hipMemcpyDeviceToHost));
    for (i = 0; i < NP; ++i) CHECK(memcmp(g + offs[i], host_full[i], (size_t)numel[i] * 2) == 0);

    /* (3) identical gradients on every rank average to themselves */
    {
        void* grad = NULL;
        const void* src[NP * N];
        int64_t lo = 0, hi = 0;
        HIP(hipMalloc(&grad, (size_t)shard_n * 2));
        for (r = 0; r < N; ++r) {
            for (i = 0; i < NP; ++i) {
                CHECK(zs3_layout_own_range(L, ids[i], r, &lo, &hi) == ZS3_OK);
                for (v = 0; v < N; ++v) src[i * N + v] = (const char*)dev_full[i] + (size_t)lo * 2;
            }
            CHECK(zs3_reduce_scatter_local(L, r, ZS3_BF16, NP, ids, src, grad, NULL, NULL) == ZS3_OK);
            HIP(hipDeviceSynchronize());
            HIP(hipMemcpy(h, grad, (size_t)shard_n * 2, hipMemcpyDeviceToHost));
            {
                uint16_t* s = (uint16_t*)malloc((size_t)shard_n * 2);
                HIP(hipMemcpy(s, shards[r], (size_t)shard_n * 2, hipMemcpyDeviceToHost));
                CHECK(memcmp(h, s, (size_t)shard_n * 2) == 0);     /* the shard holds the same slices and zeros */
                free(s);
            }
        }
        HIP(hipFree(grad));
    }

    for (r = 0; r < N; ++r) HIP(hipFree(shards[r]));
    for (i = 0; i < NP; ++i) {
        HIP(hipFree(dev_full[i]));
        free(host_full[i]);
    }
    HIP(hipFree(wire));
    HIP(hipFree(gathered));
    free(h);
    free(g);
    zs3_layout_destroy(L);
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
