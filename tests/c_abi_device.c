/* A plain C99 caller of the zs3 device entry points with no Python or torch
 * in the process: hipMalloc'd buffers, the toy 2-layer model over N = 4
 * ranks (bf16), and checks whose answers follow from the definitions:
 *   - partition then gather (pack + unpack) gives every parameter back;
 *   - padding of a rank's shard is written as 0;
 *   - when every rank sends the same gradient, the averaged slice equals it
 *     bit for bit (N = 4 is a power of two, so sum / N is exact);
 *   - every bucket of a pass gathered in one launch gives the parameters back;
 *   - the rest of the last rank's step: the norm from the reduce-scatter's
 *     partial sums (and from the allocation-free call, bit for bit the
 *     same), the fp32 master from the shard, and one Adam step, each
 *     against the same IEEE float operations done here.
 * Built and run by tests/test_c_abi.py on a GPU; prints "ok". */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zs3.h"

static float widen_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t round_bf16(float f) {    /* round to nearest even; NaN stays NaN */
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static uint32_t bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

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

    /* (4) every bucket of a pass in one launch: buckets {0, 1} and {2, 3},
     * each with its own wire and gathered buffer; rank 0 gathers */
    {
        const int64_t bids[NP] = {0, 1, 2, 3};
        const int32_t starts[3] = {0, 2, 4};
        int64_t bchunk[2], bfull[2];
        void* bwire[2];
        void* bgath[2];
        void* owns[2];
        const void* rch[2 * N];
        int b;
        for (b = 0; b < 2; ++b) {
            CHECK(zs3_bucket_sizes(L, 2, bids + 2 * b, &bchunk[b], &bfull[b]) == ZS3_OK);
            HIP(hipMalloc(&bwire[b], (size_t)(N * bchunk[b]) * 2));
            HIP(hipMalloc(&bgath[b], (size_t)bfull[b] * 2));
            for (v = 0; v < N; ++v) {
                void* c = (char*)bwire[b] + (size_t)(v * bchunk[b]) * 2;
                rch[b * N + v] = c;
                if (v != 0)
                    CHECK(zs3_gather_coalesced(L, v, ZS3_BF16, ZS3_PACK, 2, bids + 2 * b, shards[v], c, NULL, NULL,
                                               NULL, NULL) == ZS3_OK);
            }
            owns[b] = (void*)rch[b * N];
        }
        CHECK(zs3_gather_coalesced_buckets(L, 0, ZS3_BF16, 2, starts, bids, shards[0], owns, rch, bgath, NULL) ==
              ZS3_OK);
        HIP(hipDeviceSynchronize());
        for (b = 0; b < 2; ++b) {
            HIP(hipMemcpy(g, bgath[b], (size_t)bfull[b] * 2, hipMemcpyDeviceToHost));
            CHECK(memcmp(g, host_full[2 * b], (size_t)numel[2 * b] * 2) == 0);
            CHECK(memcmp(g + numel[2 * b], host_full[2 * b + 1], (size_t)numel[2 * b + 1] * 2) == 0);
            HIP(hipFree(bwire[b]));
            HIP(hipFree(bgath[b]));
        }
    }

    /* (5) the rest of the last rank's step */
    {
        const int32_t rk = N - 1;
        int64_t n_slots = 0, lo = 0, hi = 0, e;
        void* grad = NULL;
        double* partials = NULL;
        double* sumsq = NULL;
        double* outd = NULL;      /* norm: [0] cached call, [1] allocation-free call */
        float* outs = NULL;       /* scale, same two */
        int32_t* outf = NULL;     /* non-finite flag, same two */
        float *master = NULL, *m = NULL, *vv = NULL;
        const void* src[NP * N];
        double host_sumsq[N + 1], got_sumsq[2][N + 1], total = 0.0, norm_ref, coef;
        double got_norm[2];
        float got_scale[2], scale_ref;
        int32_t got_flag[2];
        uint16_t* sh = (uint16_t*)malloc((size_t)shard_n * 2);
        uint16_t* gr = (uint16_t*)malloc((size_t)shard_n * 2);
        uint16_t* sh2 = (uint16_t*)malloc((size_t)shard_n * 2);
        float* hw = (float*)malloc((size_t)shard_n * 4);
        float* hm = (float*)malloc((size_t)shard_n * 4);
        float* hv = (float*)malloc((size_t)shard_n * 4);
        zs3_adam_params hp;

        CHECK(zs3_layout_norm_slots(L, &n_slots, NULL) == ZS3_OK && n_slots > 0);
        HIP(hipMalloc(&grad, (size_t)shard_n * 2));
        HIP(hipMalloc((void**)&partials, (size_t)n_slots * 8));
        HIP(hipMalloc((void**)&sumsq, (N + 1) * 8));
        HIP(hipMalloc((void**)&outd, 2 * 8));
        HIP(hipMalloc((void**)&outs, 2 * 4));
        HIP(hipMalloc((void**)&outf, 2 * 4));
        HIP(hipMalloc((void**)&master, (size_t)shard_n * 4));
        HIP(hipMalloc((void**)&m, (size_t)shard_n * 4));
        HIP(hipMalloc((void**)&vv, (size_t)shard_n * 4));

        /* every rank sends the full parameters as its gradient: the averaged
         * gradient is the shard, and rank v's partial sum of squares is the
         * sum over its own real elements (no persistent parameters: T = 0) */
        for (v = 0; v <= N; ++v) host_sumsq[v] = 0.0;
        for (v = 0; v < N; ++v)
            for (i = 0; i < NP; ++i) {
                CHECK(zs3_layout_own_range(L, ids[i], v, &lo, &hi) == ZS3_OK);
                for (e = lo; e < hi; ++e) {
                    const double x = (double)widen_bf16(host_full[i][e]);
                    host_sumsq[v] += x * x;
                }
            }
        for (i = 0; i < NP; ++i) {
            CHECK(zs3_layout_own_range(L, ids[i], rk, &lo, &hi) == ZS3_OK);
            for (v = 0; v < N; ++v) src[i * N + v] = (const char*)dev_full[i] + (size_t)lo * 2;
        }
        HIP(hipMemset(partials, 0xFF, (size_t)n_slots * 8));       /* NaN until written */
        CHECK(zs3_reduce_scatter_local(L, rk, ZS3_BF16, NP, ids, src, grad, partials, NULL) == ZS3_OK);
        for (i = 0; i < 2; ++i) {
            HIP(hipMemcpy(sumsq, host_sumsq, (N + 1) * 8, hipMemcpyHostToDevice));
            if (i == 0)
                CHECK(zs3_grad_norm_partials(L, rk, partials, sumsq, 1, 1.0, 1.0, outd, outs, outf, NULL) == ZS3_OK);
            else
                CHECK(zs3_grad_norm_partials_noalloc(L, rk, partials, sumsq, 1, 1.0, 1.0, outd + 1, outs + 1, outf + 1,
                                                     NULL) == ZS3_OK);
            HIP(hipDeviceSynchronize());
            HIP(hipMemcpy(got_sumsq[i], sumsq, (N + 1) * 8, hipMemcpyDeviceToHost));
        }
        HIP(hipMemcpy(got_norm, outd, 2 * 8, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(got_scale, outs, 2 * 4, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(got_flag, outf, 2 * 4, hipMemcpyDeviceToHost));
        for (v = 0; v < N; ++v) total += v == rk ? got_sumsq[0][rk] : host_sumsq[v];
        norm_ref = __builtin_sqrt(total);
        coef = 1.0 / (norm_ref + 1e-6);
        if (coef > 1.0) coef = 1.0;
        scale_ref = (float)coef;
        CHECK(__builtin_fabs(got_sumsq[0][rk] - host_sumsq[rk]) <= 1e-12 * host_sumsq[rk]);
        CHECK(got_sumsq[0][N] == 0.0);
        /* the norm is sqrt of the same double sum; the scale within one float ulp */
        CHECK(__builtin_fabs(got_norm[0] - norm_ref) <= 4e-16 * norm_ref && got_flag[0] == 0);
        CHECK(__builtin_fabs(got_scale[0] - scale_ref) <= 1.2e-7f * scale_ref);
        CHECK(norm_ref > 1.0);                                      /* the clip is active */
        /* the allocation-free call: the same bits */
        CHECK(memcmp(got_sumsq[0], got_sumsq[1], (N + 1) * 8) == 0);
        CHECK(memcmp(&got_norm[0], &got_norm[1], 8) == 0 && bits(got_scale[0]) == bits(got_scale[1]) &&
              got_flag[1] == 0);

        /* the fp32 master of the whole shard: the exact widening at real
         * positions, 0 at padding; both moments 0 */
        HIP(hipMemset(master, 0xFF, (size_t)shard_n * 4));
        HIP(hipMemset(m, 0xFF, (size_t)shard_n * 4));
        HIP(hipMemset(vv, 0xFF, (size_t)shard_n * 4));
        CHECK(zs3_init_master(L, rk, ZS3_BF16, 0, shard_n, shards[rk], master, m, vv, NULL) == ZS3_OK);
        HIP(hipDeviceSynchronize());
        HIP(hipMemcpy(sh, shards[rk], (size_t)shard_n * 2, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(gr, grad, (size_t)shard_n * 2, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(hw, master, (size_t)shard_n * 4, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(hm, m, (size_t)shard_n * 4, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(hv, vv, (size_t)shard_n * 4, hipMemcpyDeviceToHost));
        CHECK(memcmp(gr, sh, (size_t)shard_n * 2) == 0);
        for (i = 0; i < NP; ++i) {
            int64_t ps = 0, off = 0;
            CHECK(zs3_layout_param(L, ids[i], NULL, &ps, NULL, &off) == ZS3_OK);
            CHECK(zs3_layout_own_range(L, ids[i], rk, &lo, &hi) == ZS3_OK);
            for (e = 0; e < ps; ++e) {
                const float want = e < hi - lo ? widen_bf16(sh[off + e]) : 0.0f;
                if (bits(hw[off + e]) != bits(want) || bits(hm[off + e]) != 0 || bits(hv[off + e]) != 0) {
                    CHECK(bits(hw[off + e]) == bits(want) && bits(hm[off + e]) == 0 && bits(hv[off + e]) == 0);
                    break;
                }
            }
        }

        /* one Adam step (t = 1, no weight decay) with the norm's clip scale,
         * against the same float operations here (ISO C: no contraction) */
        hp.lr = 1e-3;
        hp.beta1 = 0.9;
        hp.beta2 = 0.999;
        hp.eps = 1e-8;
        hp.weight_decay = 0.0;
        hp.step = 1;
        CHECK(zs3_adam_step(L, rk, ZS3_BF16, 0, shard_n, master, m, vv, grad, shards[rk], outs, outf, &hp, NULL) ==
              ZS3_OK);
        HIP(hipDeviceSynchronize());
        {
            const float lr = (float)hp.lr, b1 = (float)hp.beta1, b2 = (float)hp.beta2;
            const float omb1 = (float)(1.0 - hp.beta1), omb2 = (float)(1.0 - hp.beta2);
            const float bc1 = (float)(1.0 - hp.beta1), bc2 = (float)(1.0 - hp.beta2), eps = (float)hp.eps;
            float* w2 = (float*)malloc((size_t)shard_n * 4);
            float* m2 = (float*)malloc((size_t)shard_n * 4);
            float* v2 = (float*)malloc((size_t)shard_n * 4);
            int bad = 0;
            HIP(hipMemcpy(w2, master, (size_t)shard_n * 4, hipMemcpyDeviceToHost));
            HIP(hipMemcpy(m2, m, (size_t)shard_n * 4, hipMemcpyDeviceToHost));
            HIP(hipMemcpy(v2, vv, (size_t)shard_n * 4, hipMemcpyDeviceToHost));
            HIP(hipMemcpy(sh2, shards[rk], (size_t)shard_n * 2, hipMemcpyDeviceToHost));
            for (i = 0; i < NP && !bad; ++i) {
                int64_t ps = 0, off = 0;
                CHECK(zs3_layout_param(L, ids[i], NULL, &ps, NULL, &off) == ZS3_OK);
                CHECK(zs3_layout_own_range(L, ids[i], rk, &lo, &hi) == ZS3_OK);
                for (e = 0; e < ps; ++e) {
                    const int64_t k = off + e;
                    float w = hw[k], mm = hm[k], va = hv[k];
                    uint16_t s16 = sh[k];
                    if (e < hi - lo) {
                        const float gg = widen_bf16(gr[k]) * got_scale[0];
                        float mh, vh, den;
                        mm = b1 * mm + omb1 * gg;
                        va = b2 * va + omb2 * (gg * gg);
                        mh = mm / bc1;
                        vh = va / bc2;
                        den = __builtin_sqrtf(vh) + eps;
                        w = w - lr * (mh / den);
                        s16 = round_bf16(w);
                    }
                    if (bits(w2[k]) != bits(w) || bits(m2[k]) != bits(mm) || bits(v2[k]) != bits(va) || sh2[k] != s16) {
                        CHECK(bits(w2[k]) == bits(w) && bits(m2[k]) == bits(mm) && bits(v2[k]) == bits(va) &&
                              sh2[k] == s16);
                        bad = 1;
                        break;
                    }
                }
            }
            free(w2);
            free(m2);
            free(v2);
        }
        HIP(hipFree(grad));
        HIP(hipFree(partials));
        HIP(hipFree(sumsq));
        HIP(hipFree(outd));
        HIP(hipFree(outs));
        HIP(hipFree(outf));
        HIP(hipFree(master));
        HIP(hipFree(m));
        HIP(hipFree(vv));
        free(sh);
        free(gr);
        free(sh2);
        free(hw);
        free(hm);
        free(hv);
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
