// Seeded random exercise of the zs3 host entry points (layout, queries,
// bucket and sub-group planning, the coordinator, argument errors, and the
// aliasing checks of the device entry points, which reject a call before
// any device work), for
// AddressSanitizer / UBSan / ThreadSanitizer builds of the host code.  No
// device calls.  Runs once on the main thread, then on four threads at once,
// each with its own seed and its own layouts (no state is shared between
// layouts apart from the allocation-free norm's device scratch, which these
// calls never reach; the last error is per thread).  Built and run by
// tests/test_host_sanitizers.py; prints "ok".
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "zs3.h"

namespace {

thread_local uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
int64_t uniform(int64_t lo, int64_t hi) { return lo + static_cast<int64_t>(next() % static_cast<uint64_t>(hi - lo + 1)); }

std::atomic<int> failures{0};
void check(bool ok, const char* what, int iter) {
    if (!ok) {
        std::printf("iteration %d: %s\n", iter, what);
        ++failures;
    }
}

void fuzz(uint64_t seed, int iters) {
    g_state = seed;
    for (int it = 0; it < iters; ++it) {
        const int32_t N = static_cast<int32_t>(uniform(1, 70));
        const int32_t n = static_cast<int32_t>(uniform(0, 40));
        const int64_t T = uniform(0, 3) == 0 ? 0 : uniform(0, 5000);
        std::vector<int64_t> ids(n), numel(n);
        for (int32_t i = 0; i < n; ++i) {
            ids[i] = 3 * i + uniform(0, 2);
            numel[i] = uniform(0, 4) == 0 ? uniform(1, 20) : uniform(1, 200000);
        }
        for (int32_t i = n - 1; i > 0; --i) std::swap(ids[i], ids[uniform(0, i)]);
        zs3_layout_t L = nullptr;
        check(zs3_layout_create(N, T, n, ids.data(), numel.data(), &L) == ZS3_OK, "create", it);
        if (L == nullptr) continue;
        int64_t shard = 0, bytes = 0, sum = 0;
        check(zs3_layout_totals(L, &shard, &bytes) == ZS3_OK && bytes == 16 * shard, "totals", it);
        for (int32_t i = 0; i < n; ++i) {
            int64_t d = 0, nm = 0, ps = 0, off = 0, lo = 0, hi = 0;
            int32_t pers = 0;
            check(zs3_layout_param_at(L, i, &d, &nm, &ps, &pers, &off) == ZS3_OK && off == sum, "param_at", it);
            sum += ps;
            const int32_t r = static_cast<int32_t>(uniform(0, N - 1));
            check(zs3_layout_own_range(L, d, r, &lo, &hi) == ZS3_OK && lo <= hi && (hi <= nm || hi == lo), "own_range", it);
        }
        check(sum == shard, "shard sum", it);
        // planning with a too-small capacity, then the right one
        for (int32_t kind : {ZS3_GATHER_BUCKETS, ZS3_REDUCE_BUCKETS}) {
            const int64_t limit = uniform(1, 400000);
            int32_t nb = 0;
            std::vector<int32_t> starts(1);
            std::vector<int64_t> out(n + 1);
            zs3_status s = zs3_plan_buckets(L, kind, limit, 0, &nb, starts.data(), out.data());
            if (s == ZS3_EINVAL) {
                starts.assign(nb + 1, 0);
                s = zs3_plan_buckets(L, kind, limit, nb + 1, &nb, starts.data(), out.data());
            }
            check(s == ZS3_OK, "plan_buckets", it);
            if (s == ZS3_OK && nb > 0 && kind == ZS3_GATHER_BUCKETS) {
                int64_t chunk = 0, full = 0;
                check(zs3_bucket_sizes(L, starts[1] - starts[0], out.data(), &chunk, &full) == ZS3_OK, "sizes", it);
            }
        }
        {
            int32_t ng = 0;
            std::vector<int64_t> be(2);
            zs3_status s = zs3_sub_groups(L, uniform(1, 300000), 0, &ng, be.data());
            if (s == ZS3_EINVAL && ng > 0) {
                be.assign(2 * ng, 0);
                s = zs3_sub_groups(L, uniform(1, 300000), ng, &ng, be.data());
            }
        }
        // coordinator over random modules (parameters may repeat across modules)
        if (n > 0) {
            const int32_t nm = static_cast<int32_t>(uniform(1, 12));
            std::vector<int32_t> mstart(nm + 1, 0);
            std::vector<int64_t> mids;
            for (int32_t m = 0; m < nm; ++m) {
                const int32_t k = static_cast<int32_t>(uniform(0, 4));
                std::vector<int64_t> pick;
                for (int32_t j = 0; j < k; ++j) {
                    const int64_t d = ids[uniform(0, n - 1)];
                    bool dup = false;
                    for (int64_t x : pick) dup |= x == d;
                    if (!dup) pick.push_back(d);
                }
                for (int64_t d : pick) mids.push_back(d);
                mstart[m + 1] = static_cast<int32_t>(mids.size());
            }
            zs3_coord_config cfg;
            cfg.prefetch_bucket_size = uniform(0, 300000);
            cfg.max_live_parameters = uniform(1, 1000000);
            cfg.max_reuse_distance = uniform(0, 500000);
            zs3_coord_t C = nullptr;
            check(zs3_coord_create(L, nm, mstart.data(), mids.data(), &cfg, &C) == ZS3_OK, "coord_create", it);
            if (C != nullptr) {
                std::vector<int64_t> buf(mids.size() + n + 1);
                int32_t kinds[2], gst[3], cnt = 0, mode = 0;
                for (int step = 0; step < 4; ++step) {
                    const int32_t len = static_cast<int32_t>(uniform(1, 2 * nm));
                    for (int32_t j = 0; j < len; ++j) {
                        const int32_t m = step < 3 ? (j % nm) : static_cast<int32_t>(uniform(0, nm - 1));
                        if (zs3_coord_fetch(C, m, &cnt, kinds, gst, buf.data()) == ZS3_OK)
                            (void)zs3_coord_release(C, m, &cnt, buf.data());
                    }
                    (void)zs3_coord_release_all(C, &cnt, buf.data());
                    check(zs3_coord_reset_step(C, &mode) == ZS3_OK, "reset", it);
                }
                uint64_t a = 0, b = 0;
                int32_t f = 0;
                (void)zs3_coord_trace_signature(C, &a, &b, &f);
                check(zs3_coord_fetch(C, nm, &cnt, kinds, gst, buf.data()) == ZS3_EINVAL, "bad module", it);
                zs3_coord_destroy(C);
            }
        }
        // aliasing: a source inside a written range, or two outputs that
        // touch, is rejected before any device work (the sort-and-sweep
        // over every byte range of the call; the addresses are never used)
        if (n > 0) {
            const uintptr_t base = uintptr_t(1) << 40;
            const int32_t r = static_cast<int32_t>(uniform(0, N - 1));
            std::vector<const void*> src(static_cast<size_t>(n) * N);
            std::vector<std::pair<int64_t, int64_t>> written;
            int64_t victim = -1;
            for (int32_t i = 0; i < n; ++i) {
                int64_t nm = 0, ps = 0, off = 0, lo = 0, hi = 0;
                int32_t pers = 0;
                check(zs3_layout_param(L, ids[i], &nm, &ps, &pers, &off) == ZS3_OK, "param", it);
                check(zs3_layout_own_range(L, ids[i], r, &lo, &hi) == ZS3_OK, "own range", it);
                if (hi > lo && victim < 0) victim = i;
                written.emplace_back(off, ps);
                for (int32_t v = 0; v < N; ++v)
                    src[static_cast<size_t>(i) * N + v] =
                        reinterpret_cast<const void*>(base + (uintptr_t(1) << 34) + 2 * uniform(0, 1 << 28));
            }
            if (victim >= 0) {
                // the victim's first source starts inside some parameter's written range
                const auto& w = written[uniform(0, n - 1)];
                const uintptr_t grad = base;
                src[static_cast<size_t>(victim) * N] =
                    reinterpret_cast<const void*>(grad + 2 * (w.first + uniform(0, w.second - 1)));
                check(zs3_reduce_scatter_local(L, r, ZS3_BF16, n, ids.data(), src.data(),
                                               reinterpret_cast<void*>(grad), nullptr, nullptr) == ZS3_EALIAS,
                      "reduce-scatter alias", it);
            }
            // two buckets whose gathered buffers overlap
            std::vector<int64_t> part;
            for (int32_t i = 0; i < n; ++i) {
                int32_t pers = 0;
                (void)zs3_layout_param(L, ids[i], nullptr, nullptr, &pers, nullptr);
                if (!pers) part.push_back(ids[i]);
            }
            if (part.size() >= 2) {
                const int32_t starts[3] = {0, 1, 2};
                const uintptr_t shard = base, full0 = base + (uintptr_t(1) << 36);
                void* owns[2] = {reinterpret_cast<void*>(base + (uintptr_t(1) << 35)),
                                 reinterpret_cast<void*>(base + (uintptr_t(1) << 35) + (uintptr_t(1) << 30))};
                void* fulls[2] = {reinterpret_cast<void*>(full0), reinterpret_cast<void*>(full0)};   // same start
                std::vector<const void*> rch(2 * static_cast<size_t>(N));
                for (int32_t b = 0; b < 2; ++b)
                    for (int32_t v = 0; v < N; ++v)
                        rch[static_cast<size_t>(b) * N + v] =
                            v == r ? owns[b]
                                   : reinterpret_cast<const void*>(base + (uintptr_t(1) << 37) +
                                                                   (uintptr_t(b * N + v) << 29));
                check(zs3_gather_coalesced_buckets(L, r, ZS3_BF16, 2, starts, part.data(),
                                                   reinterpret_cast<const void*>(shard), owns, rch.data(), fulls,
                                                   nullptr) == ZS3_EALIAS,
                      "gather buckets alias", it);
            }
        }
        // argument errors of the entry points that take plain ranges
        {
            float* fake = reinterpret_cast<float*>(uintptr_t(1) << 40);
            check(zs3_init_master(L, 0, ZS3_BF16, 1, 0, fake, fake, nullptr, nullptr, nullptr) == ZS3_EINVAL,
                  "init range", it);
            check(zs3_grad_norm_partials_noalloc(L, 0, nullptr, nullptr, 0, 1.0, 1.0, nullptr, nullptr, nullptr,
                                                 nullptr) == ZS3_EINVAL,
                  "noalloc null", it);
        }
        // argument errors
        check(zs3_layout_param(L, -7, nullptr, nullptr, nullptr, nullptr) == ZS3_ENOTFOUND, "not found", it);
        check(zs3_layout_own_range(L, n > 0 ? ids[0] : 0, N, nullptr, nullptr) != ZS3_OK, "bad rank", it);
        zs3_layout_destroy(L);
    }
}

}  // namespace

int main() {
    fuzz(0x9E3779B97F4A7C15ull, 400);
    {
        const int64_t d[2] = {1, 1}, m[2] = {5, 5};
        zs3_layout_t L = nullptr;
        check(zs3_layout_create(2, 0, 2, d, m, &L) == ZS3_EDUPID && L == nullptr, "dup", -1);
    }
    // four threads at once; then the last error stays per thread
    std::vector<std::thread> pool;
    for (int t = 0; t < 4; ++t) pool.emplace_back(fuzz, 1000003ull * (t + 1), 150);
    for (auto& th : pool) th.join();
    {
        const int64_t d[2] = {1, 1}, m[2] = {5, 5};
        zs3_layout_t L = nullptr;
        (void)zs3_layout_create(2, 0, 2, d, m, &L);     // fails on this thread: duplicate ds_id
        std::string other;
        std::thread th([&] {
            const int64_t one = 0, n = 4;
            zs3_layout_t M = nullptr;
            (void)zs3_layout_create(1, 0, 1, &one, &n, &M);   // succeeds on another thread
            other = zs3_last_error();
            zs3_layout_destroy(M);
        });
        th.join();
        check(std::strlen(zs3_last_error()) > 0, "own thread's error kept", -2);
        check(other.find("duplicate") == std::string::npos, "error leaked to another thread", -2);
    }
    if (failures == 0) std::printf("ok\n");
    return failures == 0 ? 0 : 1;
}
