// The trace-driven fetch/release coordinator of ZeRO-3: host-only planning
// of which parameters to all-gather (now, or ahead of time) and which to
// release, exported through the C ABI in zs3.h.
//
// Pages cited: [codex] "03 · ZeRO-3: parameter sharding and the all-gather
// schedule" (ai-reference-codex), sections 5.1 (trace), 5.2 (fetch), 5.3
// (release) and 7 (dynamic graphs, ordering, cross-rank consistency).
//
// Data structures: parameters are held by layout index; each module keeps
// its partitioned parameters in ascending ds_id; a complete trace keeps,
// per parameter, the sorted trace positions that use it and the prefix
// sums of module sizes along the trace, so that the reuse test of a
// release is a binary search and a subtraction instead of a scan.

#include "zs3.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

// Shared with api.cpp: the thread's last error message and the layout's
// parameter facts.
namespace zs3 {
zs3_status set_error(zs3_status s, const char* msg);
bool layout_param(zs3_layout_t L, int64_t ds_id, int64_t* numel, bool* persistent);
}  // namespace zs3

namespace {

zs3_status fail(zs3_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return zs3::set_error(s, buf);
}

zs3_status ok() { return zs3::set_error(ZS3_OK, ""); }

uint64_t fnv1a64(const std::vector<int64_t>& v) {
    uint64_t h = 14695981039346656037ull;
    for (int64_t x : v) {
        const uint64_t u = static_cast<uint64_t>(x);
        for (int i = 0; i < 8; ++i) {
            h ^= (u >> (8 * i)) & 0xffu;
            h *= 1099511628211ull;
        }
    }
    return h;
}

}  // namespace

struct zs3_coord {
    // parameters (dense index)
    std::vector<int64_t> ds_id, numel;
    std::vector<char> persistent;
    std::unordered_map<int64_t, int32_t> index;
    // modules: partitioned parameters (ascending ds_id) and their total size
    std::vector<std::vector<int32_t>> mod;
    std::vector<int64_t> mod_size;
    zs3_coord_config cfg{};

    int32_t mode = ZS3_TRACE_INVALID;
    std::vector<int8_t> status;
    int64_t live = 0;
    std::vector<int32_t> trace;                       // module per trace position
    std::vector<std::pair<int32_t, int32_t>> script;  // (trace position, parameter)
    std::vector<std::vector<int32_t>> uses;           // parameter -> trace positions (complete trace)
    std::vector<int64_t> prefix;                      // prefix[j] = sum of module sizes at positions < j
    int32_t step_pos = 0;
    size_t cursor = 0;
    std::vector<int32_t> marked;                      // latest script position the prefetcher popped
    std::vector<int32_t> fetched_at;                  // module -> trace position of its fetch, -1 if none
    int32_t invalidations = 0;

    void invalidate() {
        mode = ZS3_TRACE_INVALID;
        ++invalidations;
    }

    void build_script() {
        script.clear();
        uses.assign(ds_id.size(), {});
        prefix.assign(trace.size() + 1, 0);
        for (size_t k = 0; k < trace.size(); ++k) {
            prefix[k + 1] = prefix[k] + mod_size[trace[k]];
            for (int32_t p : mod[trace[k]]) {
                script.emplace_back(static_cast<int32_t>(k), p);
                uses[p].push_back(static_cast<int32_t>(k));
            }
        }
    }

    // A later trace position uses p within max_reuse_distance elements of
    // module sizes strictly between ([codex] 5.3).
    bool reused_soon(int32_t p, int32_t k) const {
        const auto& u = uses[p];
        auto it = std::upper_bound(u.begin(), u.end(), k);
        if (it == u.end()) return false;
        return prefix[*it] - prefix[k + 1] <= cfg.max_reuse_distance;
    }
};

namespace {

zs3_status check_coord(const zs3_coord* c) {
    if (c == nullptr) return fail(ZS3_EINVAL, "coordinator is NULL");
    return ZS3_OK;
}

zs3_status check_module(const zs3_coord* c, int32_t m) {
    if (m < 0 || m >= static_cast<int32_t>(c->mod.size()))
        return fail(ZS3_EINVAL, "module %d outside [0, %zu)", m, c->mod.size());
    return ZS3_OK;
}

// Writes the ascending ds_ids of `ps` (dense indices) to out.
int32_t put_ids(const zs3_coord* c, std::vector<int32_t> ps, int64_t* out) {
    std::sort(ps.begin(), ps.end(), [&](int32_t a, int32_t b) { return c->ds_id[a] < c->ds_id[b]; });
    for (size_t i = 0; i < ps.size(); ++i) out[i] = c->ds_id[ps[i]];
    return static_cast<int32_t>(ps.size());
}

}  // namespace

extern "C" {

zs3_status zs3_coord_create(zs3_layout_t layout, int32_t n_modules, const int32_t* module_start,
                            const int64_t* module_ds_ids, const zs3_coord_config* cfg, zs3_coord_t* out) {
    if (out == nullptr) return fail(ZS3_EINVAL, "out is NULL");
    *out = nullptr;
    if (layout == nullptr || cfg == nullptr) return fail(ZS3_EINVAL, "layout or cfg is NULL");
    if (n_modules < 0 || (n_modules > 0 && module_start == nullptr)) return fail(ZS3_EINVAL, "bad module table");
    if (cfg->prefetch_bucket_size < 0 || cfg->max_live_parameters < 0 || cfg->max_reuse_distance < 0)
        return fail(ZS3_EINVAL, "negative coordinator limit");
    std::unique_ptr<zs3_coord> c(new (std::nothrow) zs3_coord());
    if (!c) return fail(ZS3_ENOMEM, "coordinator allocation failed");
    c->cfg = *cfg;
    if (n_modules > 0 && module_start[0] != 0) return fail(ZS3_EINVAL, "module_start[0] != 0");
    for (int32_t m = 0; m < n_modules; ++m) {
        const int32_t a = module_start[m], b = module_start[m + 1];
        if (b < a) return fail(ZS3_EINVAL, "module_start is not ascending at %d", m);
        if (b > a && module_ds_ids == nullptr) return fail(ZS3_EINVAL, "module_ds_ids is NULL");
        std::vector<int32_t> ps;
        std::unordered_set<int64_t> seen;
        for (int32_t i = a; i < b; ++i) {
            const int64_t d = module_ds_ids[i];
            if (!seen.insert(d).second) return fail(ZS3_EDUPID, "ds_id %lld twice in module %d", (long long)d, m);
            auto it = c->index.find(d);
            int32_t p;
            if (it == c->index.end()) {
                int64_t n;
                bool pers;
                if (!zs3::layout_param(layout, d, &n, &pers))
                    return fail(ZS3_ENOTFOUND, "ds_id %lld of module %d is not in the layout", (long long)d, m);
                p = static_cast<int32_t>(c->ds_id.size());
                c->index.emplace(d, p);
                c->ds_id.push_back(d);
                c->numel.push_back(n);
                c->persistent.push_back(pers ? 1 : 0);
            } else {
                p = it->second;
            }
            if (!c->persistent[p]) ps.push_back(p);
        }
        std::sort(ps.begin(), ps.end(), [&](int32_t x, int32_t y) { return c->ds_id[x] < c->ds_id[y]; });
        int64_t size = 0;
        for (int32_t p : ps) size += c->numel[p];
        c->mod.push_back(std::move(ps));
        c->mod_size.push_back(size);
    }
    c->status.assign(c->ds_id.size(), ZS3_PARAM_NOT_AVAILABLE);
    for (size_t p = 0; p < c->ds_id.size(); ++p)
        if (c->persistent[p]) c->status[p] = ZS3_PARAM_AVAILABLE;
    c->marked.assign(c->ds_id.size(), -1);
    c->fetched_at.assign(c->mod.size(), -1);
    *out = c.release();
    return ok();
}

void zs3_coord_destroy(zs3_coord_t c) { delete c; }

zs3_status zs3_coord_fetch(zs3_coord_t c, int32_t module, int32_t* n_gathers, int32_t* kinds, int32_t* starts,
                           int64_t* ds_ids) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    if ((s = check_module(c, module)) != ZS3_OK) return s;
    if (n_gathers == nullptr || kinds == nullptr || starts == nullptr || ds_ids == nullptr)
        return fail(ZS3_EINVAL, "NULL output");
    const int32_t k = c->step_pos++;
    c->fetched_at[module] = k;
    // [codex] 5.1: record the module, or check it against the script
    if (c->mode == ZS3_TRACE_RECORD) {
        c->trace.push_back(module);
    } else if (c->mode == ZS3_TRACE_COMPLETE &&
               (k >= static_cast<int32_t>(c->trace.size()) || c->trace[k] != module)) {
        c->invalidate();
    }
    int32_t ng = 0, used = 0;
    starts[0] = 0;
    // [codex] 5.2 (i): gather what the module needs and is not live
    std::vector<int32_t> need;
    for (int32_t p : c->mod[module]) {
        if (c->status[p] == ZS3_PARAM_NOT_AVAILABLE) {
            need.push_back(p);
            c->status[p] = ZS3_PARAM_INFLIGHT;
            c->live += c->numel[p];
        }
    }
    if (!need.empty()) {
        used += put_ids(c, need, ds_ids + used);
        kinds[ng] = ZS3_GATHER_CURRENT;
        starts[++ng] = used;
    }
    // (ii): wait -- the module's parameters are available
    for (int32_t p : c->mod[module]) c->status[p] = ZS3_PARAM_AVAILABLE;
    // (iii): prefetch along the script
    if (c->mode == ZS3_TRACE_COMPLETE && c->cfg.prefetch_bucket_size > 0) {
        while (c->cursor < c->script.size() && c->script[c->cursor].first <= k) ++c->cursor;
        std::vector<int32_t> bucket;
        int64_t filled = 0;
        while (c->cursor < c->script.size()) {
            const int32_t pos = c->script[c->cursor].first, p = c->script[c->cursor].second;
            if (c->status[p] != ZS3_PARAM_NOT_AVAILABLE) {
                c->marked[p] = std::max(c->marked[p], pos);
                ++c->cursor;
                continue;
            }
            const int64_t n = c->numel[p];
            if (!bucket.empty() && filled + n > c->cfg.prefetch_bucket_size) break;
            if (c->live + n > c->cfg.max_live_parameters) break;
            bucket.push_back(p);
            filled += n;
            c->live += n;
            c->status[p] = ZS3_PARAM_INFLIGHT;
            c->marked[p] = std::max(c->marked[p], pos);
            ++c->cursor;
        }
        if (!bucket.empty()) {
            used += put_ids(c, bucket, ds_ids + used);
            kinds[ng] = ZS3_GATHER_PREFETCH;
            starts[++ng] = used;
        }
    }
    *n_gathers = ng;
    return ok();
}

zs3_status zs3_coord_release(zs3_coord_t c, int32_t module, int32_t* n_released, int64_t* ds_ids) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    if ((s = check_module(c, module)) != ZS3_OK) return s;
    if (n_released == nullptr || ds_ids == nullptr) return fail(ZS3_EINVAL, "NULL output");
    const int32_t k = c->fetched_at[module];
    if (k < 0) return fail(ZS3_EINVAL, "module %d was not fetched in this step", module);
    c->fetched_at[module] = -1;
    std::vector<int32_t> out;
    for (int32_t p : c->mod[module]) {
        if (c->status[p] != ZS3_PARAM_AVAILABLE) continue;
        if (c->marked[p] > k) continue;                                      // the prefetcher needs it
        if (c->mode == ZS3_TRACE_COMPLETE && c->reused_soon(p, k)) continue;  // reused within the window
        c->status[p] = ZS3_PARAM_NOT_AVAILABLE;
        c->live -= c->numel[p];
        out.push_back(p);
    }
    *n_released = put_ids(c, out, ds_ids);
    return ok();
}

zs3_status zs3_coord_release_all(zs3_coord_t c, int32_t* n_released, int64_t* ds_ids) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    if (n_released == nullptr || ds_ids == nullptr) return fail(ZS3_EINVAL, "NULL output");
    std::vector<int32_t> out;
    for (size_t p = 0; p < c->ds_id.size(); ++p) {
        if (c->persistent[p] || c->status[p] == ZS3_PARAM_NOT_AVAILABLE) continue;
        c->status[p] = ZS3_PARAM_NOT_AVAILABLE;
        c->live -= c->numel[p];
        out.push_back(static_cast<int32_t>(p));
    }
    std::fill(c->fetched_at.begin(), c->fetched_at.end(), -1);
    *n_released = put_ids(c, out, ds_ids);
    return ok();
}

zs3_status zs3_coord_reset_step(zs3_coord_t c, int32_t* mode) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    if (c->mode == ZS3_TRACE_COMPLETE && c->step_pos != static_cast<int32_t>(c->trace.size())) c->invalidate();
    if (c->mode == ZS3_TRACE_INVALID) {
        c->mode = ZS3_TRACE_RECORD;
        c->trace.clear();
        c->script.clear();
    } else if (c->mode == ZS3_TRACE_RECORD) {
        c->mode = ZS3_TRACE_COMPLETE;
        c->build_script();
    }
    c->step_pos = 0;
    c->cursor = 0;
    std::fill(c->marked.begin(), c->marked.end(), -1);
    std::fill(c->fetched_at.begin(), c->fetched_at.end(), -1);
    if (mode) *mode = c->mode;
    return ok();
}

zs3_status zs3_coord_info(zs3_coord_t c, int32_t* mode, int64_t* live_numel, int32_t* trace_len,
                          int32_t* invalidations) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    if (mode) *mode = c->mode;
    if (live_numel) *live_numel = c->live;
    if (trace_len) *trace_len = static_cast<int32_t>(c->trace.size());
    if (invalidations) *invalidations = c->invalidations;
    return ok();
}

zs3_status zs3_coord_param_status(zs3_coord_t c, int64_t ds_id, int32_t* status) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    if (status == nullptr) return fail(ZS3_EINVAL, "status is NULL");
    auto it = c->index.find(ds_id);
    if (it == c->index.end()) return fail(ZS3_ENOTFOUND, "ds_id %lld belongs to no module", (long long)ds_id);
    *status = c->status[it->second];
    return ok();
}

zs3_status zs3_coord_trace_signature(zs3_coord_t c, uint64_t* module_order, uint64_t* param_order,
                                     int32_t* n_fetches) {
    zs3_status s = check_coord(c);
    if (s != ZS3_OK) return s;
    std::vector<int64_t> mods(c->trace.begin(), c->trace.end()), params;
    params.reserve(c->script.size());
    for (const auto& e : c->script) params.push_back(c->ds_id[e.second]);
    if (module_order) *module_order = fnv1a64(mods);
    if (param_order) *param_order = fnv1a64(params);
    if (n_fetches) *n_fetches = static_cast<int32_t>(c->trace.size());
    return ok();
}

}  // extern "C"
