// C ABI of libzs3: argument validation, the host-side layout planner, the
// per-layout cache of device work lists, and the kernel launches.
//
// Pages cited: [codex] "03 · ZeRO-3: parameter sharding and the all-gather
// schedule" (ai-reference-codex), [csdn] "DeepSpeed ZeRO Stage 3: parameter
// partitioning ..." (adg.csdn.net), [llmnex] "ZeRO-3 core flow" (llmnex.top).

#include "zs3.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "zs3_internal.hpp"

using namespace zs3;

namespace {

thread_local std::string g_last_error;

zs3_status fail(zs3_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

zs3_status ok() {
    g_last_error.clear();
    return ZS3_OK;
}

// ------------------------------------------------------------- layout

struct Slot {
    int64_t ds_id;
    int64_t numel;
    int64_t ps;          // partition size
    int64_t offset;      // shard offset
    bool persistent;

    // [lo, hi) of the flattened parameter that `rank` holds real data for
    // ([codex] 3.1 element range; [codex] 5.3 persistent = whole).
    void own_range(int32_t rank, int64_t* lo, int64_t* hi) const {
        if (persistent) {
            *lo = 0;
            *hi = numel;
            return;
        }
        const int64_t a = static_cast<int64_t>(rank) * ps;
        const int64_t b = std::min(a + ps, numel);
        *lo = a;
        *hi = std::max(a, b);
    }
    int64_t real(int32_t rank) const {
        int64_t lo, hi;
        own_range(rank, &lo, &hi);
        return hi - lo;
    }
};

struct Key {
    std::vector<int64_t> w;
    bool operator==(const Key& o) const { return w == o.w; }
};

// One multiply-xorshift round per 64-bit word (a call's key can hold tens of
// thousands of words: every pointer of a single-launch reduce-scatter).
struct KeyHash {
    size_t operator()(const Key& k) const {
        uint64_t h = 0x9e3779b97f4a7c15ull ^ k.w.size();
        for (int64_t x : k.w) {
            h ^= static_cast<uint64_t>(x) + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
            h *= 0xff51afd7ed558ccdull;
            h ^= h >> 32;
        }
        return static_cast<size_t>(h);
    }
};

// A device work list: one allocation holding the tables of one call shape.
struct Plan {
    void* dev = nullptr;
    size_t bytes = 0;
    int64_t n_pieces = 0;
    int64_t n_part = 0;           // norm: spans [0, n_part) are partitioned
    int64_t n_blocks = 0;         // norm: workgroups of the sum-of-squares pass
    bool co_aligned = true;       // reduce-scatter: every source co-aligned with its dst
    size_t off_segs = 0, off_pieces = 0, off_srcs = 0, off_scratch = 0;

    std::shared_ptr<CopyInline> copy_inline;   // set: the plan travels in the kernel arguments
    std::shared_ptr<RsInline> rs_inline;
    std::shared_ptr<AdamInline> adam_inline;

    template <typename T>
    T* at(size_t off) const { return reinterpret_cast<T*>(static_cast<char*>(dev) + off); }
};

enum Op : int64_t {
    kOpPartition = 1, kOpPack, kOpUnpack, kOpReduce, kOpNorm, kOpAdam, kOpGather, kOpScatterPack,
    kOpScatterReduce, kOpNormSlots, kOpInitMaster, kOpGatherBuckets
};

constexpr size_t kMaxPlans = 1 << 14;

}  // namespace

struct zs3_layout;

namespace zs3 {
// Used by the coordinator (coord.cpp): the thread's last error, and a
// parameter's facts by ds_id.
zs3_status set_error(zs3_status s, const char* msg) {
    g_last_error = msg;
    return s;
}
bool layout_param(zs3_layout* L, int64_t ds_id, int64_t* numel, bool* persistent);
}  // namespace zs3

struct zs3_layout {
    int32_t world = 1;
    int64_t threshold = 0;
    std::vector<Slot> params;                       // ascending ds_id
    std::unordered_map<int64_t, int32_t> index;     // ds_id -> position
    int64_t shard_numel = 0;
    std::vector<int64_t> slot_base;                 // first norm slot of each parameter (layout order)
    int64_t n_slots = 0, n_part_slots = 0;
    std::unordered_map<Key, Plan, KeyHash> plans;
    std::unordered_map<int, std::vector<hipEvent_t>> events;   // per device: the offload pipeline's events

    ~zs3_layout() {
        release_plans();
        if (!events.empty()) {
            (void)hipDeviceSynchronize();
            for (auto& kv : events)
                for (hipEvent_t e : kv.second) (void)hipEventDestroy(e);
        }
    }

    void release_plans() {
        if (plans.empty()) return;
        (void)hipDeviceSynchronize();     // no cached table may be freed while a kernel reads it
        for (auto& kv : plans) {
            if (kv.second.dev != nullptr) (void)hipFree(kv.second.dev);
        }
        plans.clear();
    }
};

bool zs3::layout_param(zs3_layout* L, int64_t ds_id, int64_t* numel, bool* persistent) {
    auto it = L->index.find(ds_id);
    if (it == L->index.end()) return false;
    *numel = L->params[it->second].numel;
    *persistent = L->params[it->second].persistent;
    return true;
}

namespace {

int device_id() {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess) d = -1;
    return d;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + static_cast<uintptr_t>(bbytes) && y < x + static_cast<uintptr_t>(abytes);
}

zs3_status check_dtype(int32_t dtype) {
    if (dtype != ZS3_FP16 && dtype != ZS3_BF16) return fail(ZS3_EDTYPE, "dtype %d is not ZS3_FP16 or ZS3_BF16", dtype);
    return ZS3_OK;
}

zs3_status check_layout_rank(const zs3_layout* L, int32_t rank) {
    if (L == nullptr) return fail(ZS3_EINVAL, "layout is NULL");
    if (rank < 0 || rank >= L->world) return fail(ZS3_EINVAL, "rank %d outside [0, %d)", rank, L->world);
    return ZS3_OK;
}

zs3_status check_ptr16(const void* p, const char* what) {
    if (p == nullptr) return fail(ZS3_EINVAL, "%s is NULL", what);
    if (!aligned(p, 2)) return fail(ZS3_EINVAL, "%s is not 2-byte aligned", what);
    return ZS3_OK;
}

// Resolve a request's ds_ids to layout positions.  order[k] = position in
// the request of the k-th parameter in ascending ds_id.
zs3_status resolve(const zs3_layout* L, int32_t n, const int64_t* ds_ids, bool allow_persistent,
                   std::vector<int32_t>* pos, std::vector<int32_t>* order) {
    if (n < 0) return fail(ZS3_EINVAL, "n = %d < 0", n);
    if (n > 0 && ds_ids == nullptr) return fail(ZS3_EINVAL, "ds_ids is NULL");
    pos->resize(n);
    std::unordered_set<int64_t> seen;
    seen.reserve(static_cast<size_t>(n) * 2);
    for (int32_t i = 0; i < n; ++i) {
        auto it = L->index.find(ds_ids[i]);
        if (it == L->index.end()) return fail(ZS3_ENOTFOUND, "ds_id %lld is not in the layout", (long long)ds_ids[i]);
        if (!seen.insert(ds_ids[i]).second) return fail(ZS3_EDUPID, "ds_id %lld requested twice", (long long)ds_ids[i]);
        if (!allow_persistent && L->params[it->second].persistent)
            return fail(ZS3_EPERSIST, "ds_id %lld is persistent (never partitioned, never gathered)",
                        (long long)ds_ids[i]);
        (*pos)[i] = it->second;
    }
    order->resize(n);
    for (int32_t i = 0; i < n; ++i) (*order)[i] = i;
    std::sort(order->begin(), order->end(), [&](int32_t a, int32_t b) { return (*pos)[a] < (*pos)[b]; });
    return ZS3_OK;
}

// Split a contiguous segment into workgroup pieces whose starts (after the
// first) are 16-byte aligned in the destination.
void add_pieces(std::vector<Piece>* out, int32_t seg, uintptr_t dst_addr, int64_t count, int64_t P) {
    if (count <= 0) return;
    const int64_t head = static_cast<int64_t>(((16u - (dst_addr & 15u)) & 15u) >> 1);
    const int64_t first = std::min(count, head + P);
    out->push_back(Piece{0, seg, static_cast<int32_t>(first)});
    for (int64_t b = first; b < count; b += P) out->push_back(Piece{b, seg, static_cast<int32_t>(std::min(P, count - b))});
}

// Split [begin, begin+count) of a flat array into spans that, after the
// first, start at multiples of 8 elements when the array base is 16-byte
// aligned (`head` = elements until the first aligned position).
void add_spans(std::vector<Span>* out, int64_t begin, int64_t count, int64_t head, int64_t P) {
    if (count <= 0) return;
    const int64_t first = std::min(count, head + P);
    out->push_back(Span{begin, static_cast<int32_t>(first), 0});
    for (int64_t b = first; b < count; b += P)
        out->push_back(Span{begin + b, static_cast<int32_t>(std::min(P, count - b)), 0});
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Upload the host tables of a new plan in one allocation.
zs3_status upload(Plan* plan, const std::vector<std::pair<const void*, size_t>>& parts, size_t scratch_bytes,
                  std::vector<size_t>* offs) {
    size_t total = 0;
    offs->clear();
    for (const auto& p : parts) {
        offs->push_back(total);
        total = align_up(total + p.second, 256);
    }
    plan->off_scratch = total;
    total += scratch_bytes;
    if (total == 0) total = 256;
    void* dev = nullptr;
    if (hipMalloc(&dev, total) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ZS3_ENOMEM, "hipMalloc of a %zu-byte work list failed", total);
    }
    std::vector<char> host(total - scratch_bytes, 0);
    for (size_t i = 0; i < parts.size(); ++i)
        if (parts[i].second) std::memcpy(host.data() + (*offs)[i], parts[i].first, parts[i].second);
    if (!host.empty() && hipMemcpy(dev, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipFree(dev);
        return fail(ZS3_EHIP, "upload of a work list failed");
    }
    plan->dev = dev;
    plan->bytes = total;
    return ZS3_OK;
}

zs3_status store_plan(zs3_layout* L, Key&& key, Plan&& plan, Plan** out) {
    if (L->plans.size() >= kMaxPlans) L->release_plans();
    auto it = L->plans.emplace(std::move(key), std::move(plan)).first;
    *out = &it->second;
    return ZS3_OK;
}

// Workgroups of one launch: n_pieces * sub must fit a 32-bit grid of work-items.
zs3_status check_grid(int64_t n_pieces, int sub) {
    if (n_pieces * sub * kBlock >= (int64_t(1) << 32)) return fail(ZS3_EINVAL, "request too large for one launch");
    return ZS3_OK;
}

zs3_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ZS3_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- copy plans (partition, pack, unpack) --------------------------------

zs3_status build_copy_plan(zs3_layout* L, Key&& key, const std::vector<CopySeg>& segs_in, Plan** out) {
    // merge segments that continue each other in both source and destination
    std::vector<CopySeg> segs;
    for (const CopySeg& s : segs_in) {
        if (s.count <= 0) continue;
        if (!segs.empty() && segs.back().dst2 == nullptr && s.dst2 == nullptr) {
            CopySeg& b = segs.back();
            const bool dst_next = b.dst + b.count == s.dst;
            const bool src_next = (b.src == nullptr && s.src == nullptr) ||
                                  (b.src != nullptr && s.src != nullptr && b.src + b.count == s.src);
            if (dst_next && src_next) {
                b.count += s.count;
                continue;
            }
        }
        segs.push_back(s);
    }
    std::vector<Piece> pieces;
    for (size_t i = 0; i < segs.size(); ++i)
        add_pieces(&pieces, static_cast<int32_t>(i), reinterpret_cast<uintptr_t>(segs[i].dst), segs[i].count, kCopyPiece);
    zs3_status s = check_grid(static_cast<int64_t>(pieces.size()), kCopySub);
    if (s != ZS3_OK) return s;
    if (segs.size() <= static_cast<size_t>(kCopyInlineSegs)) {
        auto ci = std::make_shared<CopyInline>();
        std::memset(ci.get(), 0, sizeof(CopyInline));
        ci->nseg = static_cast<int32_t>(segs.size());
        std::vector<int32_t> per_seg(segs.size(), 0);
        for (const Piece& pc : pieces) ++per_seg[pc.seg];
        int32_t np = 0;
        for (size_t i = 0; i < segs.size(); ++i) {
            ci->piece_start[i] = np;
            np += per_seg[i];
            ci->head[i] = static_cast<int32_t>(((16u - (reinterpret_cast<uintptr_t>(segs[i].dst) & 15u)) & 15u) >> 1);
            ci->src[i] = segs[i].src;
            ci->dst[i] = segs[i].dst;
            ci->count[i] = segs[i].count;
            ci->dst2[i] = segs[i].dst2;
            ci->count2[i] = segs[i].count2;
        }
        ci->piece_start[segs.size()] = np;
        Plan plan;
        plan.n_pieces = np;
        plan.copy_inline = std::move(ci);
        return store_plan(L, std::move(key), std::move(plan), out);
    }
    Plan plan;
    plan.n_pieces = static_cast<int64_t>(pieces.size());
    std::vector<size_t> offs;
    s = upload(&plan, {{segs.data(), segs.size() * sizeof(CopySeg)}, {pieces.data(), pieces.size() * sizeof(Piece)}},
               0, &offs);
    if (s != ZS3_OK) return s;
    plan.off_segs = offs[0];
    plan.off_pieces = offs[1];
    return store_plan(L, std::move(key), std::move(plan), out);
}

zs3_status run_copy(CopyKind kind, const Plan* p, void* stream) {
    if (p->copy_inline)
        return hip_status(launch_copy_inline(kind, *p->copy_inline, static_cast<hipStream_t>(stream)),
                          "copy kernel launch");
    return hip_status(launch_copy(kind, p->at<CopySeg>(p->off_segs), p->at<Piece>(p->off_pieces), p->n_pieces,
                                  static_cast<hipStream_t>(stream)),
                      "copy kernel launch");
}

Plan* find_plan(zs3_layout* L, const Key& k) {
    auto it = L->plans.find(k);
    return it == L->plans.end() ? nullptr : &it->second;
}

// ---- reduce-scatter plans (both gradient paths) ----------------------------

zs3_status build_rs_plan(zs3_layout* L, Key&& key, const std::vector<RsSeg>& segs,
                         const std::vector<const uint16_t*>& srcs, int32_t N, Plan** out) {
    std::vector<Piece> pieces;
    bool co = true;
    for (size_t i = 0; i < segs.size(); ++i) {
        add_pieces(&pieces, static_cast<int32_t>(i), reinterpret_cast<uintptr_t>(segs[i].dst), segs[i].total, kRsPiece);
        for (int32_t v = 0; v < N; ++v) {
            const uint16_t* q = srcs[segs[i].src_index + v];
            if (q != nullptr && ((reinterpret_cast<uintptr_t>(q) ^ reinterpret_cast<uintptr_t>(segs[i].dst)) & 15u) != 0)
                co = false;
        }
    }
    zs3_status s = check_grid(static_cast<int64_t>(pieces.size()), rs_wide(N, co) ? kRsWideSub : kRsSub);
    if (s != ZS3_OK) return s;
    Plan np;
    np.n_pieces = static_cast<int64_t>(pieces.size());
    np.co_aligned = co;
    if (segs.size() <= static_cast<size_t>(kRsInlineSegs) &&
        segs.size() * static_cast<size_t>(N) <= static_cast<size_t>(kRsInlineSrcs)) {
        auto ri = std::make_shared<RsInline>();
        std::memset(ri.get(), 0, sizeof(RsInline));
        ri->nseg = static_cast<int32_t>(segs.size());
        ri->world = N;
        std::vector<int32_t> per_seg(segs.size(), 0);
        for (const Piece& pc : pieces) ++per_seg[pc.seg];
        int32_t npc = 0;
        for (size_t i = 0; i < segs.size(); ++i) {
            ri->piece_start[i] = npc;
            npc += per_seg[i];
            ri->head[i] = static_cast<int32_t>(((16u - (reinterpret_cast<uintptr_t>(segs[i].dst) & 15u)) & 15u) >> 1);
            ri->dst[i] = segs[i].dst;
            ri->real[i] = segs[i].real;
            ri->total[i] = segs[i].total;
            ri->slot[i] = segs[i].slot;
            for (int32_t v = 0; v < N; ++v) ri->src[i * N + v] = srcs[segs[i].src_index + v];
        }
        ri->piece_start[segs.size()] = npc;
        np.rs_inline = std::move(ri);
    } else {
        std::vector<size_t> offs;
        s = upload(&np,
                   {{segs.data(), segs.size() * sizeof(RsSeg)},
                    {pieces.data(), pieces.size() * sizeof(Piece)},
                    {srcs.data(), srcs.size() * sizeof(const uint16_t*)}},
                   0, &offs);
        if (s != ZS3_OK) return s;
        np.off_segs = offs[0];
        np.off_pieces = offs[1];
        np.off_srcs = offs[2];
    }
    return store_plan(L, std::move(key), std::move(np), out);
}

zs3_status run_rs(RsPath path, const Plan* plan, int32_t dtype, int32_t N, double* partials, void* stream) {
    if (plan->rs_inline)
        return hip_status(launch_reduce_scatter_inline(path, dtype, *plan->rs_inline, plan->co_aligned, partials,
                                                       static_cast<hipStream_t>(stream)),
                          "reduce-scatter kernel launch");
    return hip_status(launch_reduce_scatter(path, dtype, plan->at<RsSeg>(plan->off_segs),
                                            plan->at<Piece>(plan->off_pieces), plan->n_pieces,
                                            plan->at<const uint16_t*>(plan->off_srcs), N, plan->co_aligned, partials,
                                            static_cast<hipStream_t>(stream)),
                      "reduce-scatter kernel launch");
}

// The fused sums of squares need the layout's whole slot array, 8-byte
// aligned and apart from the gradient buffer.
zs3_status check_partials(const zs3_layout* L, const double* partials, const void* grad_flat) {
    if (partials == nullptr) return ZS3_OK;
    if (!aligned(partials, 8)) return fail(ZS3_EINVAL, "partials is not 8-byte aligned");
    if (overlap(partials, 8 * L->n_slots, grad_flat, 2 * L->shard_numel))
        return fail(ZS3_EALIAS, "partials overlaps grad_flat");
    return ZS3_OK;
}

}  // namespace

namespace {

AdamConsts adam_consts(const zs3_adam_params* hp) {
    AdamConsts c;
    const double t = static_cast<double>(hp->step);
    c.lr = static_cast<float>(hp->lr);
    c.b1 = static_cast<float>(hp->beta1);
    c.b2 = static_cast<float>(hp->beta2);
    c.omb1 = static_cast<float>(1.0 - hp->beta1);
    c.omb2 = static_cast<float>(1.0 - hp->beta2);
    c.bc1 = static_cast<float>(1.0 - std::pow(hp->beta1, t));
    c.bc2 = static_cast<float>(1.0 - std::pow(hp->beta2, t));
    c.eps = static_cast<float>(hp->eps);
    c.lrwd = static_cast<float>(hp->lr * hp->weight_decay);
    c.has_wd = hp->weight_decay != 0.0 ? 1 : 0;
    return c;
}

// The Adam launch over [begin, end) of the flat arrays (validated by the caller).
zs3_status adam_launch(zs3_layout* L, int32_t rank, int32_t dtype, int64_t begin, int64_t end, float* master,
                       float* exp_avg, float* exp_avg_sq, const void* grad_flat, void* shard_flat, const float* scale,
                       const int32_t* nonfinite, const AdamConsts& c, void* stream) {
    zs3_status s;
    const bool vec_ok = aligned(master, 16) && aligned(exp_avg, 16) && aligned(exp_avg_sq, 16) &&
                        aligned(grad_flat, 16) && aligned(shard_flat, 16);
    Key key{{kOpAdam, device_id(), rank, begin, end}};
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        // real runs of [begin, end): padding positions are skipped
        std::vector<std::pair<int64_t, int64_t>> runs;
        for (const Slot& p : L->params) {
            const int64_t a = std::max(begin, p.offset);
            const int64_t b = std::min(end, p.offset + p.real(rank));
            if (b <= a) continue;
            if (!runs.empty() && runs.back().first + runs.back().second == a) runs.back().second += b - a;
            else runs.emplace_back(a, b - a);
        }
        std::vector<Span> spans;
        for (auto& r : runs) add_spans(&spans, r.first, r.second, (8 - (r.first & 7)) & 7, kAdamPiece);
        if ((s = check_grid(static_cast<int64_t>(spans.size()), kAdamSub)) != ZS3_OK) return s;
        Plan np;
        np.n_pieces = static_cast<int64_t>(spans.size());
        if (runs.size() <= static_cast<size_t>(kAdamInlineRuns)) {
            auto ai = std::make_shared<AdamInline>();
            std::memset(ai.get(), 0, sizeof(AdamInline));
            ai->nrun = static_cast<int32_t>(runs.size());
            int32_t np_ = 0;
            size_t si = 0;
            for (size_t i = 0; i < runs.size(); ++i) {
                ai->piece_start[i] = np_;
                ai->begin[i] = runs[i].first;
                ai->count[i] = runs[i].second;
                // spans of run i are consecutive in `spans`
                while (si < spans.size() && spans[si].begin < runs[i].first + runs[i].second) {
                    ++np_;
                    ++si;
                }
            }
            ai->piece_start[runs.size()] = np_;
            np.adam_inline = std::move(ai);
        } else {
            std::vector<size_t> offs;
            s = upload(&np, {{spans.data(), spans.size() * sizeof(Span)}}, 0, &offs);
            if (s != ZS3_OK) return s;
            np.off_pieces = offs[0];
        }
        store_plan(L, std::move(key), std::move(np), &plan);
    }
    if (plan->adam_inline)
        return hip_status(launch_adam_inline(dtype, *plan->adam_inline, master, exp_avg, exp_avg_sq,
                                             static_cast<const uint16_t*>(grad_flat), static_cast<uint16_t*>(shard_flat),
                                             scale, nonfinite, c, vec_ok, static_cast<hipStream_t>(stream)),
                          "Adam kernel launch");
    return hip_status(launch_adam(dtype, plan->at<Span>(plan->off_pieces), plan->n_pieces, master, exp_avg, exp_avg_sq,
                                  static_cast<const uint16_t*>(grad_flat), static_cast<uint16_t*>(shard_flat), scale,
                                  nonfinite, c, vec_ok, static_cast<hipStream_t>(stream)),
                      "Adam kernel launch");
}

}  // namespace

namespace {

// Chunk offsets c_j (prefix sums of partition sizes) and full offsets f_j
// (prefix sums of numels) of a bucket, in ascending ds_id; returns the
// chunk and full sizes.
void bucket_offsets(const zs3_layout* L, const std::vector<int32_t>& pos, const std::vector<int32_t>& order,
                    std::vector<int64_t>* c, std::vector<int64_t>* f, int64_t* chunk, int64_t* full) {
    c->assign(pos.size(), 0);
    f->assign(pos.size(), 0);
    int64_t a = 0, b = 0;
    for (int32_t k : order) {
        (*c)[k] = a;
        (*f)[k] = b;
        a += L->params[pos[k]].ps;
        b += L->params[pos[k]].numel;
    }
    *chunk = a;
    *full = b;
}

// The segments of one bucket's fused gather (pack and unpack in one launch,
// the wire's own slot being the pack's output): the own shard's partitions
// into the own chunk and, when the two are co-aligned, from the same loads
// into the own part of each gathered view; then every other rank's chunk
// into its parts of the views ([codex] 5.2: ds_id order, views of one flat
// buffer; padding is never unpacked).
void fused_gather_segments(const zs3_layout* L, int32_t rank, const std::vector<int32_t>& pos,
                           const std::vector<int32_t>& order, const std::vector<int64_t>& c,
                           const std::vector<int64_t>& f, const void* shard_flat, void* own_chunk,
                           const void* const* rank_chunks, void* full_flat, std::vector<CopySeg>* segs) {
    const int32_t N = L->world;
    const uint16_t* shard = static_cast<const uint16_t*>(shard_flat);
    uint16_t* own = static_cast<uint16_t*>(own_chunk);
    uint16_t* dst = static_cast<uint16_t*>(full_flat);
    for (int32_t k : order) {
        const Slot& p = L->params[pos[k]];
        int64_t lo, hi;
        p.own_range(rank, &lo, &hi);
        uint16_t* own_dst = own + c[k];
        uint16_t* full_dst = dst + f[k] + lo;
        // read the own shard once for both destinations when they are co-aligned
        const bool both = hi > lo && ((reinterpret_cast<uintptr_t>(own_dst) ^ reinterpret_cast<uintptr_t>(full_dst)) & 15u) == 0;
        if (both) {
            segs->push_back(CopySeg{shard + p.offset, own_dst, p.ps, full_dst, hi - lo});
        } else {
            segs->push_back(CopySeg{shard + p.offset, own_dst, p.ps, nullptr, 0});
            segs->push_back(CopySeg{shard + p.offset, full_dst, hi - lo, nullptr, 0});
        }
    }
    for (int32_t k : order) {
        const Slot& p = L->params[pos[k]];
        for (int32_t v = 0; v < N; ++v) {
            if (v == rank) continue;
            int64_t lo, hi;
            p.own_range(v, &lo, &hi);
            segs->push_back(CopySeg{static_cast<const uint16_t*>(rank_chunks[v]) + c[k], dst + f[k] + lo, hi - lo,
                                    nullptr, 0});
        }
    }
}

// Byte ranges a call writes and reads: no written range may overlap another
// range (sort and sweep, O(k log k) for calls over many buffers).
struct Range {
    uintptr_t lo, hi;
    bool write;
    int32_t tag;
};

const Range* first_overlap(std::vector<Range>* rs, const Range** other) {
    std::sort(rs->begin(), rs->end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    const Range* max_any = nullptr;      // range with the largest end so far
    const Range* max_write = nullptr;    // written range with the largest end so far
    for (const Range& r : *rs) {
        if (r.hi <= r.lo) continue;
        if (r.write && max_any != nullptr && r.lo < max_any->hi) {
            *other = max_any;
            return &r;
        }
        if (!r.write && max_write != nullptr && r.lo < max_write->hi) {
            *other = max_write;
            return &r;
        }
        if (max_any == nullptr || r.hi > max_any->hi) max_any = &r;
        if (r.write && (max_write == nullptr || r.hi > max_write->hi)) max_write = &r;
    }
    return nullptr;
}

}  // namespace

// ======================================================================
// C ABI
// ======================================================================

extern "C" {

int32_t zs3_abi_version(void) { return ZS3_ABI_VERSION; }

const char* zs3_status_str(zs3_status s) {
    switch (s) {
        case ZS3_OK: return "ok";
        case ZS3_EINVAL: return "invalid argument";
        case ZS3_EDTYPE: return "unsupported dtype";
        case ZS3_EDUPID: return "duplicate ds_id";
        case ZS3_ENOTFOUND: return "ds_id not in layout";
        case ZS3_EPERSIST: return "persistent parameter in a request for partitioned ones";
        case ZS3_EALIAS: return "overlapping input and output";
        case ZS3_EHIP: return "HIP error";
        case ZS3_ENOMEM: return "out of memory";
        default: return "unknown status";
    }
}

const char* zs3_last_error(void) { return g_last_error.c_str(); }

zs3_status zs3_time_next_launch(void* start_event, void* stop_event) {
    set_launch_events(static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
    return ok();
}

zs3_status zs3_layout_create(int32_t world_size, int64_t persistence_threshold, int32_t n_params,
                             const int64_t* ds_id, const int64_t* numel, zs3_layout_t* out) {
    if (out == nullptr) return fail(ZS3_EINVAL, "out is NULL");
    *out = nullptr;
    if (world_size < 1) return fail(ZS3_EINVAL, "world_size %d < 1", world_size);
    if (persistence_threshold < 0) return fail(ZS3_EINVAL, "persistence_threshold < 0");
    if (n_params < 0) return fail(ZS3_EINVAL, "n_params < 0");
    if (n_params > 0 && (ds_id == nullptr || numel == nullptr)) return fail(ZS3_EINVAL, "ds_id or numel is NULL");
    std::unique_ptr<zs3_layout> L(new (std::nothrow) zs3_layout());
    if (!L) return fail(ZS3_ENOMEM, "layout allocation failed");
    L->world = world_size;
    L->threshold = persistence_threshold;
    std::vector<int32_t> order(n_params);
    for (int32_t i = 0; i < n_params; ++i) {
        if (ds_id[i] < 0) return fail(ZS3_EINVAL, "ds_id[%d] = %lld < 0", i, (long long)ds_id[i]);
        if (numel[i] < 1) return fail(ZS3_EINVAL, "numel[%d] = %lld < 1", i, (long long)numel[i]);
        order[i] = i;
    }
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return ds_id[a] < ds_id[b]; });
    int64_t offset = 0;
    L->params.reserve(n_params);
    for (int32_t k = 0; k < n_params; ++k) {
        const int32_t i = order[k];
        if (k > 0 && ds_id[order[k - 1]] == ds_id[i]) return fail(ZS3_EDUPID, "duplicate ds_id %lld", (long long)ds_id[i]);
        Slot s;
        s.ds_id = ds_id[i];
        s.numel = numel[i];
        s.persistent = numel[i] < persistence_threshold;
        s.ps = s.persistent ? s.numel : (s.numel + world_size - 1) / world_size;
        s.offset = offset;
        offset += s.ps;
        L->index.emplace(s.ds_id, k);
        L->params.push_back(s);
    }
    L->shard_numel = offset;
    // norm slots: partitioned parameters first, then persistent ones
    L->slot_base.assign(L->params.size(), 0);
    int64_t slot = 0;
    for (int pass = 0; pass < 2; ++pass) {
        for (size_t k = 0; k < L->params.size(); ++k) {
            const Slot& p = L->params[k];
            if (p.persistent != (pass == 1)) continue;
            L->slot_base[k] = slot;
            slot += kNormSlotsPerGroup * norm_slot_groups(p.ps);
        }
        if (pass == 0) L->n_part_slots = slot;
    }
    L->n_slots = slot;
    *out = L.release();
    return ok();
}

void zs3_layout_destroy(zs3_layout_t layout) { delete layout; }

zs3_status zs3_layout_info(zs3_layout_t L, int32_t* world_size, int64_t* threshold, int32_t* n_params,
                           int64_t* shard_numel, int64_t* bytes_per_rank) {
    if (L == nullptr) return fail(ZS3_EINVAL, "layout is NULL");
    if (world_size) *world_size = L->world;
    if (threshold) *threshold = L->threshold;
    if (n_params) *n_params = static_cast<int32_t>(L->params.size());
    if (shard_numel) *shard_numel = L->shard_numel;
    if (bytes_per_rank) *bytes_per_rank = 16 * L->shard_numel;
    return ok();
}

zs3_status zs3_layout_totals(zs3_layout_t L, int64_t* shard_numel, int64_t* bytes_per_rank) {
    return zs3_layout_info(L, nullptr, nullptr, nullptr, shard_numel, bytes_per_rank);
}

static void put_slot(const Slot& s, int64_t* numel, int64_t* ps, int32_t* persistent, int64_t* offset) {
    if (numel) *numel = s.numel;
    if (ps) *ps = s.ps;
    if (persistent) *persistent = s.persistent ? 1 : 0;
    if (offset) *offset = s.offset;
}

zs3_status zs3_layout_param_at(zs3_layout_t L, int32_t index, int64_t* ds_id, int64_t* numel, int64_t* ps,
                               int32_t* persistent, int64_t* offset) {
    if (L == nullptr) return fail(ZS3_EINVAL, "layout is NULL");
    if (index < 0 || index >= static_cast<int32_t>(L->params.size())) return fail(ZS3_EINVAL, "index %d out of range", index);
    const Slot& s = L->params[index];
    if (ds_id) *ds_id = s.ds_id;
    put_slot(s, numel, ps, persistent, offset);
    return ok();
}

zs3_status zs3_layout_param(zs3_layout_t L, int64_t ds_id, int64_t* numel, int64_t* ps, int32_t* persistent,
                            int64_t* offset) {
    if (L == nullptr) return fail(ZS3_EINVAL, "layout is NULL");
    auto it = L->index.find(ds_id);
    if (it == L->index.end()) return fail(ZS3_ENOTFOUND, "ds_id %lld is not in the layout", (long long)ds_id);
    put_slot(L->params[it->second], numel, ps, persistent, offset);
    return ok();
}

zs3_status zs3_layout_own_range(zs3_layout_t L, int64_t ds_id, int32_t rank, int64_t* lo, int64_t* hi) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    auto it = L->index.find(ds_id);
    if (it == L->index.end()) return fail(ZS3_ENOTFOUND, "ds_id %lld is not in the layout", (long long)ds_id);
    int64_t a, b;
    L->params[it->second].own_range(rank, &a, &b);
    if (lo) *lo = a;
    if (hi) *hi = b;
    return ok();
}

// Greedy bucketing: close the bucket before an item that would take it past
// `limit`, unless the bucket is empty.
zs3_status zs3_plan_buckets(zs3_layout_t L, int32_t kind, int64_t limit, int32_t cap, int32_t* n_buckets,
                            int32_t* starts, int64_t* ds_ids_out) {
    if (L == nullptr || n_buckets == nullptr) return fail(ZS3_EINVAL, "layout or n_buckets is NULL");
    if (kind != ZS3_GATHER_BUCKETS && kind != ZS3_REDUCE_BUCKETS) return fail(ZS3_EINVAL, "unknown bucket kind %d", kind);
    if (limit < 1) return fail(ZS3_EINVAL, "bucket limit < 1");
    std::vector<const Slot*> items;
    if (kind == ZS3_GATHER_BUCKETS) {
        for (const Slot& s : L->params)
            if (!s.persistent) items.push_back(&s);
    } else {
        for (auto it = L->params.rbegin(); it != L->params.rend(); ++it) items.push_back(&*it);
    }
    std::vector<int32_t> st;
    int64_t fill = 0;
    for (size_t i = 0; i < items.size(); ++i) {
        if (st.empty() || (fill > 0 && fill + items[i]->numel > limit)) {
            st.push_back(static_cast<int32_t>(i));
            fill = 0;
        }
        fill += items[i]->numel;
    }
    const int32_t nb = static_cast<int32_t>(st.size());
    *n_buckets = nb;
    if (cap < nb + 1 || starts == nullptr || (ds_ids_out == nullptr && !items.empty()))
        return fail(ZS3_EINVAL, "output capacity too small: %d buckets need %d starts", nb, nb + 1);
    for (int32_t b = 0; b < nb; ++b) starts[b] = st[b];
    starts[nb] = static_cast<int32_t>(items.size());
    for (size_t i = 0; i < items.size(); ++i) ds_ids_out[i] = items[i]->ds_id;
    return ok();
}

zs3_status zs3_sub_groups(zs3_layout_t L, int64_t sub_group_size, int32_t cap, int32_t* n_groups, int64_t* begin_end) {
    if (L == nullptr || n_groups == nullptr) return fail(ZS3_EINVAL, "layout or n_groups is NULL");
    if (sub_group_size < 1) return fail(ZS3_EINVAL, "sub_group_size < 1");
    std::vector<std::pair<int64_t, int64_t>> groups;
    int64_t fill = 0;
    for (const Slot& s : L->params) {
        if (groups.empty() || (fill > 0 && fill + s.ps > sub_group_size)) {
            groups.emplace_back(s.offset, s.offset);
            fill = 0;
        }
        groups.back().second = s.offset + s.ps;
        fill += s.ps;
    }
    const int32_t ng = static_cast<int32_t>(groups.size());
    *n_groups = ng;
    if (cap < ng || (begin_end == nullptr && ng > 0)) return fail(ZS3_EINVAL, "output capacity too small: %d groups", ng);
    for (int32_t g = 0; g < ng; ++g) {
        begin_end[2 * g] = groups[g].first;
        begin_end[2 * g + 1] = groups[g].second;
    }
    return ok();
}

zs3_status zs3_bucket_sizes(zs3_layout_t L, int32_t n, const int64_t* ds_ids, int64_t* chunk_numel, int64_t* full_numel) {
    if (L == nullptr) return fail(ZS3_EINVAL, "layout is NULL");
    std::vector<int32_t> pos, order;
    zs3_status s = resolve(L, n, ds_ids, false, &pos, &order);
    if (s != ZS3_OK) return s;
    int64_t c = 0, f = 0;
    for (int32_t i = 0; i < n; ++i) {
        c += L->params[pos[i]].ps;
        f += L->params[pos[i]].numel;
    }
    if (chunk_numel) *chunk_numel = c;
    if (full_numel) *full_numel = f;
    return ok();
}

// ---------------------------------------------------------------- (1)

zs3_status zs3_partition(zs3_layout_t L, int32_t rank, int32_t dtype, int32_t n, const int64_t* ds_ids,
                         const void* const* full_params, void* shard_flat, void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    std::vector<int32_t> pos, order;
    if ((s = resolve(L, n, ds_ids, true, &pos, &order)) != ZS3_OK) return s;
    if (n == 0) return ok();
    if (full_params == nullptr) return fail(ZS3_EINVAL, "full_params is NULL");
    if ((s = check_ptr16(shard_flat, "shard_flat")) != ZS3_OK) return s;
    const int64_t shard_bytes = 2 * L->shard_numel;
    for (int32_t i = 0; i < n; ++i) {
        if ((s = check_ptr16(full_params[i], "full_params[i]")) != ZS3_OK) return s;
        if (overlap(full_params[i], 2 * L->params[pos[i]].numel, shard_flat, shard_bytes))
            return fail(ZS3_EALIAS, "full_params[%d] overlaps shard_flat", i);
    }
    Key key{{kOpPartition, device_id(), rank, n, reinterpret_cast<int64_t>(shard_flat)}};
    for (int32_t k : order) {
        key.w.push_back(L->params[pos[k]].ds_id);
        key.w.push_back(reinterpret_cast<int64_t>(full_params[k]));
    }
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        std::vector<CopySeg> segs;
        uint16_t* base = static_cast<uint16_t*>(shard_flat);
        for (int32_t k : order) {
            const Slot& p = L->params[pos[k]];
            int64_t lo, hi;
            p.own_range(rank, &lo, &hi);
            const uint16_t* src = static_cast<const uint16_t*>(full_params[k]);
            segs.push_back(CopySeg{src + lo, base + p.offset, hi - lo, nullptr, 0});
            segs.push_back(CopySeg{nullptr, base + p.offset + (hi - lo), p.ps - (hi - lo), nullptr, 0});
        }
        if ((s = build_copy_plan(L, std::move(key), segs, &plan)) != ZS3_OK) return s;
    }
    return run_copy(kCopyPartition, plan, stream);
}

// ---------------------------------------------------------------- (2)

zs3_status zs3_gather_coalesced(zs3_layout_t L, int32_t rank, int32_t dtype, int32_t mode, int32_t n,
                                const int64_t* ds_ids, const void* shard_flat, void* own_chunk,
                                const void* const* rank_chunks, void* full_flat, int64_t* full_offsets,
                                void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if (mode < 1 || mode > (ZS3_PACK | ZS3_UNPACK)) return fail(ZS3_EINVAL, "mode %d is not PACK, UNPACK or both", mode);
    std::vector<int32_t> pos, order;
    if ((s = resolve(L, n, ds_ids, false, &pos, &order)) != ZS3_OK) return s;
    const int32_t N = L->world;
    // chunk offsets c_j and full offsets f_j in ascending ds_id
    std::vector<int64_t> c, f;
    int64_t chunk, full;
    bucket_offsets(L, pos, order, &c, &f, &chunk, &full);
    const bool do_pack = (mode & ZS3_PACK) != 0, do_unpack = (mode & ZS3_UNPACK) != 0;
    if (do_pack) {
        if ((s = check_ptr16(shard_flat, "shard_flat")) != ZS3_OK) return s;
        if ((s = check_ptr16(own_chunk, "own_chunk")) != ZS3_OK) return s;
        if (overlap(shard_flat, 2 * L->shard_numel, own_chunk, 2 * chunk))
            return fail(ZS3_EALIAS, "own_chunk overlaps shard_flat");
    }
    if (do_unpack) {
        if (rank_chunks == nullptr) return fail(ZS3_EINVAL, "rank_chunks is NULL");
        if ((s = check_ptr16(full_flat, "full_flat")) != ZS3_OK) return s;
        for (int32_t v = 0; v < N; ++v) {
            if ((s = check_ptr16(rank_chunks[v], "rank_chunks[v]")) != ZS3_OK) return s;
            if (overlap(rank_chunks[v], 2 * chunk, full_flat, 2 * full))
                return fail(ZS3_EALIAS, "rank_chunks[%d] overlaps full_flat", v);
        }
        if (do_pack && overlap(own_chunk, 2 * chunk, full_flat, 2 * full))
            return fail(ZS3_EALIAS, "own_chunk overlaps full_flat");
    }
    if (full_offsets != nullptr)
        for (int32_t i = 0; i < n; ++i) full_offsets[i] = f[i];
    if (n == 0) return ok();

    // Pack and unpack in one launch when the wire's own slot is the pack's
    // output: the own rank's part of the unpack then equals the shard's
    // partitions, so it is read from the shard and both run together.
    if (do_pack && do_unpack && rank_chunks[rank] == own_chunk) {
        Key key{{kOpGather, device_id(), rank, reinterpret_cast<int64_t>(shard_flat),
                 reinterpret_cast<int64_t>(own_chunk), reinterpret_cast<int64_t>(full_flat)}};
        for (int32_t v = 0; v < N; ++v) key.w.push_back(reinterpret_cast<int64_t>(rank_chunks[v]));
        for (int32_t k : order) key.w.push_back(L->params[pos[k]].ds_id);
        Plan* plan = find_plan(L, key);
        if (plan == nullptr) {
            std::vector<CopySeg> segs;
            fused_gather_segments(L, rank, pos, order, c, f, shard_flat, own_chunk, rank_chunks, full_flat, &segs);
            if ((s = build_copy_plan(L, std::move(key), segs, &plan)) != ZS3_OK) return s;
        }
        return run_copy(kCopyGather, plan, stream);
    }

    if (do_pack) {
        Key key{{kOpPack, device_id(), rank, reinterpret_cast<int64_t>(shard_flat), reinterpret_cast<int64_t>(own_chunk)}};
        for (int32_t k : order) key.w.push_back(L->params[pos[k]].ds_id);
        Plan* plan = find_plan(L, key);
        if (plan == nullptr) {
            std::vector<CopySeg> segs;
            const uint16_t* src = static_cast<const uint16_t*>(shard_flat);
            uint16_t* dst = static_cast<uint16_t*>(own_chunk);
            for (int32_t k : order) {
                const Slot& p = L->params[pos[k]];
                segs.push_back(CopySeg{src + p.offset, dst + c[k], p.ps, nullptr, 0});
            }
            if ((s = build_copy_plan(L, std::move(key), segs, &plan)) != ZS3_OK) return s;
        }
        if ((s = run_copy(kCopyPack, plan, stream)) != ZS3_OK) return s;
    }
    if (do_unpack) {
        Key key{{kOpUnpack, device_id(), reinterpret_cast<int64_t>(full_flat)}};
        for (int32_t v = 0; v < N; ++v) key.w.push_back(reinterpret_cast<int64_t>(rank_chunks[v]));
        for (int32_t k : order) key.w.push_back(L->params[pos[k]].ds_id);
        Plan* plan = find_plan(L, key);
        if (plan == nullptr) {
            std::vector<CopySeg> segs;
            uint16_t* dst = static_cast<uint16_t*>(full_flat);
            for (int32_t k : order) {
                const Slot& p = L->params[pos[k]];
                for (int32_t v = 0; v < N; ++v) {
                    int64_t lo, hi;
                    p.own_range(v, &lo, &hi);
                    const uint16_t* src = static_cast<const uint16_t*>(rank_chunks[v]) + c[k];
                    segs.push_back(CopySeg{src, dst + f[k] + lo, hi - lo, nullptr, 0});
                }
            }
            if ((s = build_copy_plan(L, std::move(key), segs, &plan)) != ZS3_OK) return s;
        }
        if ((s = run_copy(kCopyUnpack, plan, stream)) != ZS3_OK) return s;
    }
    return ok();
}

zs3_status zs3_gather_coalesced_buckets(zs3_layout_t L, int32_t rank, int32_t dtype, int32_t n_buckets,
                                        const int32_t* bucket_start, const int64_t* ds_ids, const void* shard_flat,
                                        void* const* own_chunks, const void* const* rank_chunks,
                                        void* const* full_flats, void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if (n_buckets < 0) return fail(ZS3_EINVAL, "n_buckets = %d < 0", n_buckets);
    if (n_buckets == 0) return ok();
    if (bucket_start == nullptr || own_chunks == nullptr || rank_chunks == nullptr || full_flats == nullptr)
        return fail(ZS3_EINVAL, "bucket_start, own_chunks, rank_chunks or full_flats is NULL");
    if (bucket_start[0] != 0) return fail(ZS3_EINVAL, "bucket_start[0] = %d, not 0", bucket_start[0]);
    if ((s = check_ptr16(shard_flat, "shard_flat")) != ZS3_OK) return s;
    const int32_t N = L->world;
    std::vector<Range> ranges;
    ranges.push_back(Range{reinterpret_cast<uintptr_t>(shard_flat),
                           reinterpret_cast<uintptr_t>(shard_flat) + 2 * static_cast<uintptr_t>(L->shard_numel), false, -1});
    struct B {
        std::vector<int32_t> pos, order;
        std::vector<int64_t> c, f;
    };
    std::vector<B> bk(n_buckets);
    std::unordered_set<int64_t> seen;
    for (int32_t b = 0; b < n_buckets; ++b) {
        const int32_t a = bucket_start[b], e = bucket_start[b + 1];
        if (e <= a) return fail(ZS3_EINVAL, "bucket %d is empty or bucket_start is not increasing", b);
        if ((s = resolve(L, e - a, ds_ids + a, false, &bk[b].pos, &bk[b].order)) != ZS3_OK) return s;
        for (int32_t i = a; i < e; ++i)
            if (!seen.insert(ds_ids[i]).second) return fail(ZS3_EDUPID, "ds_id %lld in two buckets", (long long)ds_ids[i]);
        int64_t chunk, full;
        bucket_offsets(L, bk[b].pos, bk[b].order, &bk[b].c, &bk[b].f, &chunk, &full);
        if ((s = check_ptr16(own_chunks[b], "own_chunks[b]")) != ZS3_OK) return s;
        if ((s = check_ptr16(full_flats[b], "full_flats[b]")) != ZS3_OK) return s;
        if (rank_chunks[static_cast<int64_t>(b) * N + rank] != own_chunks[b])
            return fail(ZS3_EINVAL, "rank_chunks[%d*N + rank] is not own_chunks[%d]", b, b);
        const uintptr_t oc = reinterpret_cast<uintptr_t>(own_chunks[b]), ff = reinterpret_cast<uintptr_t>(full_flats[b]);
        ranges.push_back(Range{oc, oc + 2 * static_cast<uintptr_t>(chunk), true, b});
        ranges.push_back(Range{ff, ff + 2 * static_cast<uintptr_t>(full), true, b});
        for (int32_t v = 0; v < N; ++v) {
            if (v == rank) continue;
            const void* q = rank_chunks[static_cast<int64_t>(b) * N + v];
            if ((s = check_ptr16(q, "rank_chunks[b*N+v]")) != ZS3_OK) return s;
            const uintptr_t x = reinterpret_cast<uintptr_t>(q);
            ranges.push_back(Range{x, x + 2 * static_cast<uintptr_t>(chunk), false, b});
        }
    }
    const Range* other = nullptr;
    if (const Range* bad = first_overlap(&ranges, &other))
        return fail(ZS3_EALIAS, "an output of bucket %d overlaps a buffer of bucket %d", bad->write ? bad->tag : other->tag,
                    bad->write ? other->tag : bad->tag);

    Key key{{kOpGatherBuckets, device_id(), rank, reinterpret_cast<int64_t>(shard_flat), n_buckets}};
    for (int32_t b = 0; b < n_buckets; ++b) {
        key.w.push_back(bucket_start[b + 1]);
        key.w.push_back(reinterpret_cast<int64_t>(full_flats[b]));
        for (int32_t v = 0; v < N; ++v) key.w.push_back(reinterpret_cast<int64_t>(rank_chunks[static_cast<int64_t>(b) * N + v]));
        for (int32_t k : bk[b].order) key.w.push_back(L->params[bk[b].pos[k]].ds_id);
    }
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        std::vector<CopySeg> segs;
        for (int32_t b = 0; b < n_buckets; ++b)
            fused_gather_segments(L, rank, bk[b].pos, bk[b].order, bk[b].c, bk[b].f, shard_flat, own_chunks[b],
                                  rank_chunks + static_cast<int64_t>(b) * N, full_flats[b], &segs);
        if ((s = build_copy_plan(L, std::move(key), segs, &plan)) != ZS3_OK) return s;
    }
    return run_copy(kCopyGather, plan, stream);
}

// ---------------------------------------------------------------- (3)

zs3_status zs3_reduce_scatter_local(zs3_layout_t L, int32_t rank, int32_t dtype, int32_t n, const int64_t* ds_ids,
                                    const void* const* src, void* grad_flat, double* partials, void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    std::vector<int32_t> pos, order;
    if ((s = resolve(L, n, ds_ids, true, &pos, &order)) != ZS3_OK) return s;
    if (n == 0) return ok();
    if (src == nullptr) return fail(ZS3_EINVAL, "src is NULL");
    if ((s = check_ptr16(grad_flat, "grad_flat")) != ZS3_OK) return s;
    if ((s = check_partials(L, partials, grad_flat)) != ZS3_OK) return s;
    const int32_t N = L->world;
    uint16_t* gbase = static_cast<uint16_t*>(grad_flat);
    // no source may overlap a written range (the parameters' partitions of
    // grad_flat, and partials): one sort-and-sweep over every range
    std::vector<Range> ranges;
    ranges.reserve(static_cast<size_t>(n) * (N + 1) + 1);
    for (int32_t i = 0; i < n; ++i) {
        const Slot& p = L->params[pos[i]];
        const uintptr_t w = reinterpret_cast<uintptr_t>(gbase + p.offset);
        ranges.push_back(Range{w, w + 2 * static_cast<uintptr_t>(p.ps), true, -1});
        const int64_t real = p.real(rank);
        if (real == 0) continue;
        for (int32_t v = 0; v < N; ++v) {
            const void* q = src[static_cast<int64_t>(i) * N + v];
            if ((s = check_ptr16(q, "src[i*N+v]")) != ZS3_OK) return s;
            const uintptr_t x = reinterpret_cast<uintptr_t>(q);
            ranges.push_back(Range{x, x + 2 * static_cast<uintptr_t>(real), false, i * N + v});
        }
    }
    if (partials != nullptr) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(partials);
        ranges.push_back(Range{x, x + 8 * static_cast<uintptr_t>(L->n_slots), true, -2});
    }
    const Range* other = nullptr;
    if (const Range* bad = first_overlap(&ranges, &other)) {
        const Range* rd = bad->write ? other : bad;
        const Range* wr = bad->write ? bad : other;
        if (rd->write)
            return fail(ZS3_EALIAS, "partials overlaps grad_flat");
        return fail(ZS3_EALIAS, "src[%d*N+%d] overlaps %s", rd->tag / N, rd->tag % N,
                    wr->tag == -2 ? "partials" : "the written part of grad_flat");
    }
    Key key{{kOpReduce, device_id(), rank, reinterpret_cast<int64_t>(grad_flat)}};
    for (int32_t k : order) {
        key.w.push_back(L->params[pos[k]].ds_id);
        for (int32_t v = 0; v < N; ++v) key.w.push_back(reinterpret_cast<int64_t>(src[static_cast<int64_t>(k) * N + v]));
    }
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        std::vector<RsSeg> segs;
        std::vector<const uint16_t*> srcs;
        for (int32_t k : order) {
            const Slot& p = L->params[pos[k]];
            const int64_t real = p.real(rank);
            segs.push_back(RsSeg{gbase + p.offset, real, p.ps, static_cast<int64_t>(srcs.size()), L->slot_base[pos[k]]});
            for (int32_t v = 0; v < N; ++v)
                srcs.push_back(real == 0 ? nullptr : static_cast<const uint16_t*>(src[static_cast<int64_t>(k) * N + v]));
        }
        if ((s = build_rs_plan(L, std::move(key), segs, srcs, N, &plan)) != ZS3_OK) return s;
    }
    return run_rs(kRsContiguous, plan, dtype, N, partials, stream);
}

zs3_status zs3_reduce_scatter_coalesced(zs3_layout_t L, int32_t rank, int32_t dtype, int32_t mode, int32_t n,
                                        const int64_t* ds_ids, const void* const* grads, void* send,
                                        const void* const* recv_chunks, void* grad_flat, double* partials,
                                        void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if (mode != ZS3_PACK && mode != ZS3_REDUCE && mode != (ZS3_PACK | ZS3_REDUCE))
        return fail(ZS3_EINVAL, "mode %d is not PACK, REDUCE or both", mode);
    std::vector<int32_t> pos, order;
    if ((s = resolve(L, n, ds_ids, false, &pos, &order)) != ZS3_OK) return s;
    const int32_t N = L->world;
    std::vector<int64_t> c(n);
    int64_t chunk = 0;
    for (int32_t k : order) {
        c[k] = chunk;
        chunk += L->params[pos[k]].ps;
    }
    const bool do_pack = (mode & ZS3_PACK) != 0, do_reduce = (mode & ZS3_REDUCE) != 0;
    uint16_t* gbase = static_cast<uint16_t*>(grad_flat);
    if (do_pack) {
        if (n > 0 && grads == nullptr) return fail(ZS3_EINVAL, "grads is NULL");
        if ((s = check_ptr16(send, "send")) != ZS3_OK) return s;
        for (int32_t i = 0; i < n; ++i) {
            if ((s = check_ptr16(grads[i], "grads[i]")) != ZS3_OK) return s;
            if (overlap(grads[i], 2 * L->params[pos[i]].numel, send, 2 * N * chunk))
                return fail(ZS3_EALIAS, "grads[%d] overlaps send", i);
        }
    }
    if (do_reduce) {
        if (recv_chunks == nullptr) return fail(ZS3_EINVAL, "recv_chunks is NULL");
        if ((s = check_ptr16(grad_flat, "grad_flat")) != ZS3_OK) return s;
        if ((s = check_partials(L, partials, grad_flat)) != ZS3_OK) return s;
        for (int32_t v = 0; v < N; ++v) {
            if ((s = check_ptr16(recv_chunks[v], "recv_chunks[v]")) != ZS3_OK) return s;
            for (int32_t j = 0; j < n; ++j) {
                const Slot& o = L->params[pos[j]];
                if (overlap(recv_chunks[v], 2 * chunk, gbase + o.offset, 2 * o.ps))
                    return fail(ZS3_EALIAS, "recv_chunks[%d] overlaps the written part of grad_flat", v);
            }
            if (partials != nullptr && overlap(recv_chunks[v], 2 * chunk, partials, 8 * L->n_slots))
                return fail(ZS3_EALIAS, "recv_chunks[%d] overlaps partials", v);
        }
        if (do_pack)
            for (int32_t j = 0; j < n; ++j) {
                const Slot& o = L->params[pos[j]];
                if (overlap(send, 2 * N * chunk, gbase + o.offset, 2 * o.ps))
                    return fail(ZS3_EALIAS, "send overlaps the written part of grad_flat");
            }
    }
    if (n == 0) return ok();

    if (do_pack) {
        Key key{{kOpScatterPack, device_id(), reinterpret_cast<int64_t>(send)}};
        for (int32_t k : order) {
            key.w.push_back(L->params[pos[k]].ds_id);
            key.w.push_back(reinterpret_cast<int64_t>(grads[k]));
        }
        Plan* plan = find_plan(L, key);
        if (plan == nullptr) {
            // chunk d = partition d of every parameter in ascending ds_id, zeros past numel
            std::vector<CopySeg> segs;
            uint16_t* out = static_cast<uint16_t*>(send);
            for (int32_t d = 0; d < N; ++d) {
                for (int32_t k : order) {
                    const Slot& p = L->params[pos[k]];
                    int64_t lo, hi;
                    p.own_range(d, &lo, &hi);
                    uint16_t* dst = out + static_cast<int64_t>(d) * chunk + c[k];
                    segs.push_back(CopySeg{static_cast<const uint16_t*>(grads[k]) + lo, dst, hi - lo, nullptr, 0});
                    segs.push_back(CopySeg{nullptr, dst + (hi - lo), p.ps - (hi - lo), nullptr, 0});
                }
            }
            if ((s = build_copy_plan(L, std::move(key), segs, &plan)) != ZS3_OK) return s;
        }
        if ((s = run_copy(kCopyScatterPack, plan, stream)) != ZS3_OK) return s;
    }
    if (do_reduce) {
        Key key{{kOpScatterReduce, device_id(), rank, reinterpret_cast<int64_t>(grad_flat)}};
        for (int32_t v = 0; v < N; ++v) key.w.push_back(reinterpret_cast<int64_t>(recv_chunks[v]));
        for (int32_t k : order) key.w.push_back(L->params[pos[k]].ds_id);
        Plan* plan = find_plan(L, key);
        if (plan == nullptr) {
            std::vector<RsSeg> segs;
            std::vector<const uint16_t*> srcs;
            for (int32_t k : order) {
                const Slot& p = L->params[pos[k]];
                const int64_t real = p.real(rank);
                segs.push_back(RsSeg{gbase + p.offset, real, p.ps, static_cast<int64_t>(srcs.size()), L->slot_base[pos[k]]});
                for (int32_t v = 0; v < N; ++v)
                    srcs.push_back(real == 0 ? nullptr : static_cast<const uint16_t*>(recv_chunks[v]) + c[k]);
            }
            if ((s = build_rs_plan(L, std::move(key), segs, srcs, N, &plan)) != ZS3_OK) return s;
        }
        if ((s = run_rs(kRsCoalesced, plan, dtype, N, partials, stream)) != ZS3_OK) return s;
    }
    return ok();
}

// ---------------------------------------------------------------- (4)

zs3_status zs3_grad_norm(zs3_layout_t L, int32_t rank, int32_t dtype, const void* grad_flat, double* sumsq,
                         int32_t finalize, double max_norm, double loss_scale, double* norm_out, float* scale_out,
                         int32_t* nonfinite, void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if ((s = check_ptr16(grad_flat, "grad_flat")) != ZS3_OK) return s;
    if (sumsq == nullptr || !aligned(sumsq, 8)) return fail(ZS3_EINVAL, "sumsq is NULL or not 8-byte aligned");
    if (finalize) {
        if (norm_out == nullptr || scale_out == nullptr || nonfinite == nullptr)
            return fail(ZS3_EINVAL, "finalize needs norm_out, scale_out and nonfinite");
        if (!aligned(norm_out, 8) || !aligned(scale_out, 4) || !aligned(nonfinite, 4))
            return fail(ZS3_EINVAL, "misaligned norm_out, scale_out or nonfinite");
        if (!(max_norm > 0.0) || !(loss_scale > 0.0)) return fail(ZS3_EINVAL, "max_norm and loss_scale must be > 0");
    }
    if (overlap(sumsq, 8 * (L->world + 1), grad_flat, 2 * L->shard_numel))
        return fail(ZS3_EALIAS, "sumsq overlaps grad_flat");
    // the scratch of the sum-of-squares pass belongs to the plan, and the
    // plan is keyed by the stream too: norm calls on different streams never
    // share scratch, and calls on one stream are ordered by it
    Key key{{kOpNorm, device_id(), rank, reinterpret_cast<int64_t>(grad_flat), reinterpret_cast<int64_t>(stream)}};
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        // real runs: partitioned first, then persistent; adjacent runs merged
        std::vector<std::pair<int64_t, int64_t>> part, pers;
        for (const Slot& p : L->params) {
            auto& runs = p.persistent ? pers : part;
            const int64_t real = p.real(rank);
            if (real == 0) continue;
            if (!runs.empty() && runs.back().first + runs.back().second == p.offset) runs.back().second += real;
            else runs.emplace_back(p.offset, real);
        }
        const uintptr_t base = reinterpret_cast<uintptr_t>(grad_flat);
        std::vector<Span> spans;
        for (auto& r : part) add_spans(&spans, r.first, r.second, ((16u - ((base + 2 * r.first) & 15u)) & 15u) >> 1, kNormPiece);
        const int64_t n_part = static_cast<int64_t>(spans.size());
        for (auto& r : pers) add_spans(&spans, r.first, r.second, ((16u - ((base + 2 * r.first) & 15u)) & 15u) >> 1, kNormPiece);
        Plan np;
        np.n_pieces = static_cast<int64_t>(spans.size());
        np.n_part = n_part;
        np.n_blocks = std::min<int64_t>(np.n_pieces * kNormSub, kNormGrid);
        std::vector<size_t> offs;
        s = upload(&np, {{spans.data(), spans.size() * sizeof(Span)}},
                   std::max<size_t>(16, 2 * static_cast<size_t>(np.n_blocks) * sizeof(double)), &offs);
        if (s != ZS3_OK) return s;
        np.off_pieces = offs[0];
        store_plan(L, std::move(key), std::move(np), &plan);
    }
    return hip_status(launch_grad_norm(dtype, static_cast<const uint16_t*>(grad_flat), plan->at<Span>(plan->off_pieces),
                                       plan->n_pieces, plan->n_part, plan->n_blocks, plan->at<double>(plan->off_scratch),
                                       sumsq, rank,
                                       L->world, finalize, max_norm, loss_scale, norm_out, scale_out, nonfinite,
                                       static_cast<hipStream_t>(stream)),
                      "grad-norm kernel launch");
}

zs3_status zs3_layout_norm_slots(zs3_layout_t L, int64_t* n_slots, int64_t* n_part_slots) {
    if (L == nullptr) return fail(ZS3_EINVAL, "layout is NULL");
    if (n_slots) *n_slots = L->n_slots;
    if (n_part_slots) *n_part_slots = L->n_part_slots;
    return ok();
}

}  // extern "C"

namespace {

// Arguments of the two slot-norm entry points.
zs3_status check_norm_partials(const zs3_layout* L, int32_t rank, const double* partials, const double* sumsq,
                               int32_t finalize, double max_norm, double loss_scale, const double* norm_out,
                               const float* scale_out, const int32_t* nonfinite) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if (partials == nullptr || !aligned(partials, 8)) return fail(ZS3_EINVAL, "partials is NULL or not 8-byte aligned");
    if (sumsq == nullptr || !aligned(sumsq, 8)) return fail(ZS3_EINVAL, "sumsq is NULL or not 8-byte aligned");
    if (finalize) {
        if (norm_out == nullptr || scale_out == nullptr || nonfinite == nullptr)
            return fail(ZS3_EINVAL, "finalize needs norm_out, scale_out and nonfinite");
        if (!aligned(norm_out, 8) || !aligned(scale_out, 4) || !aligned(nonfinite, 4))
            return fail(ZS3_EINVAL, "misaligned norm_out, scale_out or nonfinite");
        if (!(max_norm > 0.0) || !(loss_scale > 0.0)) return fail(ZS3_EINVAL, "max_norm and loss_scale must be > 0");
    }
    if (overlap(sumsq, 8 * (L->world + 1), partials, 8 * L->n_slots)) return fail(ZS3_EALIAS, "sumsq overlaps partials");
    return ZS3_OK;
}

// The allocation-free slot norm sums at most this many slots per call
// (its scratch holds kNormSlotBlocks workgroup sums; beyond this bound each
// workgroup would walk more than 65536 slots).
constexpr int64_t kNoAllocMaxSlots = kNormSlotBlocks * 65536;

}  // namespace

extern "C" {

zs3_status zs3_grad_norm_partials(zs3_layout_t L, int32_t rank, const double* partials, double* sumsq,
                                  int32_t finalize, double max_norm, double loss_scale, double* norm_out,
                                  float* scale_out, int32_t* nonfinite, void* stream) {
    zs3_status s = check_norm_partials(L, rank, partials, sumsq, finalize, max_norm, loss_scale, norm_out, scale_out,
                                       nonfinite);
    if (s != ZS3_OK) return s;
    Key key{{kOpNormSlots, device_id(), reinterpret_cast<int64_t>(stream)}};     // scratch per stream, as above
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        Plan np;
        norm_slot_split(L->n_slots, &np.n_blocks, &np.n_pieces);    // n_pieces: slots per workgroup
        std::vector<size_t> offs;
        s = upload(&np, {}, 2 * static_cast<size_t>(np.n_blocks) * sizeof(double), &offs);
        if (s != ZS3_OK) return s;
        store_plan(L, std::move(key), std::move(np), &plan);
    }
    return hip_status(launch_norm_from_slots(partials, L->n_slots, L->n_part_slots, plan->n_blocks, plan->n_pieces,
                                             plan->at<double>(plan->off_scratch), sumsq, rank, L->world, finalize,
                                             max_norm, loss_scale, norm_out, scale_out, nonfinite,
                                             static_cast<hipStream_t>(stream)),
                      "grad-norm kernel launch");
}

zs3_status zs3_grad_norm_partials_noalloc(zs3_layout_t L, int32_t rank, const double* partials, double* sumsq,
                                          int32_t finalize, double max_norm, double loss_scale, double* norm_out,
                                          float* scale_out, int32_t* nonfinite, void* stream) {
    zs3_status s = check_norm_partials(L, rank, partials, sumsq, finalize, max_norm, loss_scale, norm_out, scale_out,
                                       nonfinite);
    if (s != ZS3_OK) return s;
    if (L->n_slots > kNoAllocMaxSlots)
        return fail(ZS3_EINVAL, "layout has %lld norm slots; the allocation-free norm sums at most %lld",
                    (long long)L->n_slots, (long long)kNoAllocMaxSlots);
    return hip_status(launch_norm_from_slots_static(partials, L->n_slots, L->n_part_slots, sumsq, rank, L->world,
                                                    finalize, max_norm, loss_scale, norm_out, scale_out, nonfinite,
                                                    static_cast<hipStream_t>(stream)),
                      "grad-norm kernel launch");
}

// ---------------------------------------------------------------- (5)

zs3_status zs3_adam_step(zs3_layout_t L, int32_t rank, int32_t dtype, int64_t begin, int64_t end, float* master,
                         float* exp_avg, float* exp_avg_sq, const void* grad_flat, void* shard_flat,
                         const float* scale, const int32_t* nonfinite, const zs3_adam_params* hp, void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if (hp == nullptr) return fail(ZS3_EINVAL, "hp is NULL");
    if (hp->step < 1) return fail(ZS3_EINVAL, "step %lld < 1", (long long)hp->step);
    if (begin < 0 || end < begin || end > L->shard_numel)
        return fail(ZS3_EINVAL, "range [%lld, %lld) outside [0, %lld]", (long long)begin, (long long)end,
                    (long long)L->shard_numel);
    if (master == nullptr || exp_avg == nullptr || exp_avg_sq == nullptr || scale == nullptr)
        return fail(ZS3_EINVAL, "master, exp_avg, exp_avg_sq or scale is NULL");
    if (!aligned(master, 4) || !aligned(exp_avg, 4) || !aligned(exp_avg_sq, 4) || !aligned(scale, 4) ||
        (nonfinite != nullptr && !aligned(nonfinite, 4)))
        return fail(ZS3_EINVAL, "fp32 or int32 pointer not 4-byte aligned");
    if ((s = check_ptr16(grad_flat, "grad_flat")) != ZS3_OK) return s;
    if ((s = check_ptr16(shard_flat, "shard_flat")) != ZS3_OK) return s;
    const int64_t nb = end - begin;
    const void* arr[5] = {master + begin, exp_avg + begin, exp_avg_sq + begin,
                          static_cast<const uint16_t*>(grad_flat) + begin, static_cast<uint16_t*>(shard_flat) + begin};
    const int64_t bytes[5] = {4 * nb, 4 * nb, 4 * nb, 2 * nb, 2 * nb};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(arr[i], bytes[i], arr[j], bytes[j])) return fail(ZS3_EALIAS, "Adam arrays %d and %d overlap", i, j);
    if (nb == 0) return ok();

    return adam_launch(L, rank, dtype, begin, end, master, exp_avg, exp_avg_sq, grad_flat, shard_flat, scale,
                       nonfinite, adam_consts(hp), stream);
}

// ---------------------------------------------- (5a) fp32 master partition

zs3_status zs3_init_master(zs3_layout_t L, int32_t rank, int32_t dtype, int64_t begin, int64_t end,
                           const void* shard_flat, float* master, float* exp_avg, float* exp_avg_sq, void* stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if (begin < 0 || end < begin || end > L->shard_numel)
        return fail(ZS3_EINVAL, "range [%lld, %lld) outside [0, %lld]", (long long)begin, (long long)end,
                    (long long)L->shard_numel);
    if ((s = check_ptr16(shard_flat, "shard_flat")) != ZS3_OK) return s;
    if (master == nullptr || !aligned(master, 4)) return fail(ZS3_EINVAL, "master is NULL or not 4-byte aligned");
    if ((exp_avg != nullptr && !aligned(exp_avg, 4)) || (exp_avg_sq != nullptr && !aligned(exp_avg_sq, 4)))
        return fail(ZS3_EINVAL, "exp_avg or exp_avg_sq is not 4-byte aligned");
    const int64_t nb = end - begin;
    const void* arr[4] = {static_cast<const uint16_t*>(shard_flat) + begin, master + begin,
                          exp_avg != nullptr ? exp_avg + begin : nullptr,
                          exp_avg_sq != nullptr ? exp_avg_sq + begin : nullptr};
    const int64_t bytes[4] = {2 * nb, 4 * nb, 4 * nb, 4 * nb};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (arr[i] != nullptr && arr[j] != nullptr && overlap(arr[i], bytes[i], arr[j], bytes[j]))
                return fail(ZS3_EALIAS, "init arrays %d and %d overlap", i, j);
    if (nb == 0) return ok();
    Key key{{kOpInitMaster, device_id(), rank, begin, end}};
    Plan* plan = find_plan(L, key);
    if (plan == nullptr) {
        // alternating runs of real positions (widened) and padding (zeros)
        std::vector<std::pair<int64_t, int64_t>> runs;     // (begin, count), real runs tagged below
        std::vector<int32_t> real;
        auto add = [&](int64_t a, int64_t b, int32_t is_real) {
            if (b <= a) return;
            if (!runs.empty() && real.back() == is_real && runs.back().first + runs.back().second == a) {
                runs.back().second += b - a;
                return;
            }
            runs.emplace_back(a, b - a);
            real.push_back(is_real);
        };
        for (const Slot& p : L->params) {
            const int64_t r = p.offset + p.real(rank);
            add(std::max(begin, p.offset), std::min(end, r), 1);
            add(std::max(begin, r), std::min(end, p.offset + p.ps), 0);
        }
        std::vector<Span> spans;
        for (size_t i = 0; i < runs.size(); ++i) {
            const size_t first = spans.size();
            add_spans(&spans, runs[i].first, runs[i].second, 0, kAdamPiece);
            for (size_t k = first; k < spans.size(); ++k) spans[k].reserved = real[i];
        }
        if ((s = check_grid(static_cast<int64_t>(spans.size()), kAdamSub)) != ZS3_OK) return s;
        Plan np;
        np.n_pieces = static_cast<int64_t>(spans.size());
        std::vector<size_t> offs;
        if ((s = upload(&np, {{spans.data(), spans.size() * sizeof(Span)}}, 0, &offs)) != ZS3_OK) return s;
        np.off_pieces = offs[0];
        store_plan(L, std::move(key), std::move(np), &plan);
    }
    return hip_status(launch_init_master(dtype, plan->at<Span>(plan->off_pieces), plan->n_pieces,
                                         static_cast<const uint16_t*>(shard_flat), master, exp_avg, exp_avg_sq,
                                         static_cast<hipStream_t>(stream)),
                      "init-master kernel launch");
}

// ------------------------------------------------- (f4) offloaded Adam

zs3_status zs3_adam_step_offload(zs3_layout_t L, int32_t rank, int32_t dtype, int64_t begin, int64_t end,
                                 float* host_master, float* host_exp_avg, float* host_exp_avg_sq, float* stage,
                                 int64_t stage_elems, const void* grad_flat, void* shard_flat, const float* scale,
                                 const int32_t* nonfinite, const zs3_adam_params* hp, void* stream,
                                 void* copy_in_stream, void* copy_out_stream) {
    zs3_status s = check_layout_rank(L, rank);
    if (s != ZS3_OK) return s;
    if ((s = check_dtype(dtype)) != ZS3_OK) return s;
    if (hp == nullptr) return fail(ZS3_EINVAL, "hp is NULL");
    if (hp->step < 1) return fail(ZS3_EINVAL, "step %lld < 1", (long long)hp->step);
    if (begin < 0 || end < begin || end > L->shard_numel)
        return fail(ZS3_EINVAL, "range [%lld, %lld) outside [0, %lld]", (long long)begin, (long long)end,
                    (long long)L->shard_numel);
    float* host[3] = {host_master, host_exp_avg, host_exp_avg_sq};
    const int64_t nb = end - begin;
    for (int i = 0; i < 3; ++i) {
        if (host[i] == nullptr || !aligned(host[i], 4)) return fail(ZS3_EINVAL, "host state array %d is NULL or misaligned", i);
        for (int j = 0; j < i; ++j)
            if (overlap(host[i] + begin, 4 * nb, host[j] + begin, 4 * nb))
                return fail(ZS3_EALIAS, "host state arrays %d and %d overlap", j, i);
    }
    // staged: two slots of three arrays, each chunk + 8 elements (alignment room)
    const bool staged = stage != nullptr;
    const int64_t chunk = staged ? (stage_elems / 6 - 8) / 8 * 8 : 0;
    if (staged && !aligned(stage, 16)) return fail(ZS3_EINVAL, "stage is not 16-byte aligned");
    if (staged && chunk < 8) return fail(ZS3_EINVAL, "stage of %lld elements is too small (at least 96)", (long long)stage_elems);
    if (scale == nullptr || !aligned(scale, 4) || (nonfinite != nullptr && !aligned(nonfinite, 4)))
        return fail(ZS3_EINVAL, "scale is NULL, or scale or nonfinite is misaligned");
    if ((s = check_ptr16(grad_flat, "grad_flat")) != ZS3_OK) return s;
    if ((s = check_ptr16(shard_flat, "shard_flat")) != ZS3_OK) return s;
    const int64_t stage_bytes = staged ? 4 * 6 * (chunk + 8) : 0;
    if (overlap(stage, stage_bytes, static_cast<const uint16_t*>(grad_flat) + begin, 2 * nb) ||
        overlap(stage, stage_bytes, static_cast<uint16_t*>(shard_flat) + begin, 2 * nb) ||
        overlap(static_cast<const uint16_t*>(grad_flat) + begin, 2 * nb, static_cast<uint16_t*>(shard_flat) + begin, 2 * nb))
        return fail(ZS3_EALIAS, "stage, grad_flat and shard_flat overlap");
    if (nb == 0) return ok();
    float* mapped[3];
    for (int i = 0; i < 3; ++i) {
        hipPointerAttribute_t a;
        if (hipPointerGetAttributes(&a, host[i]) != hipSuccess || a.type != hipMemoryTypeHost ||
            a.devicePointer == nullptr) {
            (void)hipGetLastError();
            return fail(ZS3_EINVAL, "host state array %d is not pinned host memory mapped for the device", i);
        }
        mapped[i] = static_cast<float*>(a.devicePointer);
    }
    if (!staged) {
        // direct: the kernel reads and writes the host arrays through their
        // device mapping, so the state crosses the link once each way with
        // no copy engine, staging buffer or event in between
        return adam_launch(L, rank, dtype, begin, end, mapped[0], mapped[1], mapped[2], grad_flat, shard_flat, scale,
                           nonfinite, adam_consts(hp), stream);
    }

    const int dev = device_id();
    auto& ev = L->events[dev];
    if (ev.empty()) {
        for (int i = 0; i < 7; ++i) {
            hipEvent_t e;
            if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
                (void)hipGetLastError();
                for (hipEvent_t x : ev) (void)hipEventDestroy(x);
                ev.clear();
                return fail(ZS3_EHIP, "hipEventCreate failed");
            }
            ev.push_back(e);
        }
    }
    hipStream_t cs = static_cast<hipStream_t>(stream);
    hipStream_t in = copy_in_stream ? static_cast<hipStream_t>(copy_in_stream) : cs;
    hipStream_t out = copy_out_stream ? static_cast<hipStream_t>(copy_out_stream) : cs;
    hipEvent_t ev_start = ev[0], ev_in[2] = {ev[1], ev[2]}, ev_done[2] = {ev[3], ev[4]}, ev_out[2] = {ev[5], ev[6]};
    const AdamConsts c = adam_consts(hp);
    auto hip = [](hipError_t e, const char* what) { return hip_status(e, what); };

    // the copies start after everything already on the compute stream
    if ((s = hip(hipEventRecord(ev_start, cs), "event record")) != ZS3_OK) return s;
    if ((s = hip(hipStreamWaitEvent(in, ev_start, 0), "stream wait")) != ZS3_OK) return s;
    const int64_t n_chunks = (nb + chunk - 1) / chunk;
    bool used[2] = {false, false};
    for (int64_t i = 0; i < n_chunks; ++i) {
        const int64_t b = begin + i * chunk, e = std::min(end, b + chunk), n = e - b;
        const int slot = static_cast<int>(i & 1);
        float* base = stage + static_cast<int64_t>(slot) * 3 * (chunk + 8);
        const int64_t off = b & 7;      // keeps (slot array - b) 16-byte aligned, as the kernel's vector path needs
        float* dv[3] = {base + off, base + (chunk + 8) + off, base + 2 * (chunk + 8) + off};
        // _prepare_sub_group: swap in (after the slot's previous swap-out)
        if (used[slot] && (s = hip(hipStreamWaitEvent(in, ev_out[slot], 0), "stream wait")) != ZS3_OK) return s;
        for (int a = 0; a < 3; ++a)
            if ((s = hip(hipMemcpyAsync(dv[a], host[a] + b, 4 * n, hipMemcpyHostToDevice, in), "swap-in copy")) != ZS3_OK)
                return s;
        if ((s = hip(hipEventRecord(ev_in[slot], in), "event record")) != ZS3_OK) return s;
        // _optimizer_step on the staged partition
        if ((s = hip(hipStreamWaitEvent(cs, ev_in[slot], 0), "stream wait")) != ZS3_OK) return s;
        if ((s = adam_launch(L, rank, dtype, b, e, dv[0] - b, dv[1] - b, dv[2] - b, grad_flat, shard_flat, scale,
                             nonfinite, c, stream)) != ZS3_OK)
            return s;
        if ((s = hip(hipEventRecord(ev_done[slot], cs), "event record")) != ZS3_OK) return s;
        // _release_sub_group: swap out
        if ((s = hip(hipStreamWaitEvent(out, ev_done[slot], 0), "stream wait")) != ZS3_OK) return s;
        for (int a = 0; a < 3; ++a)
            if ((s = hip(hipMemcpyAsync(host[a] + b, dv[a], 4 * n, hipMemcpyDeviceToHost, out), "swap-out copy")) != ZS3_OK)
                return s;
        if ((s = hip(hipEventRecord(ev_out[slot], out), "event record")) != ZS3_OK) return s;
        used[slot] = true;
    }
    // the call is complete on the compute stream once both slots are swapped out
    for (int slot = 0; slot < 2; ++slot)
        if (used[slot] && (s = hip(hipStreamWaitEvent(cs, ev_out[slot], 0), "stream wait")) != ZS3_OK) return s;
    return ok();
}

}  // extern "C"
