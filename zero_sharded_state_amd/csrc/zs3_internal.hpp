// Internal declarations shared by the host planner / C ABI (api.cpp) and the
// HIP kernels (kernels.hip).  Device tables are plain structs so the host can
// build them and upload them in one copy.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace zs3 {

constexpr int kBlock = 256;             // threads per workgroup (4 wave64)

// Launch shape of each kernel family (tunable at build time).  A "piece" is
// the unit of the host-built work list; SUB one-shot workgroups share a
// piece, each moving VPT 16-byte vectors per thread.  Measured on MI355X,
// short-lived workgroups with one or two vectors per thread and
// non-temporal loads/stores stream HBM fastest.
#ifndef ZS3_COPY_VPT
#define ZS3_COPY_VPT 2
#endif
#ifndef ZS3_COPY_SUB
#define ZS3_COPY_SUB 4
#endif
#ifndef ZS3_RS_VPT
#define ZS3_RS_VPT 2
#endif
#ifndef ZS3_RS_SUB
#define ZS3_RS_SUB 8
#endif
#ifndef ZS3_RS_BATCH
#define ZS3_RS_BATCH 8
#endif
#ifndef ZS3_NORM_VPT
#define ZS3_NORM_VPT 2
#endif
#ifndef ZS3_NORM_GRID
#define ZS3_NORM_GRID 4096
#endif
#ifndef ZS3_ADAM_GPT
#define ZS3_ADAM_GPT 1
#endif
#ifndef ZS3_ADAM_SUB
#define ZS3_ADAM_SUB 8
#endif
// Non-temporal hints per family: on MI355X they help the copies, the
// reduce-scatter and the norm (Adam's vector path always uses them, with
// whole-line accesses and capped residency; see kernels.hip).
#ifndef ZS3_NT_COPY
#define ZS3_NT_COPY 1
#endif
#ifndef ZS3_NT_RS
#define ZS3_NT_RS 1
#endif
#ifndef ZS3_NT_NORM
#define ZS3_NT_NORM 1
#endif

constexpr int kCopyVPT = ZS3_COPY_VPT;
constexpr int kCopySub = ZS3_COPY_SUB;
constexpr int64_t kCopyPiece = int64_t(kBlock) * kCopyVPT * 8 * kCopySub;
constexpr int kRsVPT = ZS3_RS_VPT;
constexpr int kRsSub = ZS3_RS_SUB;
constexpr int64_t kRsPiece = int64_t(kBlock) * kRsVPT * 8 * kRsSub;
constexpr int kRsBatch = ZS3_RS_BATCH;     // sources whose loads are issued together
constexpr int kNormVPT = ZS3_NORM_VPT;     // vectors per thread per loop trip
constexpr int kNormGrid = ZS3_NORM_GRID;   // workgroups of the sum-of-squares pass (upper bound)
constexpr int kNormSub = 8;
constexpr int64_t kNormPiece = int64_t(kBlock) * kNormVPT * 8 * kNormSub;
constexpr int kAdamGPT = ZS3_ADAM_GPT;     // groups of 8 elements per thread
constexpr int kAdamSub = ZS3_ADAM_SUB;
constexpr int64_t kAdamPiece = int64_t(kBlock) * kAdamGPT * 8 * kAdamSub;
constexpr bool kNtCopy = ZS3_NT_COPY != 0;
constexpr bool kNtRs = ZS3_NT_RS != 0;
constexpr bool kNtNorm = ZS3_NT_NORM != 0;

// A contiguous copy: dst[0 .. count) = src[0 .. count), or zeros if src is
// null; if dst2 is set, also dst2[0 .. count2) = src[0 .. count2) from the
// same loads (count2 <= count, dst2 at the same address mod 16 as dst).
struct CopySeg {
    const uint16_t* src;
    uint16_t* dst;
    int64_t count;
    uint16_t* dst2;
    int64_t count2;
};

// One workgroup's share of a segment: elements [begin, begin + len) of it.
struct Piece {
    int64_t begin;
    int32_t seg;
    int32_t len;
};

// Reduce-scatter of one parameter's own slice.  The N source pointers of
// the segment are srcs[src_index .. src_index + N).  `slot` is the first of
// the parameter's partial sum-of-squares slots (see norm_slot_groups).
struct RsSeg {
    uint16_t* dst;
    int64_t real;        // averaged elements
    int64_t total;       // real + padding zeros (the partition size)
    int64_t src_index;
    int64_t slot;
};

// Partial sums of squares written by the reduce-scatter kernels: every
// parameter owns kNormSlotsPerGroup * norm_slot_groups(partition_size)
// consecutive slots, kSlotsPerWG per workgroup that can write its slice
// (one per workgroup, or one per wave), at a position fixed by
// the layout (partitioned parameters first, then persistent ones, each in
// ascending ds_id), so buckets reduced in any order or on any stream write
// disjoint slots.  A slice that needs one piece fewer than the bound zeroes
// the spare group.
#ifndef ZS3_NORM_WAVE_SLOTS
#define ZS3_NORM_WAVE_SLOTS 1
#endif
constexpr int kSlotsPerWG = ZS3_NORM_WAVE_SLOTS ? kBlock / 64 : 1;
constexpr int64_t kNormSlotsPerGroup = int64_t(kRsSub) * kSlotsPerWG;
__host__ __device__ constexpr int64_t norm_slot_groups(int64_t total) {
    return total <= kRsPiece ? 1 : (total + kRsPiece - 1) / kRsPiece;
}

// The wide reduce-scatter (many ranks): kRsWideSub workgroups of kBlock
// threads x 4 elements share a piece, one norm slot each; kRsWideBatch
// sources' loads in flight per round (kRsWideTailBatch for the ragged ends).
#ifndef ZS3_RS_WIDE_MIN
#define ZS3_RS_WIDE_MIN 16
#endif
#ifndef ZS3_RS_WIDE_BATCH
#define ZS3_RS_WIDE_BATCH 32
#endif
constexpr int kRsWideMin = ZS3_RS_WIDE_MIN;          // world sizes from which the wide kernel runs
constexpr int kRsWideBatch = ZS3_RS_WIDE_BATCH;
constexpr int kRsWideTailBatch = 16;
constexpr int kRsWideSub = static_cast<int>(kRsPiece / (int64_t(kBlock) * 4));
static_assert(kRsWideSub * int64_t(kBlock) * 4 == kRsPiece, "a piece must split into whole wide workgroups");
static_assert(kRsWideSub == kNormSlotsPerGroup, "one norm slot per wide workgroup");
inline bool rs_wide(int32_t world, bool co_aligned) { return co_aligned && world >= kRsWideMin; }

// Calls with few segments carry their whole plan in the kernel arguments
// (structure of arrays, < 2 KB each): the workgroup finds its segment from
// the prefix of piece counts and computes its range, with no loads before
// the data.  piece_start[nseg] is the total number of pieces.
constexpr int kCopyInlineSegs = 40;
struct CopyInline {
    int32_t nseg;
    int32_t piece_start[kCopyInlineSegs + 1];
    int32_t head[kCopyInlineSegs];            // elements before the destination is 16-byte aligned
    const uint16_t* src[kCopyInlineSegs];     // null: fill with zeros
    uint16_t* dst[kCopyInlineSegs];
    int64_t count[kCopyInlineSegs];
    uint16_t* dst2[kCopyInlineSegs];          // optional second destination (see CopySeg)
    int64_t count2[kCopyInlineSegs];
};

constexpr int kRsInlineSegs = 8;
constexpr int kRsInlineSrcs = 128;
struct RsInline {
    int32_t nseg;
    int32_t world;
    int32_t piece_start[kRsInlineSegs + 1];
    int32_t head[kRsInlineSegs];
    uint16_t* dst[kRsInlineSegs];
    int64_t real[kRsInlineSegs];
    int64_t total[kRsInlineSegs];
    int64_t slot[kRsInlineSegs];
    const uint16_t* src[kRsInlineSrcs];       // segment s, rank v at [s * world + v]
};

// Adam over a few long runs of real elements: the runs in the kernel arguments.
constexpr int kAdamInlineRuns = 16;
struct AdamInline {
    int32_t nrun;
    int32_t piece_start[kAdamInlineRuns + 1];
    int64_t begin[kAdamInlineRuns];
    int64_t count[kAdamInlineRuns];
};

// A run of flat-array positions handled by one workgroup (norm, Adam):
// absolute element indices [begin, begin + len).
struct Span {
    int64_t begin;
    int32_t len;
    int32_t reserved;
};

// fp32 constants of one Adam step, each rounded once from double.
struct AdamConsts {
    float lr, b1, b2, omb1, omb2, bc1, bc2, eps, lrwd;
    int32_t has_wd;
};

enum DType : int32_t { kFP16 = 1, kBF16 = 2 };

// kCopyGather: pack and unpack of one bucket in one launch (the unpack reads
// the own rank's part from the shard, which is what the pack puts on the wire).
// kCopyScatterPack: the send side of the non-contiguous gradient path.
enum CopyKind : int32_t { kCopyPartition = 1, kCopyPack = 2, kCopyUnpack = 3, kCopyGather = 4, kCopyScatterPack = 5 };

// Which gradient path a reduce-scatter launch serves (kernel names differ so
// that profiles tell them apart; the arithmetic is the same).
enum RsPath : int32_t { kRsContiguous = 1, kRsCoalesced = 2 };

// ---- launchers (kernels.hip) -------------------------------------------
// The calling thread's next launch records its start/end into these events.
void set_launch_events(hipEvent_t start, hipEvent_t stop);

hipError_t launch_copy(CopyKind kind, const CopySeg* segs, const Piece* pieces, int64_t n_pieces,
                       hipStream_t stream);

hipError_t launch_copy_inline(CopyKind kind, const CopyInline& plan, hipStream_t stream);
// partials: NULL, or the rank's slot array (fused sums of squares).
hipError_t launch_reduce_scatter_inline(RsPath path, int32_t dtype, const RsInline& plan, bool co_aligned,
                                        double* partials, hipStream_t stream);

hipError_t launch_reduce_scatter(RsPath path, int32_t dtype, const RsSeg* segs, const Piece* pieces,
                                 int64_t n_pieces, const uint16_t* const* srcs, int32_t world,
                                 bool co_aligned, double* partials, hipStream_t stream);

// Sums the slot array ([0, n_part) partitioned, the rest persistent) by
// n_blocks workgroups of `per_block` slots each into block_sums[2*n_blocks],
// then combines them as launch_grad_norm does.
hipError_t launch_norm_from_slots(const double* partials, int64_t n_slots, int64_t n_part, int64_t n_blocks,
                                  int64_t per_block, double* block_sums, double* sumsq, int32_t rank,
                                  int32_t world, int32_t finalize, double max_norm, double loss_scale,
                                  double* norm_out, float* scale_out, int32_t* nonfinite, hipStream_t stream);

// How the slot pass splits a slot array: about 1024 slots per workgroup, at
// most kNormSlotBlocks workgroups (the same split for every caller, so the
// allocation-free entry point sums in the same order as the cached one).
constexpr int64_t kNormSlotBlocks = 1024;
inline void norm_slot_split(int64_t n_slots, int64_t* n_blocks, int64_t* per_block) {
    int64_t b = (n_slots + 1023) / 1024;
    if (b > kNormSlotBlocks) b = kNormSlotBlocks;
    if (b < 1) b = 1;
    *n_blocks = b;
    *per_block = (n_slots + b - 1) / b;
}

// The allocation-free form of launch_norm_from_slots: the per-workgroup sums
// live in the library's static device array (2 * kNormSlotBlocks doubles per
// device) instead of caller- or layout-owned scratch.  Its address is looked
// up once per device (the first call with that device current).
hipError_t launch_norm_from_slots_static(const double* partials, int64_t n_slots, int64_t n_part, double* sumsq,
                                         int32_t rank, int32_t world, int32_t finalize, double max_norm,
                                         double loss_scale, double* norm_out, float* scale_out, int32_t* nonfinite,
                                         hipStream_t stream);

// Sums of squares of grad over the spans ([0, n_part) partitioned, the rest
// persistent) by n_blocks workgroups into partials[2*n_blocks], then one
// workgroup combines them into sumsq[rank], sumsq[world] and, if finalize,
// the norm, scale and flag.
hipError_t launch_grad_norm(int32_t dtype, const uint16_t* grad, const Span* spans, int64_t n_spans,
                            int64_t n_part, int64_t n_blocks, double* partials, double* sumsq, int32_t rank,
                            int32_t world, int32_t finalize, double max_norm, double loss_scale, double* norm_out,
                            float* scale_out, int32_t* nonfinite, hipStream_t stream);

hipError_t launch_adam_inline(int32_t dtype, const AdamInline& plan, float* master, float* exp_avg,
                              float* exp_avg_sq, const uint16_t* grad, uint16_t* shard, const float* scale,
                              const int32_t* nonfinite, const AdamConsts& c, bool vec_ok, hipStream_t stream);

hipError_t launch_adam(int32_t dtype, const Span* spans, int64_t n_spans, float* master,
                       float* exp_avg, float* exp_avg_sq, const uint16_t* grad, uint16_t* shard,
                       const float* scale, const int32_t* nonfinite, const AdamConsts& c,
                       bool vec_ok, hipStream_t stream);

// master[e] = widen(shard[e]) over real spans (reserved != 0), 0 over the
// others; exp_avg / exp_avg_sq (if not null) = 0 over every span.
hipError_t launch_init_master(int32_t dtype, const Span* spans, int64_t n_spans, const uint16_t* shard,
                              float* master, float* exp_avg, float* exp_avg_sq, hipStream_t stream);

}  // namespace zs3
