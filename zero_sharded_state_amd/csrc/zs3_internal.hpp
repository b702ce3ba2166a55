// Internal declarations shared by the host planner / C ABI (api.cpp) and the
// HIP kernels (kernels.hip).  Device tables are plain structs so the host can
// build them and upload them in one copy.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace zs3 {

constexpr int kBlock = 256;             // threads per workgroup (4 wave64)

// Elements of one workgroup's piece, per kernel family.  A piece is the
// unit of the host-built work list: one workgroup handles exactly one.
constexpr int kCopyVPT = 8;             // 16-byte vectors per thread
constexpr int64_t kCopyPiece = int64_t(kBlock) * kCopyVPT * 8;
constexpr int kRsVPT = 2;
constexpr int64_t kRsPiece = int64_t(kBlock) * kRsVPT * 8;
constexpr int kNormVPT = 8;
constexpr int64_t kNormPiece = int64_t(kBlock) * kNormVPT * 8;
constexpr int kAdamGPT = 2;             // groups of 8 elements per thread
constexpr int64_t kAdamPiece = int64_t(kBlock) * kAdamGPT * 8;

// A contiguous copy: dst[0 .. count) = src[0 .. count), or zeros if src is null.
struct CopySeg {
    const uint16_t* src;
    uint16_t* dst;
    int64_t count;
    int64_t reserved;
};

// One workgroup's share of a segment: elements [begin, begin + len) of it.
struct Piece {
    int64_t begin;
    int32_t seg;
    int32_t len;
};

// Reduce-scatter of one parameter's own slice.  The N source pointers of
// the segment are srcs[src_index .. src_index + N).
struct RsSeg {
    uint16_t* dst;
    int64_t real;        // averaged elements
    int64_t total;       // real + padding zeros (the partition size)
    int64_t src_index;
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

enum CopyKind : int32_t { kCopyPartition = 1, kCopyPack = 2, kCopyUnpack = 3 };

// ---- launchers (kernels.hip) -------------------------------------------
hipError_t launch_copy(CopyKind kind, const CopySeg* segs, const Piece* pieces, int64_t n_pieces,
                       hipStream_t stream);

hipError_t launch_reduce_scatter(int32_t dtype, const RsSeg* segs, const Piece* pieces,
                                 int64_t n_pieces, const uint16_t* const* srcs, int32_t world,
                                 bool co_aligned, hipStream_t stream);

// Per-workgroup sums of squares of grad[span] (spans [0, n_part) partitioned,
// [n_part, n_spans) persistent), then one workgroup combines them into
// sumsq[rank], sumsq[world] and, if finalize, the norm, scale and flag.
hipError_t launch_grad_norm(int32_t dtype, const uint16_t* grad, const Span* spans,
                            int64_t n_spans, int64_t n_part, double* partials, double* sumsq,
                            int32_t rank, int32_t world, int32_t finalize, double max_norm,
                            double loss_scale, double* norm_out, float* scale_out,
                            int32_t* nonfinite, hipStream_t stream);

hipError_t launch_adam(int32_t dtype, const Span* spans, int64_t n_spans, float* master,
                       float* exp_avg, float* exp_avg_sq, const uint16_t* grad, uint16_t* shard,
                       const float* scale, const int32_t* nonfinite, const AdamConsts& c,
                       bool vec_ok, hipStream_t stream);

}  // namespace zs3
