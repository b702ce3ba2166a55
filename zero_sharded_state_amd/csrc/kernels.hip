// HIP kernels of the ZeRO-3 shard step for gfx950 (MI355X).
//
// Every kernel here is HBM-bound streaming work (copies, fp32 adds, one
// fp64 square-and-add, ~40 fp32 ops of Adam per 28 bytes), so the design
// rules are: 128-bit loads and stores on 16-byte aligned addresses, enough
// bytes in flight per thread to cover HBM latency, one workgroup per
// host-built work item ("piece") so that no kernel searches for its data,
// and no MFMA (nothing here is a contraction).
//
// Pages cited: [codex] "03 · ZeRO-3: parameter sharding and the all-gather
// schedule" (ai-reference-codex), [csdn] "DeepSpeed ZeRO Stage 3: parameter
// partitioning ..." (adg.csdn.net), [llmnex] "ZeRO-3 core flow" (llmnex.top).
//
// Floating point: this file is compiled with -ffp-contract=off and
// correctly rounded fp32 division and square root, so each fp32 expression
// below is the sequence of IEEE operations it spells, with no fused
// multiply-add.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "zs3_internal.hpp"

// Scratch of the allocation-free norm entry point: the slot pass's two
// sums (partitioned, persistent) per workgroup, at most kNormSlotBlocks
// workgroups: 16 KiB.  Every GPU the library runs on holds its own copy
// until the process ends; every call on that GPU shares it.  In host code
// this name is only a stand-in for the symbol: kernels get the per-device
// address that hipGetSymbolAddress returns (static_norm_scratch below).
static __device__ __align__(256) double scratch[2 * zs3::kNormSlotBlocks];

namespace zs3 {
namespace {

// ---------------------------------------------------------------- 16-bit

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ float widen(uint32_t bits16);

template <>
__device__ __forceinline__ float widen<kFP16>(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

template <>
__device__ __forceinline__ float widen<kBF16>(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest, ties to even.
template <int D>
__device__ __forceinline__ uint32_t narrow(float f);

template <>
__device__ __forceinline__ uint32_t narrow<kFP16>(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <>
__device__ __forceinline__ uint32_t narrow<kBF16>(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // NaN stays NaN, quiet
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }
__device__ __forceinline__ uint32_t pack2(uint32_t a, uint32_t b) { return a | (b << 16); }

// Streaming 16-byte loads and stores, non-temporal when NT: every byte of
// these kernels is touched once per call.
template <bool NT>
__device__ __forceinline__ v4u ld_stream(const void* p) {
    const v4u* q = reinterpret_cast<const v4u*>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}
template <bool NT>
__device__ __forceinline__ void st_stream(void* p, v4u v) {
    v4u* q = reinterpret_cast<v4u*>(p);
    if constexpr (NT) __builtin_nontemporal_store(v, q);
    else *q = v;
}
// The copy kernels' 16-byte stores: non-temporal, with the sc1 cache-policy
// bit (CDNA3/4 global memory instructions).  On cache-cold copies larger
// than the Infinity Cache this measured 1.3% faster gathers than the plain
// non-temporal store (and slower reduce-scatter stores, which keep that).
// A vector store of ordinary data to a valid address; only the caching
// hint differs.  The compiler cannot see that this asm is a store, so it
// does not keep the wait states a store of more than 8 bytes needs before
// a VALU instruction may overwrite its data registers (two on this GPU
// family): the s_nop 1 inside the block provides them, whatever the
// compiler schedules next.
__device__ __forceinline__ void st_copy(void* p, v4u v) {
    v4u* q = reinterpret_cast<v4u*>(p);
    if constexpr (kNtCopy) asm volatile("global_store_dwordx4 %0, %1, off nt sc1\n\ts_nop 1" ::"v"(q), "v"(v) : "memory");
    else *q = v;
}

// Elements before `p` reaches 16-byte alignment (p is 2-byte aligned).
__device__ __forceinline__ int64_t head16(const void* p) {
    return static_cast<int64_t>(((16u - (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)) & 15u)) & 15u) >> 1);
}

// The 16 bytes that start SO bytes into the aligned block `lo` and run on
// into the next aligned block `hi` (16-bit data, SO even, 0 < SO < 16).
template <int SO>
__device__ __forceinline__ v4u shift_pair(v4u lo, v4u hi) {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    constexpr int d = SO / 4;
    v4u r;
    if constexpr (SO % 4 == 0) {
        r.x = w[d]; r.y = w[d + 1]; r.z = w[d + 2]; r.w = w[d + 3];
    } else {
        r.x = __builtin_amdgcn_alignbyte(w[d + 1], w[d], 2);
        r.y = __builtin_amdgcn_alignbyte(w[d + 2], w[d + 1], 2);
        r.z = __builtin_amdgcn_alignbyte(w[d + 3], w[d + 2], 2);
        r.w = __builtin_amdgcn_alignbyte(w[d + 4], w[d + 3], 2);
    }
    return r;
}

// 16 bytes of 16-bit data starting at p, whose byte address is SO (mod 16).
// SO != 0 reads the two aligned 16-byte blocks that hold those bytes and
// shifts; both blocks contain bytes of the requested range, so neither can
// cross into a page the range does not touch.  (The second block is the
// next lane's first and should hit in cache; non-temporal loads of both
// measured 5% slower.)
template <int SO, bool NT>
__device__ __forceinline__ v4u load_shift(const uint16_t* p) {
    if constexpr (SO == 0) {
        return ld_stream<NT>(p);
    } else {
        const v4u* a = reinterpret_cast<const v4u*>(reinterpret_cast<uintptr_t>(p) - SO);
        return shift_pair<SO>(a[0], a[1]);
    }
}

// Runtime-offset variant: `so` is uniform across the workgroup, so the
// switch is a scalar branch.
template <bool NT>
__device__ __forceinline__ v4u load_any(const uint16_t* p, uint32_t so) {
    switch (so) {
        case 0: return load_shift<0, NT>(p);
        case 2: return load_shift<2, NT>(p);
        case 4: return load_shift<4, NT>(p);
        case 6: return load_shift<6, NT>(p);
        case 8: return load_shift<8, NT>(p);
        case 10: return load_shift<10, NT>(p);
        case 12: return load_shift<12, NT>(p);
        default: return load_shift<14, NT>(p);
    }
}

// ------------------------------------------------------------ copy kernel
// Partition ([codex] 3.1: own range into the shard, padding zeroed), pack
// and unpack ([codex] 5.2: ds_id-ordered flat chunk, then per-parameter
// views of the gathered buffer) are all lists of contiguous copies; the
// host turns each call into segments and pieces.  kCopySub workgroups share
// a piece: after the piece's head elements (until the destination is
// 16-byte aligned, done by sub-block 0), sub-block `sub` moves vectors
// [sub*B*V, (sub+1)*B*V) and the last one the tail elements.

template <int SO>
__device__ __forceinline__ void copy_body(const uint16_t* src, uint16_t* dst, uint16_t* dst2, int64_t n2,
                                          int64_t i0, int64_t nv, int t) {
    v4u r[kCopyVPT];
    if constexpr (SO != 0) {
        // The lanes of a wave hold consecutive vectors, so a lane's second
        // block is the next lane's first: one load per lane, the second
        // block from a shuffle, and a load of its own only where there is no
        // next lane (the wave's last lane, the piece's last vector).  All
        // loads are issued before the first shuffle waits.  (Measured on
        // ragged fp16 gathers: 2% faster than two loads per lane.)
        const int lane = t & 63;
        v4u lo[kCopyVPT], hi[kCopyVPT];
#pragma unroll
        for (int u = 0; u < kCopyVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            const v4u* a = reinterpret_cast<const v4u*>(reinterpret_cast<uintptr_t>(src + 8 * i) - SO);
            lo[u] = v4u{0u, 0u, 0u, 0u};
            hi[u] = v4u{0u, 0u, 0u, 0u};
            if (i < nv) {
                lo[u] = ld_stream<kNtCopy>(a);
                if (lane == 63 || i + 1 >= nv) hi[u] = ld_stream<kNtCopy>(a + 1);
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            v4u nx;
            nx.x = static_cast<uint32_t>(__shfl_down(static_cast<int>(lo[u].x), 1, 64));
            nx.y = static_cast<uint32_t>(__shfl_down(static_cast<int>(lo[u].y), 1, 64));
            nx.z = static_cast<uint32_t>(__shfl_down(static_cast<int>(lo[u].z), 1, 64));
            nx.w = static_cast<uint32_t>(__shfl_down(static_cast<int>(lo[u].w), 1, 64));
            if (!(lane == 63 || i + 1 >= nv)) hi[u] = nx;
            r[u] = shift_pair<SO>(lo[u], hi[u]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kCopyVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            if (i < nv) r[u] = load_shift<SO, kNtCopy>(src + 8 * i);
        }
    }
#pragma unroll
    for (int u = 0; u < kCopyVPT; ++u) {
        const int64_t i = i0 + t + int64_t(u) * kBlock;
        if (i < nv) {
            st_copy(dst + 8 * i, r[u]);
            if (dst2 != nullptr && 8 * i < n2) {
                if (8 * i + 8 <= n2) {
                    st_copy(dst2 + 8 * i, r[u]);
                } else {
                    for (int e = 0; e < 8 && 8 * i + e < n2; ++e)
                        dst2[8 * i + e] = static_cast<uint16_t>((e & 1) ? hi16(r[u][e >> 1]) : lo16(r[u][e >> 1]));
                }
            }
        }
    }
}

// The work of one piece: elements [begin, begin + len) of a segment (and,
// for a two-destination segment, of its second destination where the
// segment's first count2 elements go).
__device__ __forceinline__ void copy_piece(const uint16_t* seg_src, uint16_t* seg_dst, uint16_t* seg_dst2,
                                           int64_t count2, int64_t begin, int64_t len, int sub, int t) {
    uint16_t* dst = seg_dst + begin;
    uint16_t* dst2 = seg_dst2 != nullptr ? seg_dst2 + begin : nullptr;
    int64_t n2 = seg_dst2 != nullptr ? count2 - begin : 0;     // elements of this piece that also go to dst2
    const uint16_t* src = seg_src != nullptr ? seg_src + begin : nullptr;
    int64_t n = len;
    int64_t h = head16(dst);
    if (h > n) h = n;
    if (sub == 0 && t < h) {
        const uint16_t x = src != nullptr ? src[t] : uint16_t(0);
        dst[t] = x;
        if (t < n2) dst2[t] = x;
    }
    dst += h;
    n -= h;
    if (src != nullptr) src += h;
    if (dst2 != nullptr) dst2 += h;
    n2 -= h;
    const int64_t nv = n >> 3;
    const int64_t i0 = int64_t(sub) * kBlock * kCopyVPT;
    if (src == nullptr) {
        const v4u z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kCopyVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            if (i < nv) st_copy(dst + 8 * i, z);
        }
    } else {
        switch (static_cast<uint32_t>(reinterpret_cast<uintptr_t>(src)) & 15u) {
            case 0: copy_body<0>(src, dst, dst2, n2, i0, nv, t); break;
            case 2: copy_body<2>(src, dst, dst2, n2, i0, nv, t); break;
            case 4: copy_body<4>(src, dst, dst2, n2, i0, nv, t); break;
            case 6: copy_body<6>(src, dst, dst2, n2, i0, nv, t); break;
            case 8: copy_body<8>(src, dst, dst2, n2, i0, nv, t); break;
            case 10: copy_body<10>(src, dst, dst2, n2, i0, nv, t); break;
            case 12: copy_body<12>(src, dst, dst2, n2, i0, nv, t); break;
            default: copy_body<14>(src, dst, dst2, n2, i0, nv, t); break;
        }
    }
    const int64_t rem = n & 7;
    if (sub == kCopySub - 1 && t < rem) {
        const uint16_t x = src != nullptr ? src[nv * 8 + t] : uint16_t(0);
        dst[nv * 8 + t] = x;
        if (nv * 8 + t < n2) dst2[nv * 8 + t] = x;
    }
}

// Piece `q` of a segment of `count` elements whose destination needs `head`
// elements to reach 16-byte alignment: the same split as the host's work
// lists (first piece head + P elements, then P at a time).
__device__ __forceinline__ void piece_range(int64_t q, int64_t count, int64_t head, int64_t P, int64_t* begin,
                                            int64_t* len) {
    const int64_t first = count < head + P ? count : head + P;
    if (q == 0) {
        *begin = 0;
        *len = first;
    } else {
        const int64_t b = first + (q - 1) * P;
        *begin = b;
        *len = count - b < P ? count - b : P;
    }
}

// Segment holding piece `pidx`: the number of segment starts at or below it.
template <int MAXSEG>
__device__ __forceinline__ int find_seg(const int32_t (&piece_start)[MAXSEG + 1], int nseg, int32_t pidx) {
    int s = 0;
#pragma unroll
    for (int j = 1; j < MAXSEG; ++j) s += (j < nseg && piece_start[j] <= pidx) ? 1 : 0;
    return s;
}

// One body, five kernel names (partition, pack, unpack, fused gather, the
// non-contiguous path's send-side pack) so that profiles attribute time to
// each step of the method.  Two ways to
// find the work: a device work list (k_copy) or, for calls with few
// segments, the whole plan in the kernel arguments (k_copy_inline), which
// saves the dependent loads of the list at the start of every launch.
template <int OP>
__global__ __launch_bounds__(kBlock) void k_copy(const CopySeg* __restrict__ segs,
                                                 const Piece* __restrict__ pieces) {
    const uint32_t pidx = blockIdx.x / kCopySub;
    const int sub = static_cast<int>(blockIdx.x % kCopySub);
    const Piece pc = pieces[pidx];
    const CopySeg sg = segs[pc.seg];
    copy_piece(sg.src, sg.dst, sg.dst2, sg.count2, pc.begin, pc.len, sub, threadIdx.x);
}

template <int OP>
__global__ __launch_bounds__(kBlock) void k_copy_inline(const CopyInline plan) {
    const int32_t pidx = static_cast<int32_t>(blockIdx.x / kCopySub);
    const int sub = static_cast<int>(blockIdx.x % kCopySub);
    const int s = find_seg<kCopyInlineSegs>(plan.piece_start, plan.nseg, pidx);
    int64_t begin, len;
    piece_range(pidx - plan.piece_start[s], plan.count[s], plan.head[s], kCopyPiece, &begin, &len);
    copy_piece(plan.src[s], plan.dst[s], plan.dst2[s], plan.count2[s], begin, len, sub, threadIdx.x);
}

// ----------------------------------------------------- sums of squares

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Deterministic workgroup sum: butterfly within each wave, then the four
// wave totals in wave order.  Result valid in thread 0.
__device__ __forceinline__ double block_sum(double x, double* sh) {
    x = wave_sum(x);
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    if (lane == 0) sh[wv] = x;
    __syncthreads();
    double r = 0.0;
    if (threadIdx.x == 0) {
        for (int i = 0; i < kBlock / 64; ++i) r += sh[i];
    }
    __syncthreads();
    return r;
}

template <int D>
__device__ __forceinline__ double sq(uint32_t bits16) {
    const double x = static_cast<double>(widen<D>(bits16));
    return x * x;
}

// The same exact square with one fp64 operation fewer: the square of an
// fp16 value (11-bit significand, |x| <= 65504, |x| >= 2^-24) is exact in
// fp32, and so is that of a bf16 value whose biased exponent lies in
// [64, 190] (8-bit significand, square a normal fp32); other bf16 values
// (zero, tiny, huge, inf, NaN) take the fp64 square.
template <int D>
__device__ __forceinline__ double sq_fast(uint32_t bits16) {
    const float x = widen<D>(bits16);
    if constexpr (D == kFP16) {
        return static_cast<double>(x * x);
    } else {
        const uint32_t e = (bits16 >> 7) & 0xffu;
        if (e - 64u <= 126u) return static_cast<double>(x * x);
        const double xd = static_cast<double>(x);
        return xd * xd;
    }
}

// ---------------------------------------------------- reduce-scatter kernel
// [codex] 6.2 / [csdn] step 3: own slice of the average of the N ranks'
// gradients.  Each output element is ((0 + g_0) + g_1 + ... + g_{N-1}) / N
// in fp32, ranks in order, then rounded to the 16-bit type; padding
// positions get 0.  Pieces are split among kRsSub workgroups as in k_copy.

struct Divider {
    float n;        // N as float
    float inv;      // 1/N, exact when N is a power of two
    bool pow2;
    __device__ __forceinline__ float operator()(float x) const {
        // x / 2^k and x * 2^-k are the same correctly rounded value
        return pow2 ? x * inv : x / n;
    }
};

// Source pointers of one segment: from a device table or from the kernel
// arguments.
struct TableSrcs {
    const uint16_t* const* p;
    __device__ __forceinline__ const uint16_t* operator()(int v) const { return p[v]; }
};
struct InlineSrcs {
    const RsInline& plan;
    int base;
    __device__ __forceinline__ const uint16_t* operator()(int v) const { return plan.src[base + v]; }
};

// Ragged ends are summed with 2-byte loads (a source may end at its last
// real element, so no 16-byte load may run past it).  The loads of
// kRsBatch sources are issued together and then added in rank order, so a
// thread waits for memory world/kRsBatch times instead of world times.
template <int D, class SRC>
__device__ __forceinline__ uint16_t rs_elem(const SRC& sp, int world, Divider div, int64_t k, int64_t real) {
    if (k >= real) return 0;
    float acc = 0.0f;
    for (int vb = 0; vb < world; vb += kRsBatch) {
        uint32_t x[kRsBatch];
#pragma unroll
        for (int j = 0; j < kRsBatch; ++j)
            if (vb + j < world) x[j] = sp(vb + j)[k];
#pragma unroll
        for (int j = 0; j < kRsBatch; ++j)
            if (vb + j < world) acc += widen<D>(x[j]);
    }
    return static_cast<uint16_t>(narrow<D>(div(acc)));
}

// The 8 elements [k, k + 8) of a vector that ends the real part or lies
// past it: its real elements with 2-byte loads, all 8 elements of a batch
// of sources in flight together, zeros for the padding.
template <int D, bool NORM, class SRC>
__device__ __forceinline__ void rs_tail_vector(uint16_t* dst, const SRC& sp, int world, Divider div, int64_t k,
                                               int64_t real, double& ss) {
    int64_t ne = real - k;
    if (ne < 0) ne = 0;
    if (ne > 8) ne = 8;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    if (ne > 0) {
        for (int vb = 0; vb < world; vb += kRsBatch) {
            uint32_t x[kRsBatch][8];
#pragma unroll
            for (int j = 0; j < kRsBatch; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (vb + j < world && e < ne) x[j][e] = sp(vb + j)[k + e];
#pragma unroll
            for (int j = 0; j < kRsBatch; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (vb + j < world && e < ne) acc[e] += widen<D>(x[j][e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint16_t x = e < ne ? static_cast<uint16_t>(narrow<D>(div(acc[e]))) : uint16_t(0);
        dst[e] = x;
        if constexpr (NORM) ss += sq_fast<D>(x);
    }
}

// Writes one element and, with NORM, adds the square of what was written.
template <int D, bool NORM, class SRC>
__device__ __forceinline__ void rs_put(uint16_t* dst, const SRC& sp, int world, Divider div, int64_t k,
                                       int64_t real, double& ss) {
    const uint16_t x = rs_elem<D>(sp, world, div, k, real);
    *dst = x;
    if constexpr (NORM) ss += sq_fast<D>(x);
}

// Returns the thread's sum of squares of the values it wrote (0 unless NORM).
template <int D, bool ALIGNED, bool NORM, class SRC>
__device__ __forceinline__ double rs_piece(const SRC& sp, uint16_t* seg_dst, int64_t real, int64_t begin,
                                           int64_t len, int world, Divider div, int sub, int t) {
    double ss = 0.0;
    int64_t k0 = begin;
    int64_t n = len;
    uint16_t* dst = seg_dst + k0;
    int64_t h = head16(dst);
    if (h > n) h = n;
    if (sub == 0 && t < h) rs_put<D, NORM>(dst + t, sp, world, div, k0 + t, real, ss);
    k0 += h;
    dst += h;
    n -= h;
    const int64_t nv = n >> 3;
    int64_t nfull = real > k0 ? (real - k0) >> 3 : 0;
    if (nfull > nv) nfull = nv;
    const int64_t i0 = int64_t(sub) * kBlock * kRsVPT;

    if (i0 + t < nfull) {
        float acc[kRsVPT][8];
#pragma unroll
        for (int u = 0; u < kRsVPT; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
        // Sources in batches of kRsBatch: all loads of a batch are issued
        // before its adds, which then run in rank order.
        for (int vb = 0; vb < world; vb += kRsBatch) {
            v4u x[kRsBatch][kRsVPT];
#pragma unroll
            for (int j = 0; j < kRsBatch; ++j) {
                if (vb + j < world) {
                    const uint16_t* s = sp(vb + j) + k0;
                    if constexpr (ALIGNED) {
#pragma unroll
                        for (int u = 0; u < kRsVPT; ++u) {
                            const int64_t i = i0 + t + int64_t(u) * kBlock;
                            if (i < nfull) x[j][u] = ld_stream<kNtRs>(s + 8 * i);
                        }
                    } else {
                        const uint32_t so = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s)) & 15u;
#pragma unroll
                        for (int u = 0; u < kRsVPT; ++u) {
                            const int64_t i = i0 + t + int64_t(u) * kBlock;
                            if (i < nfull) x[j][u] = load_any<kNtRs>(s + 8 * i, so);
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kRsBatch; ++j) {
                if (vb + j < world) {
#pragma unroll
                    for (int u = 0; u < kRsVPT; ++u) {
                        const int64_t i = i0 + t + int64_t(u) * kBlock;
                        if (i < nfull) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const uint32_t w = x[j][u][q];
                                acc[u][2 * q] += widen<D>(lo16(w));
                                acc[u][2 * q + 1] += widen<D>(hi16(w));
                            }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kRsVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            if (i < nfull) {
                uint32_t b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    b[e] = narrow<D>(div(acc[u][e]));
                    if constexpr (NORM) ss += sq_fast<D>(b[e]);
                }
                const v4u o = {pack2(b[0], b[1]), pack2(b[2], b[3]), pack2(b[4], b[5]), pack2(b[6], b[7])};
                st_stream<kNtRs>(dst + 8 * i, o);
            }
        }
    }
    // this sub-block's vectors that hold padding (the partial one and those past it)
    int64_t lo = i0 > nfull ? i0 : nfull;
    int64_t hi = i0 + int64_t(kBlock) * kRsVPT;
    if (hi > nv) hi = nv;
    for (int64_t i = lo + t; i < hi; i += kBlock) rs_tail_vector<D, NORM>(dst + 8 * i, sp, world, div, k0 + 8 * i, real, ss);
    const int64_t rem = n & 7;
    if (sub == kRsSub - 1 && t < rem) rs_put<D, NORM>(dst + nv * 8 + t, sp, world, div, k0 + nv * 8 + t, real, ss);
    return ss;
}

// ------------------------------------------ wide reduce-scatter (large N)
// With many ranks, every output element reads N sources: the kernel above
// then makes N/kRsBatch dependent rounds of loads per workgroup, and a
// bucket's slice fills few workgroups (a c5-sized bucket at N = 64: ~130).
// Here a piece is shared by kRsWideSub workgroups of 1024 elements; a
// thread holds 4 consecutive elements, reads them with one 8-byte load per
// source, and keeps kRsWideBatch sources' loads in flight, so a workgroup
// makes N/kRsWideBatch rounds and a bucket fills 4x the workgroups.  Each
// element's N adds still run in rank order (bit-identical results).  Used
// when every source is co-aligned with its destination modulo 16 bytes.

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

// 8 bytes (4 elements) at an 8-byte aligned address.
__device__ __forceinline__ void ld8(const uint16_t* p, uint32_t (&x)[2]) {
    v2u v;
    if constexpr (kNtRs) v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    else v = *reinterpret_cast<const v2u*>(p);
    x[0] = v.x;
    x[1] = v.y;
}

// `count` (<= 4) consecutive destination elements starting at slice
// position k, the first clamp(real - k, 0, count) of them real: their
// sources read with 2-byte loads, kRsWideTailBatch sources in flight.
template <int D, bool NORM, class SRC>
__device__ __forceinline__ void rs_wide_group(uint16_t* dst, const SRC& sp, int world, Divider div, int64_t k,
                                              int64_t real, int count, double& ss) {
    int64_t ne = real - k;
    if (ne < 0) ne = 0;
    if (ne > count) ne = count;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ne > 0) {
        for (int vb = 0; vb < world; vb += kRsWideTailBatch) {
            uint32_t x[kRsWideTailBatch][4];
#pragma unroll
            for (int j = 0; j < kRsWideTailBatch; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (vb + j < world && e < ne) x[j][e] = sp(vb + j)[k + e];
#pragma unroll
            for (int j = 0; j < kRsWideTailBatch; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (vb + j < world && e < ne) acc[e] += widen<D>(x[j][e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < count) {
            const uint16_t x = e < ne ? static_cast<uint16_t>(narrow<D>(div(acc[e]))) : uint16_t(0);
            dst[e] = x;
            if constexpr (NORM) ss += sq_fast<D>(x);
        }
    }
}

// Returns the thread's sum of squares of the values it wrote (0 unless NORM).
// Logical sub-block of a wide workgroup.  Workgroups are dispatched
// round-robin over the 8 XCDs, each with its own L2, and a piece's 32
// workgroups start at a multiple of 32: XCD x runs the workgroups with
// blockIdx = x (mod 8), and takes the 4 consecutive 1,024-element groups
// 4x .. 4x+3 of the piece.  Ragged slices start at 16-byte, not 128-byte,
// boundaries, so neighbouring groups share a line of every source; in one
// L2 it is fetched once.  Measured on the 64-rank set: 2.5% faster, and the
// L2 fetches 2.8% more than the sources hold instead of 6.6%.  A bijection
// of [0, 32): every group is still computed once, by a workgroup of its
// piece.
__device__ __forceinline__ int wide_sub(uint32_t b) {
    static_assert(kRsWideSub % 8 == 0, "a piece's workgroups must spread evenly over the XCDs");
    const int local = static_cast<int>(b % kRsWideSub);
    return (local % 8) * (kRsWideSub / 8) + local / 8;
}

template <int D, bool NORM, class SRC>
__device__ __forceinline__ double rs_piece_wide(const SRC& sp, uint16_t* seg_dst, int64_t real, int64_t begin,
                                                int64_t len, int world, Divider div, int sub, int t) {
    double ss = 0.0;
    int64_t k0 = begin;
    int64_t n = len;
    uint16_t* dst = seg_dst + k0;
    int64_t h = head16(dst);
    if (h > n) h = n;
    // the head (< 8 elements, until dst is 16-byte aligned): two groups of 4
    if (sub == 0 && t < 2 && 4 * t < h) {
        const int c = static_cast<int>(h - 4 * t < 4 ? h - 4 * t : 4);
        rs_wide_group<D, NORM>(dst + 4 * t, sp, world, div, k0 + 4 * t, real, c, ss);
    }
    k0 += h;
    dst += h;
    n -= h;
    const int64_t nq = n >> 2;                                // groups of 4 (8 bytes)
    int64_t nfull = real > k0 ? (real - k0) >> 2 : 0;
    if (nfull > nq) nfull = nq;
    const int64_t i = int64_t(sub) * kBlock + t;              // this thread's group
    if (i < nfull) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int vb = 0; vb < world; vb += kRsWideBatch) {
            uint32_t x[kRsWideBatch][2];
#pragma unroll
            for (int j = 0; j < kRsWideBatch; ++j)
                if (vb + j < world) ld8(sp(vb + j) + k0 + 4 * i, x[j]);
#pragma unroll
            for (int j = 0; j < kRsWideBatch; ++j) {
                if (vb + j < world) {
                    acc[0] += widen<D>(lo16(x[j][0]));
                    acc[1] += widen<D>(hi16(x[j][0]));
                    acc[2] += widen<D>(lo16(x[j][1]));
                    acc[3] += widen<D>(hi16(x[j][1]));
                }
            }
        }
        uint32_t b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            b[e] = narrow<D>(div(acc[e]));
            if constexpr (NORM) ss += sq_fast<D>(b[e]);
        }
        const v2u o = {pack2(b[0], b[1]), pack2(b[2], b[3])};
        v2u* q = reinterpret_cast<v2u*>(dst + 4 * i);
        if constexpr (kNtRs) __builtin_nontemporal_store(o, q);
        else *q = o;
    } else if (i < nq) {
        // the group holding the slice's real end, or padding past it
        rs_wide_group<D, NORM>(dst + 4 * i, sp, world, div, k0 + 4 * i, real, 4, ss);
    }
    const int64_t rem = n & 3;
    if (sub == kRsWideSub - 1 && t == 0 && rem > 0)
        rs_wide_group<D, NORM>(dst + 4 * nq, sp, world, div, k0 + 4 * nq, real, static_cast<int>(rem), ss);
    return ss;
}

// Pieces of a slice of `total` elements whose destination needs `head`
// elements to reach 16-byte alignment (the host's split), and the index of
// the piece that starts at `begin`.
__device__ __forceinline__ int64_t pieces_of(int64_t total, int64_t head) {
    const int64_t first = total < head + kRsPiece ? total : head + kRsPiece;
    return 1 + (total - first + kRsPiece - 1) / kRsPiece;
}
__device__ __forceinline__ int64_t piece_index(int64_t begin, int64_t head) {
    return begin == 0 ? 0 : 1 + (begin - head - kRsPiece) / kRsPiece;
}

// The partial sums of piece q, sub-block `sub` go to slot group q: one slot
// per workgroup (a workgroup sum) or, by default, one per wave (each wave's
// own sum, no barrier) at slot + (q*kRsSub + sub)*kSlotsPerWG + wave.  The
// last piece of a slice that needs one piece fewer than the slot bound also
// zeroes the spare group.
__device__ __forceinline__ void put_partial(double ss, double* partials, int64_t slot, int64_t q, int64_t actual,
                                            int64_t total, int sub, double* sh) {
    const bool spare = q == actual - 1 && actual < norm_slot_groups(total);
    if constexpr (kSlotsPerWG == 1) {
        const double s = block_sum(ss, sh);
        if (threadIdx.x == 0) {
            const int64_t at = slot + q * kRsSub + sub;
            partials[at] = s;
            if (spare) partials[at + kRsSub] = 0.0;
        }
    } else {
        // one slot per wave: no barrier, each wave's lane 0 writes its sum
        const double s = wave_sum(ss);
        if ((threadIdx.x & 63) == 0) {
            const int64_t at = slot + (q * kRsSub + sub) * kSlotsPerWG + (threadIdx.x >> 6);
            partials[at] = s;
            if (spare) partials[at + kNormSlotsPerGroup] = 0.0;
        }
    }
}

// Wide kernel: workgroup `sub` of piece q writes one slot, its workgroup sum
// (kRsWideSub workgroups per piece fill the group's kNormSlotsPerGroup slots).
__device__ __forceinline__ void put_partial_wide(double ss, double* partials, int64_t slot, int64_t q, int64_t actual,
                                                 int64_t total, int sub, double* sh) {
    const bool spare = q == actual - 1 && actual < norm_slot_groups(total);
    const double s = block_sum(ss, sh);
    if (threadIdx.x == 0) {
        const int64_t at = slot + q * kNormSlotsPerGroup + sub;
        partials[at] = s;
        if (spare) partials[at + kNormSlotsPerGroup] = 0.0;
    }
}

template <int D, bool NORM>
__device__ __forceinline__ void rs_table_wide(const RsSeg* __restrict__ segs, const Piece* __restrict__ pieces,
                                              const uint16_t* const* __restrict__ srcs, int world, Divider div,
                                              double* __restrict__ partials) {
    __shared__ double sh[kBlock / 64];
    const uint32_t pidx = blockIdx.x / kRsWideSub;
    const int sub = wide_sub(blockIdx.x);
    const Piece pc = pieces[pidx];
    const RsSeg sg = segs[pc.seg];
    const TableSrcs sp{srcs + sg.src_index};
    const double ss = rs_piece_wide<D, NORM>(sp, sg.dst, sg.real, pc.begin, pc.len, world, div, sub, threadIdx.x);
    if constexpr (NORM) {
        const int64_t head = head16(sg.dst);
        put_partial_wide(ss, partials, sg.slot, piece_index(pc.begin, head), pieces_of(sg.total, head), sg.total, sub,
                         sh);
    }
}

template <int D, bool NORM>
__device__ __forceinline__ void rs_inline_wide(const RsInline& plan, Divider div, double* __restrict__ partials) {
    __shared__ double sh[kBlock / 64];
    const int32_t pidx = static_cast<int32_t>(blockIdx.x / kRsWideSub);
    const int sub = wide_sub(blockIdx.x);
    const int s = find_seg<kRsInlineSegs>(plan.piece_start, plan.nseg, pidx);
    const int64_t q = pidx - plan.piece_start[s];
    int64_t begin, len;
    piece_range(q, plan.total[s], plan.head[s], kRsPiece, &begin, &len);
    const InlineSrcs sp{plan, s * plan.world};
    const double ss = rs_piece_wide<D, NORM>(sp, plan.dst[s], plan.real[s], begin, len, plan.world, div, sub,
                                             threadIdx.x);
    if constexpr (NORM)
        put_partial_wide(ss, partials, plan.slot[s], q, plan.piece_start[s + 1] - plan.piece_start[s], plan.total[s],
                         sub, sh);
}

template <int D, bool ALIGNED, bool NORM>
__device__ __forceinline__ void rs_table(const RsSeg* __restrict__ segs, const Piece* __restrict__ pieces,
                                         const uint16_t* const* __restrict__ srcs, int world, Divider div,
                                         double* __restrict__ partials) {
    __shared__ double sh[kBlock / 64];
    const uint32_t pidx = blockIdx.x / kRsSub;
    const int sub = static_cast<int>(blockIdx.x % kRsSub);
    const Piece pc = pieces[pidx];
    const RsSeg sg = segs[pc.seg];
    const TableSrcs sp{srcs + sg.src_index};
    const double ss = rs_piece<D, ALIGNED, NORM>(sp, sg.dst, sg.real, pc.begin, pc.len, world, div, sub, threadIdx.x);
    if constexpr (NORM) {
        const int64_t head = head16(sg.dst);
        put_partial(ss, partials, sg.slot, piece_index(pc.begin, head), pieces_of(sg.total, head), sg.total, sub, sh);
    }
}

template <int D, bool ALIGNED, bool NORM>
__device__ __forceinline__ void rs_inline(const RsInline& plan, Divider div, double* __restrict__ partials) {
    __shared__ double sh[kBlock / 64];
    const int32_t pidx = static_cast<int32_t>(blockIdx.x / kRsSub);
    const int sub = static_cast<int>(blockIdx.x % kRsSub);
    const int s = find_seg<kRsInlineSegs>(plan.piece_start, plan.nseg, pidx);
    const int64_t q = pidx - plan.piece_start[s];
    int64_t begin, len;
    piece_range(q, plan.total[s], plan.head[s], kRsPiece, &begin, &len);
    const InlineSrcs sp{plan, s * plan.world};
    const double ss = rs_piece<D, ALIGNED, NORM>(sp, plan.dst[s], plan.real[s], begin, len, plan.world, div, sub,
                                                 threadIdx.x);
    if constexpr (NORM)
        put_partial(ss, partials, plan.slot[s], q, plan.piece_start[s + 1] - plan.piece_start[s], plan.total[s], sub,
                    sh);
}

// One body, two kernel names per form: the contiguous path (all-reduce of a
// bucket, own interval kept) and the non-contiguous path's owner side
// (reduce of the N received chunks); profiles attribute time to each.
template <int D, bool ALIGNED, bool NORM>
__global__ __launch_bounds__(kBlock) void k_reduce_scatter(const RsSeg* __restrict__ segs,
                                                           const Piece* __restrict__ pieces,
                                                           const uint16_t* const* __restrict__ srcs,
                                                           int world, Divider div, double* __restrict__ partials) {
    rs_table<D, ALIGNED, NORM>(segs, pieces, srcs, world, div, partials);
}

template <int D, bool ALIGNED, bool NORM>
__global__ __launch_bounds__(kBlock) void k_reduce_scatter_inline(const RsInline plan, Divider div,
                                                                  double* __restrict__ partials) {
    rs_inline<D, ALIGNED, NORM>(plan, div, partials);
}

template <int D, bool ALIGNED, bool NORM>
__global__ __launch_bounds__(kBlock) void k_scatter_reduce(const RsSeg* __restrict__ segs,
                                                           const Piece* __restrict__ pieces,
                                                           const uint16_t* const* __restrict__ srcs,
                                                           int world, Divider div, double* __restrict__ partials) {
    rs_table<D, ALIGNED, NORM>(segs, pieces, srcs, world, div, partials);
}

template <int D, bool ALIGNED, bool NORM>
__global__ __launch_bounds__(kBlock) void k_scatter_reduce_inline(const RsInline plan, Divider div,
                                                                  double* __restrict__ partials) {
    rs_inline<D, ALIGNED, NORM>(plan, div, partials);
}

// Wide forms (many ranks, co-aligned sources), same two names per path.
template <int D, bool NORM>
__global__ __launch_bounds__(kBlock) void k_reduce_scatter_wide(const RsSeg* __restrict__ segs,
                                                                const Piece* __restrict__ pieces,
                                                                const uint16_t* const* __restrict__ srcs, int world,
                                                                Divider div, double* __restrict__ partials) {
    rs_table_wide<D, NORM>(segs, pieces, srcs, world, div, partials);
}

template <int D, bool NORM>
__global__ __launch_bounds__(kBlock) void k_reduce_scatter_wide_inline(const RsInline plan, Divider div,
                                                                       double* __restrict__ partials) {
    rs_inline_wide<D, NORM>(plan, div, partials);
}

template <int D, bool NORM>
__global__ __launch_bounds__(kBlock) void k_scatter_reduce_wide(const RsSeg* __restrict__ segs,
                                                                const Piece* __restrict__ pieces,
                                                                const uint16_t* const* __restrict__ srcs, int world,
                                                                Divider div, double* __restrict__ partials) {
    rs_table_wide<D, NORM>(segs, pieces, srcs, world, div, partials);
}

template <int D, bool NORM>
__global__ __launch_bounds__(kBlock) void k_scatter_reduce_wide_inline(const RsInline plan, Divider div,
                                                                       double* __restrict__ partials) {
    rs_inline_wide<D, NORM>(plan, div, partials);
}

// ------------------------------------------------------------ grad norm
// [llmnex] pitfall 1 / [codex] 6.3: local sums of squares, combined into one
// global norm and one clip coefficient.  Squares are taken in double, where
// the square of a 16-bit value is exact (helpers above the reduce-scatter,
// which can produce the same sums as it writes the averaged slice).

// Grid-stride over (span, sub-block) work items; each workgroup keeps one
// sum for partitioned spans [0, n_part) and one for persistent spans and
// writes them to partials[2*block], partials[2*block+1].
template <int D>
__global__ __launch_bounds__(kBlock) void k_sumsq(const uint16_t* __restrict__ grad,
                                                  const Span* __restrict__ spans, int64_t n_spans,
                                                  int64_t n_part, double* __restrict__ partials) {
    __shared__ double sh[kBlock / 64];
    const int t = threadIdx.x;
    double acc_part = 0.0, acc_pers = 0.0;
    const int64_t W = n_spans * kNormSub;
    for (int64_t w = blockIdx.x; w < W; w += gridDim.x) {
        const int64_t si = w / kNormSub;
        const int sub = static_cast<int>(w % kNormSub);
        const Span sp = spans[si];
        const uint16_t* p = grad + sp.begin;
        int64_t n = sp.len;
        int64_t h = head16(p);
        if (h > n) h = n;
        double acc = 0.0;
        if (sub == 0 && t < h) acc += sq<D>(p[t]);
        p += h;
        n -= h;
        const int64_t nv = n >> 3;
        const int64_t i0 = int64_t(sub) * kBlock * kNormVPT;
        v4u x[kNormVPT];
#pragma unroll
        for (int u = 0; u < kNormVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            if (i < nv) x[u] = ld_stream<kNtNorm>(p + 8 * i);
        }
#pragma unroll
        for (int u = 0; u < kNormVPT; ++u) {
            const int64_t i = i0 + t + int64_t(u) * kBlock;
            if (i < nv) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc += sq<D>(lo16(x[u][q]));
                    acc += sq<D>(hi16(x[u][q]));
                }
            }
        }
        const int64_t rem = n & 7;
        if (sub == kNormSub - 1 && t < rem) acc += sq<D>(p[nv * 8 + t]);
        if (si < n_part) acc_part += acc;
        else acc_pers += acc;
    }
    const double a = block_sum(acc_part, sh);
    const double b = block_sum(acc_pers, sh);
    if (t == 0) {
        partials[2 * blockIdx.x] = a;
        partials[2 * blockIdx.x + 1] = b;
    }
}

// Sum of the reduce-scatter's partial slots: workgroup b adds slots
// [b*per_block, (b+1)*per_block) in a fixed order, partitioned ones (index
// < n_part) and persistent ones apart.
__global__ __launch_bounds__(kBlock) void k_sum_slots(const double* __restrict__ partials, int64_t n_slots,
                                                      int64_t n_part, int64_t per_block,
                                                      double* __restrict__ block_sums) {
    __shared__ double sh[kBlock / 64];
    const int64_t b0 = int64_t(blockIdx.x) * per_block;
    int64_t b1 = b0 + per_block;
    if (b1 > n_slots) b1 = n_slots;
    double a = 0.0, b = 0.0;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += kBlock) {
        const double x = partials[i];
        if (i < n_part) a += x;
        else b += x;
    }
    a = block_sum(a, sh);
    b = block_sum(b, sh);
    if (threadIdx.x == 0) {
        block_sums[2 * blockIdx.x] = a;
        block_sums[2 * blockIdx.x + 1] = b;
    }
}

__global__ __launch_bounds__(kBlock) void k_norm_finalize(const double* __restrict__ partials, int64_t n_blocks,
                                                          double* __restrict__ sumsq, int rank, int world,
                                                          int finalize, double max_norm, double loss_scale,
                                                          double* norm_out, float* scale_out, int32_t* nonfinite) {
    __shared__ double sh[kBlock / 64];
    const int t = threadIdx.x;
    double a = 0.0, b = 0.0;
    for (int64_t i = t; i < n_blocks; i += kBlock) {
        a += partials[2 * i];
        b += partials[2 * i + 1];
    }
    a = block_sum(a, sh);
    b = block_sum(b, sh);
    if (t == 0) {
        sumsq[rank] = a;
        sumsq[world] = b;
        if (finalize) {
            double total = 0.0;
            for (int v = 0; v < world; ++v) total += (v == rank) ? a : sumsq[v];
            total += b;
            const bool bad = !(__builtin_fabs(total) <= 1.7976931348623157e308);
            const double norm = __builtin_sqrt(total);
            *norm_out = norm;
            *nonfinite = bad ? 1 : 0;
            if (bad) {
                *scale_out = __builtin_nanf("");
            } else {
                double coef = max_norm / (norm + 1e-6);
                if (coef > 1.0) coef = 1.0;
                *scale_out = static_cast<float>(coef / loss_scale);
            }
        }
    }
}

// ------------------------------------------------------------- Adam + cast
// [codex] 6.3: the optimizer steps only this rank's fp32 partition and the
// result is written back into the 16-bit shard.  One IEEE fp32 operation
// per line, in Kingma & Ba's order with bias correction and eps outside
// the square root.

__device__ __forceinline__ void adam1(float& w, float& m, float& v, float g16, float scale,
                                      const AdamConsts& c) {
    const float g = g16 * scale;
    if (c.has_wd) w = w - c.lrwd * w;
    m = c.b1 * m + c.omb1 * g;
    v = c.b2 * v + c.omb2 * (g * g);
    const float mh = m / c.bc1;
    const float vh = v / c.bc2;
    const float den = __builtin_sqrtf(vh) + c.eps;
    w = w - c.lr * (mh / den);
}

template <int D>
__device__ __forceinline__ void adam_scalar(int64_t e, float* w, float* m, float* v,
                                            const uint16_t* g, uint16_t* s, float scale,
                                            const AdamConsts& c) {
    float ww = w[e], mm = m[e], vv = v[e];
    adam1(ww, mm, vv, widen<D>(g[e]), scale, c);
    w[e] = ww;
    m[e] = mm;
    v[e] = vv;
    s[e] = static_cast<uint16_t>(narrow<D>(ww));
}

// One wave's 256*Q consecutive elements [wb, wb + 256*Q): lane l holds
// elements wb + 256k + 4l .. + 3 for k < Q, so every load and store
// instruction of the wave covers one contiguous run (1 KB of an fp32
// array, 512 B of a 16-bit one) and writes whole cache lines.  Loads and
// stores are non-temporal: each byte is touched once per step.  `skip`
// (the non-finite flag) is tested after the loads are issued.
template <int D, int Q>
__device__ __forceinline__ void adam_quads(int64_t wb, int lane, float* __restrict__ w, float* __restrict__ m,
                                           float* __restrict__ v, const uint16_t* __restrict__ g,
                                           uint16_t* __restrict__ s, float scale, bool skip, const AdamConsts& c) {
    v4f W[Q], M[Q], V[Q];
    v2u G[Q];
#pragma unroll
    for (int k = 0; k < Q; ++k) {
        const int64_t e = wb + 256 * k + 4 * lane;
        W[k] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(w + e));
        M[k] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(m + e));
        V[k] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(v + e));
        G[k] = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(g + e));
    }
    if (skip) return;
#pragma unroll
    for (int k = 0; k < Q; ++k) {
        const int64_t e = wb + 256 * k + 4 * lane;
        float ww[4], mm[4], vv[4];
        uint32_t out[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ww[q] = W[k][q];
            mm[q] = M[k][q];
            vv[q] = V[k][q];
            const uint32_t gw = G[k][q >> 1];
            adam1(ww[q], mm[q], vv[q], widen<D>((q & 1) ? hi16(gw) : lo16(gw)), scale, c);
            out[q] = narrow<D>(ww[q]);
        }
        __builtin_nontemporal_store(v4f{ww[0], ww[1], ww[2], ww[3]}, reinterpret_cast<v4f*>(w + e));
        __builtin_nontemporal_store(v4f{mm[0], mm[1], mm[2], mm[3]}, reinterpret_cast<v4f*>(m + e));
        __builtin_nontemporal_store(v4f{vv[0], vv[1], vv[2], vv[3]}, reinterpret_cast<v4f*>(v + e));
        __builtin_nontemporal_store(v2u{pack2(out[0], out[1]), pack2(out[2], out[3])}, reinterpret_cast<v2u*>(s + e));
    }
}

// Elements [b, b + n) of the flat arrays, one piece, sub-block `sub`: the
// head elements (until index % 8 == 0, where every array is 16-byte aligned
// when its base is), whole waves of 512*kAdamGPT elements as quads, and a
// wave block that runs past the end, element by element, as the tail.
template <int D, bool VEC>
__device__ __forceinline__ void adam_piece(int64_t b, int64_t n, int sub, int t, float* __restrict__ w,
                                           float* __restrict__ m, float* __restrict__ v,
                                           const uint16_t* __restrict__ g, uint16_t* __restrict__ s, float scale,
                                           bool skip, const AdamConsts& c) {
    if constexpr (!VEC) {
        if (skip) return;
        for (int64_t i = int64_t(sub) * kBlock + t; i < n; i += int64_t(kBlock) * kAdamSub)
            adam_scalar<D>(b + i, w, m, v, g, s, scale, c);
        return;
    } else {
        int64_t h = (8 - (b & 7)) & 7;
        if (h > n) h = n;
        b += h;
        n -= h;
        const int64_t ng = n >> 3;                                          // groups of 8
        const int64_t wg0 = int64_t(sub) * kBlock * kAdamGPT + int64_t(t >> 6) * 64 * kAdamGPT;   // wave's first
        if (wg0 + 64 * kAdamGPT <= ng) {
            adam_quads<D, 2 * kAdamGPT>(b + 8 * wg0, t & 63, w, m, v, g, s, scale, skip, c);
        } else if (!skip && wg0 < ng) {
            for (int e = 0; e < 8 * kAdamGPT; ++e) {
                const int64_t k = e * 64 + (t & 63);                         // element within the wave block
                if (wg0 + (k >> 3) < ng) adam_scalar<D>(b + 8 * wg0 + k, w, m, v, g, s, scale, c);
            }
        }
        if (skip) return;
        if (sub == 0 && t < h) adam_scalar<D>(b - h + t, w, m, v, g, s, scale, c);
        const int64_t rem = n & 7;
        if (sub == kAdamSub - 1 && t < rem) adam_scalar<D>(b + ng * 8 + t, w, m, v, g, s, scale, c);
    }
}

// The skip flag, the scale and the work description are read before any of
// them is tested, so their loads overlap instead of queueing one behind the
// other at the start of every (short-lived) workgroup.
template <int D, bool VEC>
__global__ __launch_bounds__(kBlock) void k_adam(const Span* __restrict__ spans, float* __restrict__ w,
                                                 float* __restrict__ m, float* __restrict__ v,
                                                 const uint16_t* __restrict__ g, uint16_t* __restrict__ s,
                                                 const float* __restrict__ scale_p,
                                                 const int32_t* __restrict__ nonfinite_p, AdamConsts c) {
    const uint32_t pidx = blockIdx.x / kAdamSub;
    const int sub = static_cast<int>(blockIdx.x % kAdamSub);
    const int32_t flag = nonfinite_p != nullptr ? *nonfinite_p : 0;
    const float scale = *scale_p;
    const Span sp = spans[pidx];
    adam_piece<D, VEC>(sp.begin, sp.len, sub, threadIdx.x, w, m, v, g, s, scale, flag != 0, c);
}

template <int D, bool VEC>
__global__ __launch_bounds__(kBlock) void k_adam_inline(const AdamInline plan, float* __restrict__ w,
                                                        float* __restrict__ m, float* __restrict__ v,
                                                        const uint16_t* __restrict__ g, uint16_t* __restrict__ s,
                                                        const float* __restrict__ scale_p,
                                                        const int32_t* __restrict__ nonfinite_p, AdamConsts c) {
    const int32_t pidx = static_cast<int32_t>(blockIdx.x / kAdamSub);
    const int sub = static_cast<int>(blockIdx.x % kAdamSub);
    const int32_t flag = nonfinite_p != nullptr ? *nonfinite_p : 0;
    const float scale = *scale_p;
    const int r = find_seg<kAdamInlineRuns>(plan.piece_start, plan.nrun, pidx);
    int64_t begin, len;
    const int64_t b0 = plan.begin[r];
    piece_range(pidx - plan.piece_start[r], plan.count[r], (8 - (b0 & 7)) & 7, kAdamPiece, &begin, &len);
    adam_piece<D, VEC>(b0 + begin, len, sub, threadIdx.x, w, m, v, g, s, scale, flag != 0, c);
}

// -------------------------------------------------- fp32 master partition
// [codex] 6.1: the optimizer's fp32 partition is made from the rank's
// 16-bit shard.  A span with `reserved` != 0 holds real positions (the
// exact widening of the shard); other spans are padding (0).  Momentum and
// variance start at 0 (each may be null: not written).  One-time set-up
// work, so plain coalesced element accesses.
template <int D>
__global__ __launch_bounds__(kBlock) void k_init_master(const Span* __restrict__ spans,
                                                        const uint16_t* __restrict__ shard, float* __restrict__ w,
                                                        float* __restrict__ m, float* __restrict__ v) {
    const uint32_t pidx = blockIdx.x / kAdamSub;
    const int sub = static_cast<int>(blockIdx.x % kAdamSub);
    const Span sp = spans[pidx];
    for (int64_t i = int64_t(sub) * kBlock + threadIdx.x; i < sp.len; i += int64_t(kBlock) * kAdamSub) {
        const int64_t e = sp.begin + i;
        w[e] = sp.reserved != 0 ? widen<D>(shard[e]) : 0.0f;
        if (m != nullptr) m[e] = 0.0f;
        if (v != nullptr) v[e] = 0.0f;
    }
}

inline dim3 grid_of(int64_t n) { return dim3(static_cast<uint32_t>(n)); }

// Dynamic LDS the vector Adam kernels reserve (and never use): with 160 KB
// of LDS per CU it lets two of their workgroups (eight waves) be resident
// per CU.  Adam streams eight arrays at once; at full residency their
// concurrent access streams slow HBM down (measured in one process on the
// same buffers: 4.74 ms at two workgroups per CU, 5.06 at three, 5.29 at
// eight, bit-identical results).
constexpr unsigned kAdamLdsReserve = 56 * 1024;

// Timing hook: when a host thread has set events, its next launch records
// the kernel's own start and end timestamps into them (hipExtLaunchKernel).
thread_local hipEvent_t t_start = nullptr;
thread_local hipEvent_t t_stop = nullptr;

template <typename K, typename... A>
void launch_shm(K kernel, dim3 grid, dim3 block, unsigned shm, hipStream_t stream, A... args) {
    if (t_start != nullptr || t_stop != nullptr) {
        hipEvent_t a = t_start, b = t_stop;
        t_start = t_stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, shm, stream, a, b, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shm, stream, args...);
    }
}

template <typename K, typename... A>
void launch(K kernel, dim3 grid, dim3 block, hipStream_t stream, A... args) {
    launch_shm(kernel, grid, block, 0, stream, args...);
}

}  // namespace

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
    t_start = start;
    t_stop = stop;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_copy(CopyKind kind, const CopySeg* segs, const Piece* pieces, int64_t n_pieces,
                       hipStream_t stream) {
    if (n_pieces <= 0) return hipSuccess;
    const dim3 g = grid_of(n_pieces * kCopySub), b(kBlock);
    switch (kind) {
        case kCopyPartition: launch(k_copy<kCopyPartition>, g, b, stream, segs, pieces); break;
        case kCopyPack: launch(k_copy<kCopyPack>, g, b, stream, segs, pieces); break;
        case kCopyUnpack: launch(k_copy<kCopyUnpack>, g, b, stream, segs, pieces); break;
        case kCopyScatterPack: launch(k_copy<kCopyScatterPack>, g, b, stream, segs, pieces); break;
        default: launch(k_copy<kCopyGather>, g, b, stream, segs, pieces); break;
    }
    return hipGetLastError();
}

hipError_t launch_copy_inline(CopyKind kind, const CopyInline& plan, hipStream_t stream) {
    const int64_t n_pieces = plan.piece_start[plan.nseg];
    if (n_pieces <= 0) return hipSuccess;
    const dim3 g = grid_of(n_pieces * kCopySub), b(kBlock);
    switch (kind) {
        case kCopyPartition: launch(k_copy_inline<kCopyPartition>, g, b, stream, plan); break;
        case kCopyPack: launch(k_copy_inline<kCopyPack>, g, b, stream, plan); break;
        case kCopyUnpack: launch(k_copy_inline<kCopyUnpack>, g, b, stream, plan); break;
        case kCopyScatterPack: launch(k_copy_inline<kCopyScatterPack>, g, b, stream, plan); break;
        default: launch(k_copy_inline<kCopyGather>, g, b, stream, plan); break;
    }
    return hipGetLastError();
}

static Divider make_divider(int32_t world) {
    Divider div;
    div.n = static_cast<float>(world);
    div.pow2 = (world & (world - 1)) == 0;
    div.inv = 1.0f / static_cast<float>(world);
    return div;
}

// The 16 forms of a reduce-scatter launch: path x dtype x co-alignment x
// fused sums of squares.
template <int D, bool A, bool NORM>
void rs_launch_table(RsPath path, dim3 g, hipStream_t stream, const RsSeg* segs, const Piece* pieces,
                     const uint16_t* const* srcs, int32_t world, Divider div, double* partials) {
    if (path == kRsCoalesced)
        launch((k_scatter_reduce<D, A, NORM>), g, dim3(kBlock), stream, segs, pieces, srcs, world, div, partials);
    else
        launch((k_reduce_scatter<D, A, NORM>), g, dim3(kBlock), stream, segs, pieces, srcs, world, div, partials);
}

template <int D, bool A, bool NORM>
void rs_launch_inline(RsPath path, dim3 g, hipStream_t stream, const RsInline& plan, Divider div, double* partials) {
    if (path == kRsCoalesced)
        launch((k_scatter_reduce_inline<D, A, NORM>), g, dim3(kBlock), stream, plan, div, partials);
    else
        launch((k_reduce_scatter_inline<D, A, NORM>), g, dim3(kBlock), stream, plan, div, partials);
}

template <int D, bool NORM>
void rs_launch_table_wide(RsPath path, dim3 g, hipStream_t stream, const RsSeg* segs, const Piece* pieces,
                          const uint16_t* const* srcs, int32_t world, Divider div, double* partials) {
    if (path == kRsCoalesced)
        launch((k_scatter_reduce_wide<D, NORM>), g, dim3(kBlock), stream, segs, pieces, srcs, world, div, partials);
    else
        launch((k_reduce_scatter_wide<D, NORM>), g, dim3(kBlock), stream, segs, pieces, srcs, world, div, partials);
}

template <int D, bool NORM>
void rs_launch_inline_wide(RsPath path, dim3 g, hipStream_t stream, const RsInline& plan, Divider div,
                           double* partials) {
    if (path == kRsCoalesced)
        launch((k_scatter_reduce_wide_inline<D, NORM>), g, dim3(kBlock), stream, plan, div, partials);
    else
        launch((k_reduce_scatter_wide_inline<D, NORM>), g, dim3(kBlock), stream, plan, div, partials);
}

template <int D>
void rs_dispatch_table(RsPath path, bool co, bool norm, dim3 g, hipStream_t stream, const RsSeg* segs,
                       const Piece* pieces, const uint16_t* const* srcs, int32_t world, Divider div,
                       double* partials) {
    if (co) {
        if (norm) rs_launch_table<D, true, true>(path, g, stream, segs, pieces, srcs, world, div, partials);
        else rs_launch_table<D, true, false>(path, g, stream, segs, pieces, srcs, world, div, partials);
    } else {
        if (norm) rs_launch_table<D, false, true>(path, g, stream, segs, pieces, srcs, world, div, partials);
        else rs_launch_table<D, false, false>(path, g, stream, segs, pieces, srcs, world, div, partials);
    }
}

template <int D>
void rs_dispatch_inline(RsPath path, bool co, bool norm, dim3 g, hipStream_t stream, const RsInline& plan,
                        Divider div, double* partials) {
    if (co) {
        if (norm) rs_launch_inline<D, true, true>(path, g, stream, plan, div, partials);
        else rs_launch_inline<D, true, false>(path, g, stream, plan, div, partials);
    } else {
        if (norm) rs_launch_inline<D, false, true>(path, g, stream, plan, div, partials);
        else rs_launch_inline<D, false, false>(path, g, stream, plan, div, partials);
    }
}

hipError_t launch_reduce_scatter(RsPath path, int32_t dtype, const RsSeg* segs, const Piece* pieces,
                                 int64_t n_pieces, const uint16_t* const* srcs, int32_t world, bool co_aligned,
                                 double* partials, hipStream_t stream) {
    if (n_pieces <= 0) return hipSuccess;
    const Divider div = make_divider(world);
    const bool norm = partials != nullptr;
    if (rs_wide(world, co_aligned)) {
        const dim3 g = grid_of(n_pieces * kRsWideSub);
        if (dtype == kFP16) {
            if (norm) rs_launch_table_wide<kFP16, true>(path, g, stream, segs, pieces, srcs, world, div, partials);
            else rs_launch_table_wide<kFP16, false>(path, g, stream, segs, pieces, srcs, world, div, partials);
        } else {
            if (norm) rs_launch_table_wide<kBF16, true>(path, g, stream, segs, pieces, srcs, world, div, partials);
            else rs_launch_table_wide<kBF16, false>(path, g, stream, segs, pieces, srcs, world, div, partials);
        }
        return hipGetLastError();
    }
    const dim3 g = grid_of(n_pieces * kRsSub);
    if (dtype == kFP16) rs_dispatch_table<kFP16>(path, co_aligned, norm, g, stream, segs, pieces, srcs, world, div, partials);
    else rs_dispatch_table<kBF16>(path, co_aligned, norm, g, stream, segs, pieces, srcs, world, div, partials);
    return hipGetLastError();
}

hipError_t launch_reduce_scatter_inline(RsPath path, int32_t dtype, const RsInline& plan, bool co_aligned,
                                        double* partials, hipStream_t stream) {
    const int64_t n_pieces = plan.piece_start[plan.nseg];
    if (n_pieces <= 0) return hipSuccess;
    const Divider div = make_divider(plan.world);
    const bool norm = partials != nullptr;
    if (rs_wide(plan.world, co_aligned)) {
        const dim3 g = grid_of(n_pieces * kRsWideSub);
        if (dtype == kFP16) {
            if (norm) rs_launch_inline_wide<kFP16, true>(path, g, stream, plan, div, partials);
            else rs_launch_inline_wide<kFP16, false>(path, g, stream, plan, div, partials);
        } else {
            if (norm) rs_launch_inline_wide<kBF16, true>(path, g, stream, plan, div, partials);
            else rs_launch_inline_wide<kBF16, false>(path, g, stream, plan, div, partials);
        }
        return hipGetLastError();
    }
    const dim3 g = grid_of(n_pieces * kRsSub);
    if (dtype == kFP16) rs_dispatch_inline<kFP16>(path, co_aligned, norm, g, stream, plan, div, partials);
    else rs_dispatch_inline<kBF16>(path, co_aligned, norm, g, stream, plan, div, partials);
    return hipGetLastError();
}

hipError_t launch_norm_from_slots(const double* partials, int64_t n_slots, int64_t n_part, int64_t n_blocks,
                                  int64_t per_block, double* block_sums, double* sumsq, int32_t rank,
                                  int32_t world, int32_t finalize, double max_norm, double loss_scale,
                                  double* norm_out, float* scale_out, int32_t* nonfinite, hipStream_t stream) {
    if (n_blocks > 0) {
        launch(k_sum_slots, grid_of(n_blocks), dim3(kBlock), stream, partials, n_slots, n_part, per_block, block_sums);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    launch(k_norm_finalize, dim3(1), dim3(kBlock), stream, static_cast<const double*>(block_sums), n_blocks, sumsq,
           rank, world, finalize, max_norm, loss_scale, norm_out, scale_out, nonfinite);
    return hipGetLastError();
}

// The device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU's copy has its own address).
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static hipError_t static_norm_scratch(double** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<double*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_norm_from_slots_static(const double* partials, int64_t n_slots, int64_t n_part, double* sumsq,
                                         int32_t rank, int32_t world, int32_t finalize, double max_norm,
                                         double loss_scale, double* norm_out, float* scale_out, int32_t* nonfinite,
                                         hipStream_t stream) {
    double* block_sums = nullptr;
    const hipError_t e = static_norm_scratch(&block_sums);
    if (e != hipSuccess) return e;
    int64_t n_blocks, per_block;
    norm_slot_split(n_slots, &n_blocks, &per_block);
    // every block sum the finalize pass reads is written by this call's slot
    // pass, so nothing left in the scratch by an earlier call is ever read
    return launch_norm_from_slots(partials, n_slots, n_part, n_blocks, per_block, block_sums, sumsq, rank, world,
                                  finalize, max_norm, loss_scale, norm_out, scale_out, nonfinite, stream);
}

hipError_t launch_grad_norm(int32_t dtype, const uint16_t* grad, const Span* spans, int64_t n_spans,
                            int64_t n_part, int64_t n_blocks, double* partials, double* sumsq, int32_t rank,
                            int32_t world, int32_t finalize, double max_norm, double loss_scale, double* norm_out,
                            float* scale_out, int32_t* nonfinite, hipStream_t stream) {
    if (n_blocks > 0) {
        if (dtype == kFP16)
            launch(k_sumsq<kFP16>, grid_of(n_blocks), dim3(kBlock), stream, grad, spans, n_spans, n_part, partials);
        else
            launch(k_sumsq<kBF16>, grid_of(n_blocks), dim3(kBlock), stream, grad, spans, n_spans, n_part, partials);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    launch(k_norm_finalize, dim3(1), dim3(kBlock), stream, partials, n_blocks, sumsq, rank, world,
                       finalize, max_norm, loss_scale, norm_out, scale_out, nonfinite);
    return hipGetLastError();
}

hipError_t launch_adam(int32_t dtype, const Span* spans, int64_t n_spans, float* master, float* exp_avg,
                       float* exp_avg_sq, const uint16_t* grad, uint16_t* shard, const float* scale,
                       const int32_t* nonfinite, const AdamConsts& c, bool vec_ok, hipStream_t stream) {
    if (n_spans <= 0) return hipSuccess;
    const dim3 g = grid_of(n_spans * kAdamSub), b(kBlock);
    if (dtype == kFP16) {
        if (vec_ok) launch_shm((k_adam<kFP16, true>), g, b, kAdamLdsReserve, stream, spans, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
        else launch((k_adam<kFP16, false>), g, b, stream, spans, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
    } else {
        if (vec_ok) launch_shm((k_adam<kBF16, true>), g, b, kAdamLdsReserve, stream, spans, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
        else launch((k_adam<kBF16, false>), g, b, stream, spans, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
    }
    return hipGetLastError();
}

hipError_t launch_adam_inline(int32_t dtype, const AdamInline& plan, float* master, float* exp_avg,
                              float* exp_avg_sq, const uint16_t* grad, uint16_t* shard, const float* scale,
                              const int32_t* nonfinite, const AdamConsts& c, bool vec_ok, hipStream_t stream) {
    const int64_t n_pieces = plan.piece_start[plan.nrun];
    if (n_pieces <= 0) return hipSuccess;
    const dim3 g = grid_of(n_pieces * kAdamSub), b(kBlock);
    if (dtype == kFP16) {
        if (vec_ok) launch_shm((k_adam_inline<kFP16, true>), g, b, kAdamLdsReserve, stream, plan, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
        else launch((k_adam_inline<kFP16, false>), g, b, stream, plan, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
    } else {
        if (vec_ok) launch_shm((k_adam_inline<kBF16, true>), g, b, kAdamLdsReserve, stream, plan, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
        else launch((k_adam_inline<kBF16, false>), g, b, stream, plan, master, exp_avg, exp_avg_sq, grad, shard, scale, nonfinite, c);
    }
    return hipGetLastError();
}

hipError_t launch_init_master(int32_t dtype, const Span* spans, int64_t n_spans, const uint16_t* shard,
                              float* master, float* exp_avg, float* exp_avg_sq, hipStream_t stream) {
    if (n_spans <= 0) return hipSuccess;
    const dim3 g = grid_of(n_spans * kAdamSub), b(kBlock);
    if (dtype == kFP16) launch(k_init_master<kFP16>, g, b, stream, spans, shard, master, exp_avg, exp_avg_sq);
    else launch(k_init_master<kBF16>, g, b, stream, spans, shard, master, exp_avg, exp_avg_sq);
    return hipGetLastError();
}

}  // namespace zs3
