/*
 * zs3.h -- C ABI of the ZeRO-3 shard-step library (libzs3.so, HIP on gfx950).
 *
 * One GPU's share of a ZeRO stage-3 data-parallel training step.  The N
 * data-parallel ranks are N "virtual ranks": every buffer a real rank would
 * receive from its peers is an ordinary device buffer here, so the
 * library's kernels are exactly the local work of a rank around the
 * collectives.
 *
 * Pages cited (titles, then the section of each passage):
 *   [codex]  "03 · ZeRO-3: parameter sharding and the all-gather schedule"
 *            (DeepSpeed chapter, ai-reference-codex.pages.dev)
 *   [csdn]   "DeepSpeed ZeRO Stage 3: parameter partitioning ..." (adg.csdn.net)
 *   [llmnex] "ZeRO-3 core flow: the setting that also shards the parameters"
 *            (llmnex.top)
 *
 * Conventions shared by every call
 *   - Element counts and offsets are in elements of the buffer's type.
 *   - 16-bit buffers (parameters, gradients, shards, chunks) hold fp16 or
 *     bf16 values, selected by `dtype`; fp32 buffers hold float.
 *   - Device pointers ("dev") are caller-owned device memory (for example
 *     torch tensors' data pointers).  They must be 2-byte aligned (16-bit
 *     data) or 4-byte aligned (fp32); 16-byte alignment enables the
 *     128-bit fast paths but is not required.
 *   - Host arrays ("host") are read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call that
 *     takes a stream only enqueues work on it and returns; none
 *     synchronises (except the first use of a call shape and a full table
 *     cache, below).  Outputs are ready when the stream reaches that point.
 *   - All arguments are validated before any work is enqueued: on an
 *     argument error nothing is enqueued and the return value says why;
 *     zs3_last_error() gives a message (thread-local).  A HIP or allocation
 *     failure (ZS3_EHIP, ZS3_ENOMEM) in a call that launches several kernels
 *     (separate pack and unpack, pack and reduce, the offload pipeline) may
 *     leave the earlier launches enqueued.  Nothing throws across the ABI.
 *   - A layout caches small device tables (segment and work lists, keyed by
 *     the call's parameters and pointers).  The first call with a new key
 *     allocates and uploads its table synchronously; later identical calls
 *     reuse it.  Cached tables are freed by zs3_layout_destroy, which first
 *     waits for the device to go idle, and when a layout already holds
 *     16384 of them: the next call with a new key then waits for the
 *     device to go idle and frees them all before it builds its own (the
 *     only case in which a call synchronises).
 *   - Calls on one layout from several host threads must be serialised by
 *     the caller.  zs3_grad_norm and zs3_grad_norm_partials keep device
 *     scratch in the layout, one per call shape and stream handle: norm
 *     calls on different streams may overlap, and calls on one stream are
 *     ordered by it.  (A stream destroyed with norm work still pending must
 *     not be replaced by a new stream with the same handle before that work
 *     is done.)
 */
#ifndef ZS3_H
#define ZS3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZS3_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define ZS3_API __attribute__((visibility("default")))
#else
#define ZS3_API
#endif

typedef int32_t zs3_status;

enum {
    ZS3_OK = 0,
    ZS3_EINVAL = -1,     /* null pointer, size, rank or world size out of range, numel < 1 */
    ZS3_EDTYPE = -2,     /* dtype is neither ZS3_FP16 nor ZS3_BF16 */
    ZS3_EDUPID = -3,     /* a ds_id appears twice */
    ZS3_ENOTFOUND = -4,  /* a ds_id is not in the layout */
    ZS3_EPERSIST = -5,   /* a persistent (never partitioned) parameter where only partitioned ones may be */
    ZS3_EALIAS = -6,     /* an output overlaps an input it must not overlap */
    ZS3_EHIP = -7,       /* a HIP runtime call or kernel launch failed */
    ZS3_ENOMEM = -8      /* host or device allocation failed */
};

enum { ZS3_FP16 = 1, ZS3_BF16 = 2 };          /* 16-bit storage types */
enum { ZS3_PACK = 1, ZS3_UNPACK = 2, ZS3_REDUCE = 4 };   /* gather / scatter modes (bit mask) */
enum { ZS3_GATHER_BUCKETS = 1, ZS3_REDUCE_BUCKETS = 2 };

typedef struct zs3_layout* zs3_layout_t;

/* Adam hyperparameters.  The fp32 constants of a step (lr, beta1, beta2,
 * 1-beta1, 1-beta2, 1-beta1^step, 1-beta2^step, eps, lr*weight_decay) are
 * each computed in double from these and rounded once to float. */
typedef struct {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;   /* decoupled: w -= (lr*wd)*w before the update */
    int64_t step;          /* t >= 1 */
} zs3_adam_params;

/* ---------------------------------------------------------------- misc */

ZS3_API int32_t zs3_abi_version(void);
ZS3_API const char* zs3_status_str(zs3_status s);
/* Message of the last failed call on this host thread ("" if none). */
ZS3_API const char* zs3_last_error(void);

/* Instrumentation (for callers that measure kernels, not part of the method):
 * the next kernel this host thread launches through any zs3 call records its
 * own start and end timestamps into start_event / stop_event (hipEvent_t,
 * created by the caller, either may be NULL), as hipExtLaunchKernel does; no
 * extra commands are enqueued.  The setting applies to exactly one launch
 * (calls that launch two kernels time the first).  Always returns ZS3_OK. */
ZS3_API zs3_status zs3_time_next_launch(void* start_event, void* stop_event);

/* ------------------------------------------------------------- layout
 * [codex] 3.1: rank r holds elements [r*partition_size, (r+1)*partition_size)
 * of every flattened parameter.  [codex] 5.3: parameters with
 * numel < persistence_threshold are never partitioned: every rank holds
 * them whole.  [codex] 5.2: the coalesced gather orders parameters by
 * ds_id, so a rank's flat shard lists parameters in ascending ds_id.
 *
 * partition_size = ceil(numel / world_size) for partitioned parameters and
 * numel for persistent ones; positions >= numel of the padded flat
 * parameter are zero padding.  A rank's flat shard (and its flat gradient
 * and fp32 state) has shard_numel = sum of partition sizes elements, each
 * parameter at shard_offset = prefix sum in ascending ds_id.
 *
 * zs3_layout_create: ds_id[i] >= 0 unique, numel[i] >= 1, n_params >= 0,
 * world_size >= 1, threshold >= 0 (host arrays of n_params).  Host-only:
 * no device work.  *out receives a handle to release with
 * zs3_layout_destroy.
 */
ZS3_API zs3_status zs3_layout_create(int32_t world_size, int64_t persistence_threshold,
                             int32_t n_params, const int64_t* ds_id, const int64_t* numel,
                             zs3_layout_t* out);
/* Waits for the device to go idle, frees cached device tables and the handle.
 * NULL is ignored. */
ZS3_API void zs3_layout_destroy(zs3_layout_t layout);

/* Counts and per-parameter facts; any output pointer may be NULL. */
ZS3_API zs3_status zs3_layout_info(zs3_layout_t layout, int32_t* world_size, int64_t* persistence_threshold,
                           int32_t* n_params, int64_t* shard_numel, int64_t* bytes_per_rank);
/* bytes_per_rank = 16 * shard_numel: 16-bit param + 16-bit grad + fp32
 * master, momentum, variance per held element ([codex] section 1, 16 Psi/N;
 * [llmnex] section 1, 2 + 2 + 12 bytes). */
/* The same two totals alone (either output may be NULL). */
ZS3_API zs3_status zs3_layout_totals(zs3_layout_t layout, int64_t* shard_numel, int64_t* bytes_per_rank);

/* The index-th parameter in ascending ds_id order (0 <= index < n_params). */
ZS3_API zs3_status zs3_layout_param_at(zs3_layout_t layout, int32_t index, int64_t* ds_id, int64_t* numel,
                               int64_t* partition_size, int32_t* persistent, int64_t* shard_offset);
/* The same facts by ds_id. */
ZS3_API zs3_status zs3_layout_param(zs3_layout_t layout, int64_t ds_id, int64_t* numel,
                            int64_t* partition_size, int32_t* persistent, int64_t* shard_offset);
/* [lo, hi) of the flattened parameter that `rank` holds real data for
 * (hi == lo when the rank's range lies wholly in the padding). */
ZS3_API zs3_status zs3_layout_own_range(zs3_layout_t layout, int64_t ds_id, int32_t rank,
                                int64_t* lo, int64_t* hi);

/* ------------------------------------------------------- host planning
 * Bucket plans.  kind = ZS3_GATHER_BUCKETS: non-persistent parameters in
 * ascending ds_id, filled up to `limit` full elements ([codex] 5.2: a
 * prefetch fills up to the prefetch bucket size).  kind =
 * ZS3_REDUCE_BUCKETS: every parameter in descending ds_id (backward
 * arrival order), filled up to `limit` full elements ([codex] 6.2: grads
 * collect in a bucket that is reduced when full).  Greedy: a bucket closes
 * before a parameter that would take it past `limit`, unless it is empty.
 * Outputs: *n_buckets; bucket b is ds_ids_out[starts[b] .. starts[b+1]).
 * starts (host) needs n_buckets+1 entries and ds_ids_out (host) n_params;
 * if cap (the capacity of starts) is too small, ZS3_EINVAL is returned with
 * *n_buckets set to the number needed.
 */
ZS3_API zs3_status zs3_plan_buckets(zs3_layout_t layout, int32_t kind, int64_t limit, int32_t cap,
                            int32_t* n_buckets, int32_t* starts, int64_t* ds_ids_out);

/* Sub-groups ([codex] 6.1: the optimizer splits the parameters into
 * sub-groups of at most sub_group_size elements, its unit of stepping):
 * contiguous [begin, end) ranges of the rank's flat shard, greedy in
 * ascending ds_id, counted in shard elements, never splitting a parameter.
 * begin_end (host) receives 2*n_groups values; cap is its capacity in
 * groups (see zs3_plan_buckets for the too-small case). */
ZS3_API zs3_status zs3_sub_groups(zs3_layout_t layout, int64_t sub_group_size, int32_t cap,
                          int32_t* n_groups, int64_t* begin_end);

/* Sizes of a gather bucket: chunk_numel = sum of partition sizes (one
 * rank's chunk), full_numel = sum of numels (the gathered flat buffer). */
ZS3_API zs3_status zs3_bucket_sizes(zs3_layout_t layout, int32_t n, const int64_t* ds_ids,
                            int64_t* chunk_numel, int64_t* full_numel);

/* ---------------------------------------------------- (1) partition
 * [codex] 3.1: right after construction each parameter's own element range
 * is copied into the rank's shard; [codex] 5.3: persistent parameters are
 * copied whole.
 *
 * For each of the n requested parameters (ds_ids, host, any order, no
 * duplicates), copies the rank's own range of full_params[i] (dev, numel
 * 16-bit elements, the flattened parameter) to shard_flat[shard_offset ..]
 * (dev, shard_numel elements) and writes 0 to the padding positions of its
 * partition.  Other positions of shard_flat are not touched.
 */
ZS3_API zs3_status zs3_partition(zs3_layout_t layout, int32_t rank, int32_t dtype, int32_t n,
                         const int64_t* ds_ids, const void* const* full_params,
                         void* shard_flat, void* stream);

/* ------------------------------------------ (2) all_gather_coalesced
 * [codex] 5.2: the shards of the requested group are ordered by ds_id and
 * joined into one flat buffer, one collective gathers the whole group, and
 * each parameter's data becomes a view of the gathered flat buffer.
 * [codex] section 7: a wrong order silently yields wrong parameters, so the
 * order is fixed by ds_id whatever the request order.
 *
 * The bucket is the n parameters ds_ids (host, any order, no duplicates,
 * none persistent).  Let j run over them in ascending ds_id, c_j = prefix
 * sum of partition sizes, f_j = prefix sum of numels.
 *   mode & ZS3_PACK:   own_chunk[c_j + k] = shard_flat[shard_offset_j + k],
 *                      k < partition_size_j (padding included).
 *                      shard_flat: dev, the rank's flat shard.
 *                      own_chunk: dev, chunk_numel elements.
 *   mode & ZS3_UNPACK: full_flat[f_j + v*ps_j + k] = rank_chunks[v][c_j + k]
 *                      for every rank v and every k with v*ps_j + k < numel_j
 *                      (padding is dropped).  rank_chunks: host array of N
 *                      dev pointers, each chunk_numel elements (the
 *                      all-gather's rank-major output, one pointer per
 *                      rank).  full_flat: dev, full_numel elements.
 *                      full_offsets (host, n entries, may be NULL) receives
 *                      f_j for the i-th requested ds_id: parameter i is the
 *                      view full_flat + full_offsets[i] of numel_i elements.
 * With both bits the pack runs first; rank_chunks[rank] may then be
 * own_chunk.  Unused pointers may be NULL.
 */
ZS3_API zs3_status zs3_gather_coalesced(zs3_layout_t layout, int32_t rank, int32_t dtype, int32_t mode,
                                int32_t n, const int64_t* ds_ids, const void* shard_flat,
                                void* own_chunk, const void* const* rank_chunks, void* full_flat,
                                int64_t* full_offsets, void* stream);

/* Several gather buckets in one launch.  [codex] 5.2: each prefetch fills one
 * bucket and gathers it with one coalesced collective; [llmnex] section 4
 * (pitfalls): buckets that are too small make the step latency-bound.  This
 * call does exactly what n_buckets calls of zs3_gather_coalesced with
 * mode = ZS3_PACK | ZS3_UNPACK (the wire's own slot being the pack's
 * output) would do, bucket by bucket, with the same results bit for bit,
 * but as one kernel launch.
 * Bucket b is ds_ids[bucket_start[b] .. bucket_start[b+1]) (host; any order
 * inside a bucket, none persistent, no ds_id in two buckets; bucket_start
 * has n_buckets+1 increasing entries from 0).  own_chunks[b] and
 * full_flats[b] (host arrays of n_buckets dev pointers) are bucket b's
 * own_chunk and full_flat; rank_chunks (host, n_buckets*N dev pointers)
 * holds bucket b's N chunk pointers at [b*N .. b*N+N), with
 * rank_chunks[b*N + rank] == own_chunks[b].  shard_flat: dev, the rank's
 * flat shard.  No written buffer may overlap any other buffer of the call.
 */
ZS3_API zs3_status zs3_gather_coalesced_buckets(zs3_layout_t layout, int32_t rank, int32_t dtype, int32_t n_buckets,
                                        const int32_t* bucket_start, const int64_t* ds_ids, const void* shard_flat,
                                        void* const* own_chunks, const void* const* rank_chunks,
                                        void* const* full_flats, void* stream);

/* ------------------------------------------ (3) local reduce-scatter
 * [codex] 6.2: the contiguous-gradient path all-reduces the bucket and each
 * rank keeps only its own interval, written into the one contiguous flat
 * gradient buffer; no full gradient is ever kept.  [csdn] core algorithm
 * step 3: the reduction sums and averages, each GPU keeps its part.
 *
 * For the n parameters ds_ids (host, any order, no duplicates; persistent
 * ones allowed: their "own slice" is the whole gradient), with
 * [lo_i, hi_i) the rank's own range of parameter i:
 *   grad_flat[shard_offset_i + k] =
 *       round16( (((0 + g_0[k]) + g_1[k]) + ... + g_{N-1}[k]) / N )
 * for k < hi_i - lo_i, with g_v = src[i*N + v] and every + and / one fp32
 * operation, round16 = round to nearest even into dtype; the remaining
 * positions k < partition_size_i (padding) are written as 0.
 * src: host array of n*N dev pointers; src[i*N + v] points at element lo_i
 * of virtual rank v's gradient of parameter i (it may be NULL when
 * hi_i == lo_i).  This serves whole per-rank gradient buckets as well as
 * slice-only storage.  grad_flat: dev, shard_numel elements.  The sources
 * must not overlap the written range of grad_flat.
 */
ZS3_API zs3_status zs3_reduce_scatter_local(zs3_layout_t layout, int32_t rank, int32_t dtype, int32_t n,
                                    const int64_t* ds_ids, const void* const* src, void* grad_flat,
                                    double* partials, void* stream);
/* partials: NULL, or the rank's norm slot array (dev, n_slots doubles from
 * zs3_layout_norm_slots).  When set, the same launch also writes, into the
 * slots that belong to the n parameters, sums of x*x over the 16-bit values
 * it writes (x widened exactly to double, sums in double), so that
 * zs3_grad_norm_partials can form the norm without reading grad_flat again
 * (the fusion of the norm's read into the reduce).  Each parameter owns a
 * fixed range of slots (partitioned parameters first, then persistent
 * ones), so calls for different buckets, on any streams, write disjoint
 * slots; a call rewrites every slot of its parameters.  partials must not
 * overlap grad_flat or the sources. */

/* Norm slots of a layout: n_slots doubles in all, the first n_part_slots
 * for partitioned parameters.  The same for every rank. */
ZS3_API zs3_status zs3_layout_norm_slots(zs3_layout_t layout, int64_t* n_slots, int64_t* n_part_slots);

/* ------------------------- (3b) non-contiguous path: reduce_scatter_coalesced
 * [codex] 6.2, second gradient path: without a contiguous bucket, the
 * gradients are reduce-scattered straight to their owners, and each owner's
 * averaged interval lands in the flat gradient buffer as on the contiguous
 * path.  Reading: the wire mirrors all_gather_coalesced ([codex] 5.2, 7):
 * parameters in ascending ds_id whatever the request order, c_j = prefix
 * sum of partition sizes, C = chunk_numel = sum of partition sizes.
 *
 * The bucket is the n parameters ds_ids (host, no duplicates, none
 * persistent: persistent gradients are whole on every rank and take
 * zs3_reduce_scatter_local, the all-reduce path).
 *   mode & ZS3_PACK (the rank's send side):
 *       send[d*C + c_j + k] = g_j[d*ps_j + k] when d*ps_j + k < numel_j,
 *                             else 0,
 *       for every destination rank d < N and k < ps_j.  grads: host array
 *       of n dev pointers, grads[i] = this rank's full flattened gradient
 *       of parameter ds_ids[i] (numel_i elements).  send: dev, N*C elements
 *       (the reduce-scatter's rank-major input: chunk d goes to rank d).
 *   mode & ZS3_REDUCE (the owner side, after the collective):
 *       grad_flat[shard_offset_j + k] =
 *           round16( (((0 + r_0[c_j+k]) + r_1[c_j+k]) + ... + r_{N-1}[c_j+k]) / N )
 *       for k < hi_j - lo_j (the rank's real elements), 0 for the padding
 *       positions k < ps_j whatever the chunks hold there; fp32 operations
 *       as in zs3_reduce_scatter_local, so both paths give the same bits.
 *       recv_chunks: host array of N dev pointers, recv_chunks[v] = the C
 *       elements rank v sent to this rank (chunk `rank` of v's send
 *       buffer).  grad_flat: dev, shard_numel elements.  partials: as in
 *       zs3_reduce_scatter_local (NULL: no sums).  Fastest when every
 *       recv_chunks[v] has the byte address of grad_flat + shard_offset of
 *       the bucket's first parameter modulo 16.
 * With both bits the pack runs first (recv_chunks[rank] may then point
 * into send).  Unused pointers may be NULL.  Outputs must not overlap the
 * inputs they are computed from.
 */
ZS3_API zs3_status zs3_reduce_scatter_coalesced(zs3_layout_t layout, int32_t rank, int32_t dtype, int32_t mode,
                                        int32_t n, const int64_t* ds_ids, const void* const* grads, void* send,
                                        const void* const* recv_chunks, void* grad_flat, double* partials,
                                        void* stream);

/* ------------------------------------------------ (4) global grad norm
 * [codex] 6.3: every sub-group is unscaled and clipped with the one global
 * norm.  [llmnex] pitfall 1: each card sees only its own part of the norm;
 * the partial sums must be combined so that every partition uses the same
 * coefficient.
 *
 * Partial step (always): sumsq[rank] = sum over the rank's real partitioned
 * gradient elements of x*x, sumsq[N] = the same over the persistent
 * gradients (identical on every rank, counted once); x is the element
 * widened exactly to double and the sums are in double.  grad_flat: dev,
 * shard_numel 16-bit elements.  sumsq: dev, N+1 doubles.
 * Finalize step (finalize != 0): total = sumsq[0] + ... + sumsq[N-1] (in
 * rank order) + sumsq[N]; *norm_out = sqrt(total); *nonfinite = total is
 * inf or NaN; coef = min(1, max_norm / (norm + 1e-6));
 * *scale_out = (float)(coef / loss_scale).  The caller supplies the other
 * ranks' sumsq entries (in a multi-GPU run they arrive by an all-reduce of
 * N+1 doubles).  norm_out (double), scale_out (float), nonfinite (int32)
 * are dev pointers; they may be NULL when finalize == 0.
 * Requires max_norm > 0 and loss_scale > 0.
 */
ZS3_API zs3_status zs3_grad_norm(zs3_layout_t layout, int32_t rank, int32_t dtype, const void* grad_flat,
                         double* sumsq, int32_t finalize, double max_norm, double loss_scale,
                         double* norm_out, float* scale_out, int32_t* nonfinite, void* stream);

/* The same partial and finalize steps from the norm slots that
 * zs3_reduce_scatter_local / zs3_reduce_scatter_coalesced filled (every
 * parameter of the layout must have been reduced with partials since its
 * slots were last meant to change): sumsq[rank] = sum of the partitioned
 * slots, sumsq[N] = sum of the persistent slots, both in a fixed order
 * (the result is reproducible, and equal to zs3_grad_norm's up to the
 * order of double additions).  partials: dev, n_slots doubles.  Other
 * arguments as in zs3_grad_norm. */
ZS3_API zs3_status zs3_grad_norm_partials(zs3_layout_t layout, int32_t rank, const double* partials,
                                  double* sumsq, int32_t finalize, double max_norm, double loss_scale,
                                  double* norm_out, float* scale_out, int32_t* nonfinite, void* stream);

/* For callers that cannot allocate device memory (work under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as zs3_grad_norm_partials, with the same arguments and the
 * same results bit for bit, that allocates nothing -- no hipMalloc, no
 * hipFree, no layout table.  Its only scratch (the slot pass's per-workgroup
 * sums, 16 KiB) is a static device array of the library: each GPU holds one
 * copy until the process ends, found on the call's first use of that GPU.
 * Every call on a GPU shares that copy, so calls that overlap on one GPU
 * (on different streams, or from several host threads) race and may return
 * wrong sums; serialise them.  Each call writes every scratch entry it
 * reads, so nothing needs clearing between calls.  Limit: layouts with more
 * than 1024 * 65536 norm slots (zs3_layout_norm_slots) get ZS3_EINVAL. */
ZS3_API zs3_status zs3_grad_norm_partials_noalloc(zs3_layout_t layout, int32_t rank, const double* partials,
                                          double* sumsq, int32_t finalize, double max_norm, double loss_scale,
                                          double* norm_out, float* scale_out, int32_t* nonfinite, void* stream);

/* ----------------------------------------- (5) fused Adam + 16-bit cast
 * [codex] 6.3: per sub-group, the rank's fp32 partition is stepped by the
 * real optimizer (it sees only this rank's shard) and the result is written
 * back into the 16-bit shard.  [llmnex] section 1: the optimizer state is an
 * fp32 master weight, momentum and variance per element.
 *
 * For every real (non-padding) position e of the rank's flat shard in
 * [begin, end), one IEEE fp32 operation per step, no contraction:
 *   g = float(grad_flat[e]) * (*scale)
 *   if wd != 0: w = w - (lr*wd) * w
 *   m = b1*m + (1-b1)*g ;  v = b2*v + (1-b2)*(g*g)
 *   den = sqrt(v / (1-b2^t)) + eps
 *   w = w - lr * ((m / (1-b1^t)) / den)
 *   shard_flat[e] = round16(w)
 * with w = master[e], m = exp_avg[e], v = exp_avg_sq[e] (Kingma & Ba's Adam
 * with bias correction; the pages name the state but print no formula).
 * Padding positions are not touched.  If nonfinite is not NULL and
 * *nonfinite != 0 the kernel writes nothing.
 * master, exp_avg, exp_avg_sq: dev fp32, grad_flat and shard_flat: dev
 * 16-bit, all the rank's whole flat arrays (shard_numel elements, indexed
 * from 0).  scale: dev float (from zs3_grad_norm).  hp: host.
 * 0 <= begin <= end <= shard_numel.  The five arrays must not overlap.
 */
ZS3_API zs3_status zs3_adam_step(zs3_layout_t layout, int32_t rank, int32_t dtype, int64_t begin, int64_t end,
                         float* master, float* exp_avg, float* exp_avg_sq, const void* grad_flat,
                         void* shard_flat, const float* scale, const int32_t* nonfinite,
                         const zs3_adam_params* hp, void* stream);

/* ------------------------------------------ (5a) fp32 master partition
 * [codex] 6.1: when the optimizer is built, each sub-group's fp32 partition
 * is created from the rank's 16-bit shard, and that fp32 master is what the
 * optimizer steps.  [llmnex] section 1: the optimizer state per element is
 * the fp32 master weight, the momentum and the variance; Adam starts both
 * moments at 0.
 *
 * For every position e in [begin, end) of the rank's flat shard:
 *   master[e] = shard_flat[e] widened exactly to float at real positions,
 *               0 at padding positions (whatever shard_flat holds there);
 *   exp_avg[e] = exp_avg_sq[e] = 0 (either pointer may be NULL: not written).
 * Positions outside [begin, end) are not touched.  shard_flat: dev 16-bit;
 * master, exp_avg, exp_avg_sq: dev fp32; all are the rank's whole flat
 * arrays (shard_numel elements, indexed from 0), only [begin, end) of them
 * is accessed.  0 <= begin <= end <= shard_numel.  The arrays must not
 * overlap.
 */
ZS3_API zs3_status zs3_init_master(zs3_layout_t layout, int32_t rank, int32_t dtype, int64_t begin, int64_t end,
                           const void* shard_flat, float* master, float* exp_avg, float* exp_avg_sq,
                           void* stream);

/* -------------------------------- (f4) Adam on optimizer state held on the host
 * [codex] 6.3: with the optimizer state offloaded, the per-sub-group step
 * first swaps the sub-group's state in (_prepare_sub_group), steps it, writes
 * the 16-bit shard, and swaps the state out again (_release_sub_group);
 * [codex] 6.1: the fp32 partitions then live in host memory.
 *
 * Same update as zs3_adam_step over [begin, end) (bit-identical results),
 * with master, exp_avg, exp_avg_sq in pinned host memory (host_*: whole
 * flat arrays of shard_numel floats, allocated with hipHostMalloc or an
 * equivalent pinned allocator that maps them for the device; other memory
 * is rejected).  Two ways to move the state:
 *   stage == NULL (direct): the kernel reads and writes the host arrays
 *       through their device mapping on `stream`: each element's state
 *       crosses the host link once in each direction, both directions at
 *       once, with no staging buffer, copy or event.
 *   stage != NULL (staged swap-in / swap-out): the range is streamed through
 *       `stage` (dev, stage_elems floats, 16-byte aligned): two slots of
 *       three arrays of chunk = floor((stage_elems/6 - 8)/8)*8 elements, so
 *       at least 96 floats.  Per chunk: host-to-device copies on
 *       copy_in_stream, the Adam kernel on `stream`, device-to-host copies
 *       on copy_out_stream, so the copies of neighbouring chunks overlap
 *       (either copy stream may be NULL: then `stream` carries it; copy
 *       streams that share a hardware queue, or run kernels too, may
 *       serialise the two directions).  The layout keeps the pipeline's
 *       events: staged steps on one layout must not overlap.
 * Ordering: the state is read after the work already on `stream`; when
 * `stream` reaches the point after the call, every element is back in host
 * memory.  The host must not touch the arrays meanwhile. */
ZS3_API zs3_status zs3_adam_step_offload(zs3_layout_t layout, int32_t rank, int32_t dtype, int64_t begin,
                                 int64_t end, float* host_master, float* host_exp_avg, float* host_exp_avg_sq,
                                 float* stage, int64_t stage_elems, const void* grad_flat, void* shard_flat,
                                 const float* scale, const int32_t* nonfinite, const zs3_adam_params* hp,
                                 void* stream, void* copy_in_stream, void* copy_out_stream);

/* ------------------------------------ (f2) trace-driven fetch/release plan
 * [codex] 5: a coordinator decides, module by module, which parameters to
 * all-gather and when to put them back in partitioned form.  Host only: no
 * device work; the gathers it returns are buckets for zs3_gather_coalesced.
 *
 * 5.1 trace.  Mode INVALID -> RECORD -> COMPLETE, advanced by
 * zs3_coord_reset_step at each end of step: the first step runs without a
 * trace, the second records the module order, and from the third on the
 * recorded order (as a parameter-level script) drives prefetching.  A fetch
 * that differs from the script drops the trace for the rest of the step
 * (mode INVALID, prefetching stops) and the next steps record it again
 * ([codex] section 7: dynamic graphs defeat prefetching).  A step that ends
 * with fewer or more fetches than the script counts as a mismatch too.
 * 5.2 fetch.  (i) The module's partitioned parameters that are not live are
 * gathered now (kind ZS3_GATHER_CURRENT); (ii) the caller waits for the
 * module's gathers; (iii) with a complete trace, the parameters that follow
 * in the script and are not live are popped into one more gather (kind
 * ZS3_GATHER_PREFETCH) until it holds prefetch_bucket_size elements (an
 * oversize parameter fills a bucket alone) or the next one would take the
 * live total past max_live_parameters; live parameters met on the way are
 * marked as needed at that later use.
 * 5.3 release.  A module's parameters go back to partitioned form unless the
 * prefetcher marked a later use, or (complete trace) a module within
 * max_reuse_distance elements further on uses them (the distance of a later
 * module = elements of the partitioned parameters of the modules strictly
 * between).  Persistent parameters are never gathered or released.
 * Readings: a parameter is live (counted against max_live_parameters) from
 * the issue of its gather to its release; every list is in ascending ds_id.
 */
typedef struct zs3_coord* zs3_coord_t;

typedef struct {
    int64_t prefetch_bucket_size;   /* elements per prefetch gather; 0 disables prefetching */
    int64_t max_live_parameters;    /* elements of gathered parameters that prefetching may not pass */
    int64_t max_reuse_distance;     /* elements */
} zs3_coord_config;

enum { ZS3_TRACE_INVALID = 0, ZS3_TRACE_RECORD = 1, ZS3_TRACE_COMPLETE = 2 };
enum { ZS3_PARAM_NOT_AVAILABLE = 0, ZS3_PARAM_INFLIGHT = 1, ZS3_PARAM_AVAILABLE = 2 };
enum { ZS3_GATHER_CURRENT = 0, ZS3_GATHER_PREFETCH = 1 };

/* Module m owns module_ds_ids[module_start[m] .. module_start[m+1]) (host;
 * module_start has n_modules+1 ascending entries from 0; ds_ids unique
 * within a module and in the layout; a parameter may belong to several
 * modules, e.g. tied weights).  The layout is read during the call only. */
ZS3_API zs3_status zs3_coord_create(zs3_layout_t layout, int32_t n_modules, const int32_t* module_start,
                            const int64_t* module_ds_ids, const zs3_coord_config* cfg, zs3_coord_t* out);
ZS3_API void zs3_coord_destroy(zs3_coord_t coord);

/* Fetch module m (before its forward or backward computation).  Outputs
 * (host): *n_gathers (0, 1 or 2) gathers, gather g being
 * ds_ids[starts[g] .. starts[g+1]) of kind kinds[g]; kinds needs 2 entries,
 * starts 3, ds_ids room for every parameter of the modules. */
ZS3_API zs3_status zs3_coord_fetch(zs3_coord_t coord, int32_t module, int32_t* n_gathers, int32_t* kinds,
                           int32_t* starts, int64_t* ds_ids);
/* Release module m (after its computation); m must have been fetched in
 * this step and not released since.  *n_released ds_ids (host) go back to
 * partitioned form. */
ZS3_API zs3_status zs3_coord_release(zs3_coord_t coord, int32_t module, int32_t* n_released, int64_t* ds_ids);
/* The pre-step pass ([codex] 6.3): every gathered parameter goes back to
 * partitioned form. */
ZS3_API zs3_status zs3_coord_release_all(zs3_coord_t coord, int32_t* n_released, int64_t* ds_ids);
/* End of step: the trace-mode transition of 5.1; *mode (may be NULL)
 * receives the new mode. */
ZS3_API zs3_status zs3_coord_reset_step(zs3_coord_t coord, int32_t* mode);
/* Current mode, live elements, recorded fetches, trace drops so far (any
 * output may be NULL). */
ZS3_API zs3_status zs3_coord_info(zs3_coord_t coord, int32_t* mode, int64_t* live_numel, int32_t* trace_len,
                          int32_t* invalidations);
ZS3_API zs3_status zs3_coord_param_status(zs3_coord_t coord, int64_t ds_id, int32_t* status);
/* What ranks must agree on once a trace is recorded ([codex] 5.1: module
 * order, parameter order, number of fetches): 64-bit FNV-1a over the
 * little-endian int64 module ids of the trace and over the ds_ids of the
 * parameter-level script, and the trace length.  Ranks compare them (for
 * example by an all-reduce of min and max); a difference would make their
 * collectives disagree. */
ZS3_API zs3_status zs3_coord_trace_signature(zs3_coord_t coord, uint64_t* module_order, uint64_t* param_order,
                                     int32_t* n_fetches);

#ifdef __cplusplus
}
#endif

#endif /* ZS3_H */
