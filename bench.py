"""Benchmark of the fused ZeRO-3 shard step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4] [--rank R]

A step is one pass of the whole hot path for one rank: forward and
backward coalesced all-gather of every gather bucket (pack + unpack), the
reduce-scatter of every gradient bucket, the global gradient norm, and the
fused Adam + cast of every sub-group (the pre-step pass that puts the
parameters back in partitioned form drops the gathered views and moves no
data).  The partition copy, which runs once per model, is timed on its own
after the steps and reported beside them.  The N
data-parallel ranks are N virtual ranks in this GPU's HBM; inputs are
synthetic (seeded N(0, 0.02) weights, N(0, 1e-3) gradients with 1% x100
outliers) and resident in HBM before timing starts.

Default launch configuration: gather buckets dealt over two streams,
gradient buckets over three streams, the slices each rank receives placed
per gradient bucket, the norm fused into the reduce, and one launch over
every bucket for a phase whose pass moves less than 4 GB (--single-launch
auto; none|gather|reduce|both choose by hand).
Variants: --reduce-path coalesced (the non-contiguous gradient path),
--schedule trace (gathers driven by the fetch/release coordinator over the
forward+backward module order), --offload 1 (the fp32 optimizer state in
pinned host memory), --fuse-norm 0, --rs-streams N.

Prints ONE JSON line: effective HBM GB/s of the step (its fixed algorithmic
byte budget / time: 2 x (pack + unpack) + reduce-scatter + norm + Adam,
the same for every variant, so a variant that fuses away a
pass shows as less time for the same work; the bytes each variant actually
has to move are reported beside it), its fraction of 8 TB/s and params/s,
the roofline entry of the dominant kernel (the fused gather) timed with HIP
events on the launch stream, and the CPU oracle timed on a bounded sample
of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "effective HBM GB/s (% of 8 TB/s) and params/s for fused ZeRO-3 shard step"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=12, help="decoder layers in the oracle's sample")
    ap.add_argument("--rs-streams", type=int, default=3, help="streams the gradient buckets are spread over")
    ap.add_argument("--gather-streams", type=int, default=2, help="streams the gather buckets are spread over")
    ap.add_argument("--kernel-timer", action="store_true",
                    help="with several gather streams, also time every gather launch of the timed steps")
    ap.add_argument("--fuse-norm", type=int, default=1, choices=(0, 1),
                    help="1: the reduce-scatter also writes the norm's partial sums (no second read of grad_flat)")
    ap.add_argument("--reduce-path", default="contiguous", choices=("contiguous", "coalesced"),
                    help="gradient path: all-reduced buckets (default) or reduce_scatter_coalesced")
    ap.add_argument("--offload", type=int, default=0, choices=(0, 1),
                    help="1: fp32 optimizer state in pinned host memory, streamed through the device per sub-group")
    ap.add_argument("--offload-chunk", type=int, default=0,
                    help="offloaded Adam: 0 reads the host state directly, else elements per staged chunk")
    ap.add_argument("--schedule", default="static", choices=("static", "trace"),
                    help="parameter gathers: static gather buckets twice (default), or the buckets the "
                         "trace-driven fetch/release coordinator returns over the forward+backward module order")
    ap.add_argument("--prefetch-bucket-size", type=float, default=None,
                    help="gather bucket limit in full elements (default: the workload's); larger than the "
                         "model puts every parameter in one bucket: one launch per gather pass")
    ap.add_argument("--reduce-bucket-size", type=float, default=None,
                    help="gradient bucket limit in full elements (default: the workload's); larger than the "
                         "model makes the gradient phase one launch")
    ap.add_argument("--recv-layout", default="bucket", choices=("rank", "bucket"),
                    help="where the slices the N ranks send this rank live: one shard-shaped copy per rank, or "
                         "per gradient bucket with its N slices next to each other")
    ap.add_argument("--single-launch", default="auto", choices=("auto", "none", "gather", "reduce", "both"),
                    help="gather: each gather pass one launch over every bucket (each bucket keeps its own wire and "
                         "gathered buffer); reduce: the gradient phase one launch over every bucket; both; auto "
                         "(default): one launch for a phase whose pass moves less than 4 GB")
    ap.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                    help="also run a plain device copy of this many GiB (counter calibration)")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace collapsed, so that a
    comment or layout edit does not count as a change of the kernels.
    (String literals are left alone; none of these files has // or /* in one.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """Digest of the code the kernels and their launch plans are built from."""
    h = hashlib.sha256()
    for f in ("kernels.hip", "api.cpp", "zs3_internal.hpp"):
        with open(os.path.join(ROOT, "zero_sharded_state_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_entry(config: str):
    """HBM bytes per gather launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"gather_traffic_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_digest") != source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


class KernelTimer:
    """Pre-created hipEvent_t pairs handed out one per timed launch; each
    launch records its own start and end timestamps into its pair."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")     # the runtime already loaded by torch and libzs3
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(a)) or self.hip.hipEventCreate(ctypes.byref(b)):
                raise RuntimeError("hipEventCreate failed")
            self.pairs.append((a.value, b.value))
        self.used = 0

    def __call__(self):
        p = self.pairs[self.used]
        self.used += 1
        return p

    def durations_ms(self):
        out = []
        ms = self.ct.c_float()
        for a, b in self.pairs[:self.used]:
            if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a), self.ct.c_void_p(b)):
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(self.ct.c_void_p(a))
            self.hip.hipEventDestroy(self.ct.c_void_p(b))


def with_bucket_sizes(cfg, prefetch=None, reduce=None):
    """The workload with its gather and/or gradient bucket limits replaced
    (None keeps the workload's)."""
    if prefetch is None and reduce is None:
        return cfg
    import dataclasses
    return dataclasses.replace(cfg, prefetch_bucket_size=int(prefetch or cfg.prefetch_bucket_size),
                               reduce_bucket_size=int(reduce or cfg.reduce_bucket_size))


# A pass of per-bucket launches pays a fixed cost per launch (ramp-up, drain,
# the kernel boundary); one launch over every bucket reads its work list from
# device memory instead of its arguments, a cost in proportion to the bytes.
# Measured crossover: passes of 0.3-1 GB run faster as one launch, passes of
# 15-36 GB as per-bucket launches over several streams.
SINGLE_LAUNCH_BELOW_BYTES = 4e9


def auto_single_launch(cfg, rank, reduce_path="contiguous", schedule="static"):
    """none / gather / reduce / both: one launch for each phase whose pass
    moves fewer algorithmic bytes than SINGLE_LAUNCH_BELOW_BYTES."""
    import zero_sharded_state_amd as zs
    h = zs.zs3_layout_create(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    try:
        own = {}
        for d in cfg.ds_ids:
            lo, hi = zs.zs3_layout_own_range(h, d, rank)
            own[d] = hi - lo
        # pack 4 B per own element + unpack 4 B per gathered element, per pass
        gather = sum(4 * own[d] + 4 * zs.zs3_layout_param(h, d)["numel"]
                     for b in zs.zs3_plan_buckets(h, zs.ZS3_GATHER_BUCKETS, cfg.prefetch_bucket_size) for d in b)
        reduce = (2 * cfg.world_size + 2) * sum(own.values())
    finally:
        zs.zs3_layout_destroy(h)
    g = schedule == "static" and gather < SINGLE_LAUNCH_BELOW_BYTES
    r = reduce_path == "contiguous" and reduce < SINGLE_LAUNCH_BELOW_BYTES
    return {(False, False): "none", (True, False): "gather", (False, True): "reduce", (True, True): "both"}[(g, r)]


def make_step(cfg, rank, rs_streams=1, gather_streams=1, fuse_norm=False, reduce_path="contiguous", offload=False,
              offload_chunk=0, recv_layout="rank", single_launch="none"):
    from zero_sharded_state_amd.shard_step import AdamConfig, ShardStep

    return ShardStep(world_size=cfg.world_size, rank=rank, threshold=cfg.threshold, ds_ids=cfg.ds_ids,
                     numels=cfg.numels, dtype=cfg.dtype, prefetch_bucket_size=cfg.prefetch_bucket_size,
                     reduce_bucket_size=cfg.reduce_bucket_size, sub_group_size=cfg.sub_group_size,
                     adam=AdamConfig(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay),
                     max_norm=cfg.max_norm, rs_streams=rs_streams, gather_streams=gather_streams,
                     fuse_norm=fuse_norm, reduce_path=reduce_path, offload=offload, offload_chunk=offload_chunk,
                     recv_layout=recv_layout, single_launch=single_launch)


def fill_inputs(step, cfg):
    from synth.gen import KIND_GRAD, KIND_WEIGHT, device_normal16

    dev = step.device
    if step.F:
        device_normal16(step.full.numel(), cfg.weight_std, cfg.dtype, dev, (cfg.seed, cfg.config_id, KIND_WEIGHT, 0),
                        out=step.full)
    if step.P:
        device_normal16(step.P, cfg.weight_std, cfg.dtype, dev, (cfg.seed, cfg.config_id, KIND_WEIGHT, 1),
                        out=step.pers_full)
    device_normal16(step.recv.numel(), cfg.grad_std, cfg.dtype, dev, (cfg.seed, cfg.config_id, KIND_GRAD, step.rank),
                    outlier_prob=cfg.outlier_prob, outlier_mult=cfg.outlier_mult, out=step.recv)
    if step.reduce_path == "coalesced":
        # the rank's own full gradients and the chunks its peers send it
        device_normal16(step.own_grads.numel(), cfg.grad_std, cfg.dtype, dev,
                        (cfg.seed, cfg.config_id, KIND_GRAD, 1000 + step.rank), outlier_prob=cfg.outlier_prob,
                        outlier_mult=cfg.outlier_mult, out=step.own_grads)
        device_normal16(step.xbuf.numel(), cfg.grad_std, cfg.dtype, dev,
                        (cfg.seed, cfg.config_id, KIND_GRAD, 2000 + step.rank), outlier_prob=cfg.outlier_prob,
                        outlier_mult=cfg.outlier_mult, out=step.xbuf)
    step.init_from_full()
    step.reduce_scatter()
    step.fill_peer_norms()


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# --------------------------------------------------------------------------

def cpu_baseline(step, cfg, layers: int):
    import numpy as np

    import oracle

    # the sample: the parameters of the first `layers` decoder layers (every
    # ds_id whose name carries a layer index < layers), same N, rank, dtype
    def layer_of(name):
        for tok in name.split("."):
            if tok.isdigit():
                return int(tok)
        return None

    ids = [d for d, p in enumerate(cfg.params) if layer_of(p.name) is not None and layer_of(p.name) < layers]
    if not ids:
        ids = list(range(min(4, len(cfg.params))))
    numels = [cfg.params[d].numel for d in ids]
    N, r, dt = step.N, step.rank, cfg.dtype
    L = oracle.make_layout(N, cfg.threshold, ids, numels)
    idset = set(ids)

    def h16(t):
        return t.cpu().numpy().view(np.uint16)

    full = {}
    for d in ids:
        p = step.by_id[d]
        if p["persistent"]:
            o = step.pers_off[d]
            full[d] = h16(step.pers_full[o:o + p["numel"]])
        else:
            o = step.full_off[d]
            full[d] = h16(step.full[o:o + p["numel"]])
    buckets = [b for b in step.gather_buckets if set(b) <= idset]
    chunks = {}
    for bi, b in enumerate(step.gather_buckets):
        if set(b) <= idset:
            _, _, w, c = step.bucket_meta[bi]
            chunks[tuple(b)] = [h16(step.wire[w + v * c:w + (v + 1) * c]) for v in range(N)]
    grads = []
    for v in range(N):
        g = {}
        for d in ids:
            p = step.by_id[d]
            lo, hi = p["own"]
            a = np.zeros(p["numel"], np.uint16)
            o = step.recv_index(v, d)
            a[lo:hi] = h16(step.recv[o:o + (hi - lo)])
            g[d] = a
        grads.append(g)
    shard = oracle.partition(L, r, full)
    master, m, v_ = oracle.init_state(shard, dt)
    grad_flat = np.zeros(L.shard_numel, np.uint16)
    hp = oracle.AdamHParams(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, 1)

    t = [time.perf_counter()]
    for _ in range(2):                                       # forward + backward all-gather
        for b in buckets:
            oracle.pack(L, r, b, shard)
            oracle.unpack(L, b, chunks[tuple(b)])
    t.append(time.perf_counter())
    oracle.reduce_scatter(L, r, dt, ids[::-1], grads, grad_flat)
    t.append(time.perf_counter())
    a, q = oracle.grad_norm_partial(L, r, dt, grad_flat)
    norm, coef, scale, bad = oracle.grad_norm_finalize([a] * N, q, cfg.max_norm)
    t.append(time.perf_counter())
    oracle.adam_step(L, r, dt, 0, L.shard_numel, master, m, v_, grad_flat, shard, scale, bad, hp)
    t.append(time.perf_counter())
    secs = t[-1] - t[0]

    part_real = sum(L.own_range(p, r)[1] - L.own_range(p, r)[0] for p in L.params if not p.persistent)
    own = sum(L.own_range(p, r)[1] - L.own_range(p, r)[0] for p in L.params)
    F = sum(sum(L.slot(d).numel for d in b) for b in buckets)
    phase_bytes = {"gather": 2 * 4 * part_real + 2 * 4 * F, "reduce_scatter": 2 * N * own + 2 * own,
                   "grad_norm": 2 * own, "adam": 28 * own}
    nbytes = sum(phase_bytes.values())
    kernels = {}
    for (name, b), t0, t1 in zip(phase_bytes.items(), t, t[1:]):
        kernels[name] = {"s": round(t1 - t0, 4), "GBps": round(b / (t1 - t0) / 1e9, 4) if t1 > t0 else None}
    return {
        "value": round(nbytes / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{layers} decoder layer(s) of the same workload ({len(ids)} params, {sum(numels):,} elements, "
                   f"{own:,} own elements of rank {r}), one whole step, numpy single-threaded; "
                   f"{nbytes / 1e9:.3f} GB algorithmic in {secs:.2f} s"),
        "params_per_s": round(own / secs, 1),
        "host_cores_available": len(os.sched_getaffinity(0)),
        "kernels": kernels,
    }


def coordinator_cost(step, cfg, steps: int = 5):
    """Host cost of the library's fetch/release coordinator on the
    workload's module order, per fetch or release call on a complete trace
    (through ctypes, preallocated arguments)."""
    import ctypes

    import zero_sharded_state_amd as zs
    from synth.modules import module_table, step_order

    _, mods = module_table(cfg)
    order = step_order(cfg)
    c = zs.zs3_coord_create(step.h, mods, {"prefetch_bucket_size": cfg.prefetch_bucket_size,
                                           "max_live_parameters": int(1e9), "max_reuse_distance": int(1e9)})
    lib = zs.lib()
    cap = sum(len(m) for m in mods)
    ids = (ctypes.c_int64 * cap)()
    kinds, starts, n = (ctypes.c_int32 * 2)(), (ctypes.c_int32 * 3)(), ctypes.c_int32()

    def native_step():
        for m in order:
            lib.zs3_coord_fetch(c, m, ctypes.byref(n), kinds, starts, ids)
            lib.zs3_coord_release(c, m, ctypes.byref(n), ids)
        lib.zs3_coord_release_all(c, ctypes.byref(n), ids)
        lib.zs3_coord_reset_step(c, None)

    for _ in range(2):
        native_step()
    t0 = time.perf_counter()
    for _ in range(steps):
        native_step()
    native = (time.perf_counter() - t0) / (steps * 2 * len(order)) * 1e6
    zs.zs3_coord_destroy(c)
    return {"calls_per_step": 2 * len(order), "us_per_call_library": round(native, 2),
            "note": "library timed through ctypes with preallocated arguments (includes the call overhead)"}


def cpu_baseline_coordinator(cfg):
    """CPU-baseline leg: the coordinator oracle on the same module order,
    per fetch or release call on a complete trace."""
    from oracle import coordinator as co
    from synth.modules import module_table, step_order

    _, mods = module_table(cfg)
    order = step_order(cfg)
    cc = co.CoordConfig(cfg.prefetch_bucket_size, int(1e9), int(1e9))
    o = co.Coordinator({d: p.numel for d, p in enumerate(cfg.params)},
                       {d: p.numel < cfg.threshold for d, p in enumerate(cfg.params)}, mods, cc)

    def oracle_step():
        for m in order:
            o.fetch(m)
            o.release(m)
        o.release_all()
        o.reset_step()

    for _ in range(2):
        oracle_step()
    t0 = time.perf_counter()
    oracle_step()
    return round((time.perf_counter() - t0) / (2 * len(order)) * 1e6, 2)


# --------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the N data-parallel ranks are virtual "
                                   "ranks in one GPU's HBM; --gpus must be 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch

    from synth import get_config

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    torch.cuda.set_device(0)
    cfg = with_bucket_sizes(get_config(args.config), args.prefetch_bucket_size, args.reduce_bucket_size)
    rank = cfg.bench_rank if args.rank is None else args.rank
    log(f"config {cfg.name}: {cfg.title}, rank {rank}")
    single = args.single_launch
    if single == "auto":
        single = auto_single_launch(cfg, rank, args.reduce_path, args.schedule)
    step = make_step(cfg, rank, args.rs_streams, args.gather_streams, bool(args.fuse_norm), args.reduce_path,
                     bool(args.offload), args.offload_chunk, args.recv_layout, single)
    log(f"layout: S+P={step.S:,} own real={step.own_real:,} F={step.F:,} gather buckets={len(step.gather_buckets)} "
        f"reduce buckets={len(step.reduce_buckets)} sub-groups={len(step.sub_groups)}")
    t0 = time.time()
    fill_inputs(step, cfg)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({torch.cuda.memory_allocated() / 2**30:.1f} GiB) in {time.time() - t0:.1f} s")

    trace = None
    if args.schedule == "trace":
        from synth.modules import module_table, step_order
        from zero_sharded_state_amd.trace_schedule import TraceGatherPass
        _, mods = module_table(cfg)
        trace = TraceGatherPass(step, mods, step_order(cfg),
                                {"prefetch_bucket_size": cfg.prefetch_bucket_size,
                                 "max_live_parameters": int(1e9), "max_reuse_distance": int(1e9)})
        t1 = time.time()
        trace.plan()
        trace.fill_peer_chunks()
        torch.cuda.synchronize()
        log(f"coordinator: {len(trace.ops)} gathers per step ({trace.kinds.count(1)} prefetch), "
            f"{trace.gathered:,} elements gathered, set up in {time.time() - t1:.1f} s")

    for _ in range(args.warmup):
        step.step(trace_pass=trace)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    phase_events = []
    stream = torch.cuda.current_stream()

    def on_phase(name):
        e = ev()
        e.record(stream)
        phase_events[-1].append((name, e))

    # With --kernel-timer and several gather streams every gather launch of
    # the timed steps records its own start/end (a few us per launch).
    per_pass = 1 if step.single_gather else len(step.gather_buckets)
    overlapped = step.gather_streams > 1 and not step.single_gather
    per_launch = overlapped and args.kernel_timer and trace is None
    timer = KernelTimer(2 * per_pass * args.steps if per_launch else 0)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        phase_events.append([])
        step.step(on_phase=on_phase, gather_timer=timer if per_launch else None, trace_pass=trace)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall:.3f} s")

    ms_per_step = wall * 1e3 / args.steps
    nbytes = step.algorithmic_bytes()          # what this variant of the step must move, per kernel
    if trace is not None:
        del nbytes["pack"], nbytes["unpack"]
        nbytes["gather_trace"] = trace.algorithmic_bytes()
    total_bytes = step.budget_bytes()          # the step's fixed budget (equal work for every variant)
    moved_bytes = sum(nbytes.values())
    gbs = total_bytes / (ms_per_step * 1e-3) / 1e9
    params_per_s = step.own_real / (ms_per_step * 1e-3)

    # per-phase times (HIP events on the launch stream)
    phases = {}
    for evs in phase_events:
        for (name, e0), (_, e1) in zip(evs, evs[1:]):
            phases[name] = phases.get(name, 0.0) + e0.elapsed_time(e1)
    phase_bytes = {"gather_fwd": (nbytes.get("pack", 0) + nbytes.get("unpack", 0)) // 2,
                   "gather_bwd": (nbytes.get("pack", 0) + nbytes.get("unpack", 0)) // 2,
                   "gather_trace": nbytes.get("gather_trace", 0),
                   "reduce_scatter": nbytes["reduce_scatter"] + nbytes.get("scatter_pack", 0),
                   "grad_norm": nbytes["grad_norm"], "adam": nbytes["adam"]}
    per_step = sorted(evs[0][1].elapsed_time(evs[-1][1]) for evs in phase_events)
    step_stats = {"min": round(per_step[0], 4), "median": round(per_step[len(per_step) // 2], 4),
                  "max": round(per_step[-1], 4)}
    kernels = {}
    for name, ms in phases.items():
        ms /= args.steps
        kernels[name] = {"ms": round(ms, 4), "bytes": phase_bytes[name],
                         "GBps": round(phase_bytes[name] / (ms * 1e-3) / 1e9, 1) if phase_bytes[name] else None,
                         "hbm_frac": (round(phase_bytes[name] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                      if phase_bytes[name] else None),
                         "params_per_s": round(step.own_real / (ms * 1e-3), 1) if ms > 0 else None}

    # Roofline entry of the dominant kernel: the fused gather (pack + unpack
    # of one bucket, k_copy<4>), bytes per launch over the average launch
    # duration.  When the step runs its gather launches back to back on one
    # stream, that is the gather phases' event time on the launch stream over
    # the launch count (it matches rocprofv3's average).  When the step deals
    # them over several streams, launches overlap in pairs and each lasts
    # about twice as long while sharing the chip, so the kernel's own
    # duration is taken from gather passes run on the launch stream alone
    # right after the timed steps (the same launches on the same buffers).
    gather_bytes = nbytes["gather_trace"] if trace is not None else nbytes["pack"] + nbytes["unpack"]
    gather_phase_ms = sum(phases.get(k, 0.0) for k in ("gather_fwd", "gather_bwd", "gather_trace"))
    if overlapped:
        # forward + backward passes of the static buckets, or whole steps of
        # the coordinator's gathers, on the launch stream alone
        cal_passes = 2 * min(args.steps, 5) if trace is None else min(args.steps, 5)
        per_cal = per_pass if trace is None else len(trace.ops)
        one_pass = (lambda: step.gather_pass(streams=1)) if trace is None else (lambda: trace.run(streams=1))
        one_pass()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(cal_passes):
            one_pass()
        e1.record(stream)
        torch.cuda.synchronize()
        launches = cal_passes * per_cal
        avg_ms = e0.elapsed_time(e1) / launches
        per_launch_bytes = gather_bytes / (2 * per_pass if trace is None else per_cal)
        what = "gather passes" if trace is None else "steps of the coordinator's gathers"
        measured = (f"{cal_passes} {what} on the launch stream alone, right after the timed steps "
                    f"(the step deals its gathers over {step.gather_streams} streams)")
    else:
        launches = (len(trace.ops) if trace is not None else 2 * per_pass) * args.steps
        avg_ms = gather_phase_ms / launches
        per_launch_bytes = gather_bytes * args.steps / launches
        measured = "the timed steps' gather phases on the launch stream"
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9
    unit = "every bucket of a pass" if step.single_gather else "one bucket"
    roofline = {"kernel": f"gather: pack + unpack of {unit} (k_copy_inline<4>, or k_copy<4> for > 40 segments)",
                "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_entry(cfg.name) if trace is None else None,
                "launches": launches, "avg_launch_ms": round(avg_ms, 5),
                "algorithmic_bytes_per_launch": int(per_launch_bytes),
                "measured_on": measured,
                "step_gather": {"streams": step.gather_streams,
                                "GBps": round(gather_bytes * args.steps / (gather_phase_ms * 1e-3) / 1e9, 1)}}
    if per_launch:
        durs = timer.durations_ms()
        roofline["step_gather"]["avg_launch_ms_overlapped"] = round(sum(durs) / len(durs), 5)
    timer.close()

    # The partition copy (construction-time, not part of the step): every
    # full parameter's own range into a scratch shard, timed on its own.
    part = torch.empty_like(step.shard)
    step.repartition(dst=part)
    reps = []
    for _ in range(5):
        e0, e1 = ev(), ev()
        e0.record(stream)
        step.repartition(dst=part)
        e1.record(stream)
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1))
    del part
    pms = sorted(reps)[len(reps) // 2]
    pbytes = step.partition_bytes()
    kernels["partition_once"] = {"ms": round(pms, 4), "bytes": pbytes,
                                 "GBps": round(pbytes / (pms * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(pbytes / (pms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "note": "once per model, outside the step: median of 5 calls"}

    if args.calibrate_copy_gib > 0:
        # a plain device copy three times with torch (the runtime's copy
        # kernel), then three times through the library's copy path (a
        # one-parameter, one-rank partition: k_copy_inline<1>)
        import zero_sharded_state_amd as zs
        n = int(args.calibrate_copy_gib * 2**30) // 2
        a = torch.empty(n, dtype=torch.int16, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        hc = zs.zs3_layout_create(1, 0, [0], [n])
        for _ in range(3):
            zs.zs3_partition(hc, 0, cfg.dtype, [0], [a], b)
        torch.cuda.synchronize()
        zs.zs3_layout_destroy(hc)
        del a, b

    coord = None
    if trace is not None:
        coord = coordinator_cost(step, cfg)
    offload = None
    if step.offload:
        link = 24 * step.own_real            # fp32 master, momentum, variance: in and out once per step
        ms = kernels["adam"]["ms"]
        offload = {"link_bytes_per_step": link, "adam_ms": ms, "link_GBps": round(link / (ms * 1e-3) / 1e9, 1),
                   "mode": "staged chunks of %d elements" % args.offload_chunk if args.offload_chunk else "direct",
                   "note": "Adam phase with the fp32 state in pinned host memory, in and out over the host link"}

    cpu = None
    if not args.no_cpu_baseline:
        log("running the CPU oracle on its sample")
        cpu = cpu_baseline(step, cfg, args.cpu_layers)
        if trace is not None:
            cpu["coordinator_us_per_call"] = cpu_baseline_coordinator(cfg)

    line = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_events": step_stats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "params_per_s": round(params_per_s, 1),
        "bytes_per_step": total_bytes,
        "bytes_moved_per_step": moved_bytes,
        "config": {
            "workload": f"{cfg.title}: fused shard step of rank {rank} ({cfg.total_params:,} params, "
                        f"{step.own_real:,} own elements)",
            "name": cfg.name, "world_size": cfg.world_size, "rank": rank, "storage_dtype": cfg.dtype,
            "params": cfg.total_params, "own_elements": step.own_real,
            "gather_buckets": len(step.gather_buckets), "reduce_buckets": len(step.reduce_buckets),
            "sub_groups": len(step.sub_groups), "prefetch_bucket_size": cfg.prefetch_bucket_size,
            "reduce_bucket_size": cfg.reduce_bucket_size, "sub_group_size": cfg.sub_group_size,
            "reduce_path": step.reduce_path, "fused_norm": step.fuse_norm, "rs_streams": step.rs_streams,
            "schedule": args.schedule, "offload": step.offload,
            "gather_streams": step.gather_streams, "recv_layout": step.recv_layout,
            "single_launch": step.single_launch,
            "single_launch_flag": args.single_launch,
        },
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "coordinator": coord,
        "offload": offload,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)
    step.destroy()


if __name__ == "__main__":
    main()
