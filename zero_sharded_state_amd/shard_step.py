"""One rank's ZeRO-3 shard step, with the N data-parallel ranks held as N
virtual ranks in one GPU's HBM.

The step issues the calls a real rank makes around its collectives, in the
order the pages give ([llmnex] section 2, [codex] 5.2, 6.2, 6.3), on one
stream (the gradient buckets, whose outputs are disjoint, may be dealt over
a few streams that fork from it and join back):

1. forward all-gather of every gather bucket: pack the own shard into the
   rank's chunk of the bucket's wire buffer, then unpack the N chunks into
   the bucket's full parameters (the other chunks stand for what the
   collective delivers);
2. backward all-gather: the same again (parameters were released after the
   forward);
3. reduce-scatter of every gradient bucket (backward order) into the flat
   gradient buffer.  Contiguous path ([codex] 6.2, the default): from the
   slices the N ranks' all-reduced buckets hold for this rank.
   Non-contiguous path (reduce_scatter_coalesced): the rank packs its own
   full gradients into N rank-major chunks, and reduces the N chunks
   addressed to it (its own plus N-1 stand-ins for what the peers send);
   persistent gradients take the all-reduce path either way.  With
   ``fuse_norm`` the reduce also writes the norm's partial sums of squares;
4. the pre-step pass that puts every parameter back in partitioned form
   ([codex] 6.3): the gathered views are dropped.  The flat shard already
   holds every parameter's own range, so no data moves (the partition copy
   itself, ``repartition``, runs once at set-up);
5. the global gradient norm and clip scale ([llmnex] pitfall 1), from
   grad_flat or, with ``fuse_norm``, from the reduce's partial sums;
6. fused Adam + cast per sub-group, on the fp32 state in HBM or, with
   ``offload``, in pinned host memory ([codex] 6.1, 6.3).  Adam is the
   only writer of the shard, so the shard is always the 16-bit rounding of
   the fp32 master.

No call synchronises; nothing is copied to the host.  All buffers are torch
tensors owned by this object; all arithmetic runs in libzs3's kernels.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

import zero_sharded_state_amd as zs


@dataclass
class AdamConfig:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


class ShardStep:
    def __init__(self, *, world_size: int, rank: int, threshold: int, ds_ids: Sequence[int],
                 numels: Sequence[int], dtype: str, prefetch_bucket_size: int, reduce_bucket_size: int,
                 sub_group_size: int, adam: AdamConfig = AdamConfig(), max_norm: float = 1.0,
                 device: str = "cuda", rs_streams: int = 1, gather_streams: int = 1,
                 fuse_norm: bool = False, reduce_path: str = "contiguous", offload: bool = False,
                 offload_chunk: int = 0, recv_layout: str = "rank", single_launch="none"):
        import torch

        if reduce_path not in ("contiguous", "coalesced"):
            raise ValueError(f"reduce_path {reduce_path!r} is not 'contiguous' or 'coalesced'")
        if recv_layout not in ("rank", "bucket"):
            raise ValueError(f"recv_layout {recv_layout!r} is not 'rank' or 'bucket'")
        self.recv_layout = recv_layout
        # single_launch "gather": each gather pass is one launch over every
        # bucket (each bucket keeps its own wire and gathered buffer);
        # "reduce": the gradient phase is one launch over every bucket's
        # parameters; "both", or "none" (one launch per bucket).  The
        # results are those of the per-bucket calls, bit for bit.
        if single_launch is True or single_launch is False:
            single_launch = "both" if single_launch else "none"
        if single_launch not in ("none", "gather", "reduce", "both"):
            raise ValueError(f"single_launch {single_launch!r} is not none, gather, reduce or both")
        self.single_gather = single_launch in ("gather", "both")
        self.single_reduce = single_launch in ("reduce", "both")
        if self.single_reduce and reduce_path != "contiguous":
            raise ValueError("a single-launch gradient phase needs the contiguous gradient path")
        self.single_launch = single_launch
        self.fuse_norm = bool(fuse_norm)
        self.reduce_path = reduce_path

        self.torch = torch
        self.N, self.rank, self.dtype = int(world_size), int(rank), dtype
        self.dcode = zs.DTYPES[dtype]
        self.adam, self.max_norm = adam, float(max_norm)
        self.device = torch.device(device)
        self.h = zs.zs3_layout_create(world_size, threshold, ds_ids, numels)
        info = zs.zs3_layout_info(self.h)
        self.S = info["shard_numel"]
        self.params = [zs.zs3_layout_param_at(self.h, i) for i in range(info["n_params"])]
        self.by_id = {p["ds_id"]: p for p in self.params}
        for p in self.params:
            p["own"] = zs.zs3_layout_own_range(self.h, p["ds_id"], self.rank)
        self.gather_buckets = zs.zs3_plan_buckets(self.h, zs.ZS3_GATHER_BUCKETS, prefetch_bucket_size)
        self.reduce_buckets = zs.zs3_plan_buckets(self.h, zs.ZS3_REDUCE_BUCKETS, reduce_bucket_size)
        self.sub_groups = zs.zs3_sub_groups(self.h, sub_group_size)

        # ---- buffer layout (element offsets) ----
        # Every bucket's gathered buffer and its all-gather buffer start on a
        # 16-byte boundary.  A one-parameter bucket's N chunks then sit at the
        # same byte address modulo 16 as the parts of the parameter they fill
        # (chunk v at v*partition_size in both), so its unpack is one
        # co-aligned 128-bit copy even when the sizes are ragged.
        self.full_off: Dict[int, int] = {}     # ds_id -> offset of its gathered view in `full`
        self.bucket_meta: List[Tuple[int, int, int, int]] = []   # (full_off, full_n, wire_off, chunk_n)
        f = w = 0
        self.F = 0                              # gathered elements (the real ones: sum of numels)
        for b in self.gather_buckets:
            chunk_n, full_n = zs.zs3_bucket_sizes(self.h, b)
            f, w = -(-f // 8) * 8, -(-w // 8) * 8
            self.bucket_meta.append((f, full_n, w, chunk_n))
            o = f
            for d in b:                         # ds_id order inside a bucket
                self.full_off[d] = o
                o += self.by_id[d]["numel"]
            f += full_n
            w += self.N * chunk_n
            self.F += full_n
        self.full_len, self.W = f, w
        self.pers = [p for p in self.params if p["persistent"]]
        self.pers_off = {}
        o = 0
        for p in self.pers:
            self.pers_off[p["ds_id"]] = o
            o += p["numel"]
        self.P = o
        self.own_real = sum(p["own"][1] - p["own"][0] for p in self.params)     # S_real + P

        i16, f32 = torch.int16, torch.float32
        dev = self.device
        self.full = torch.empty(max(1, self.full_len), dtype=i16, device=dev)  # gathered parameters
        self.pers_full = torch.empty(max(1, self.P), dtype=i16, device=dev)   # whole persistent params
        self.wire = torch.empty(max(1, self.W), dtype=i16, device=dev)        # per-bucket all-gather output
        self.shard = torch.zeros(max(1, self.S), dtype=i16, device=dev)
        self.grad = torch.zeros(max(1, self.S), dtype=i16, device=dev)
        # The slices the N ranks send this rank.  "rank": one copy of the
        # flat shard's layout per rank, at a stride rounded up to 8 elements.
        # "bucket": per gradient bucket, its N slices next to each other
        # (what an all-to-all of the bucket delivers), so the sources of one
        # element lie within one bucket's region.  Either way every source
        # of an element has the byte address of its grad_flat destination
        # modulo 16 (the reduce-scatter's co-aligned 128-bit path).
        self.recv_stride = (self.S + 7) // 8 * 8
        self._recv_region: Dict[int, Tuple[int, int, int]] = {}    # ds_id -> (base, stride, lo) of its bucket
        if recv_layout == "rank":
            recv_len = self.N * self.recv_stride
        else:
            cur = 0
            for b in self.reduce_buckets:
                lo = min(self.by_id[d]["shard_offset"] for d in b)
                hi = max(self.by_id[d]["shard_offset"] + self.by_id[d]["partition_size"] for d in b)
                stride = (hi - lo + 7) // 8 * 8
                base = cur + (lo - cur) % 8               # base = lo (mod 8): co-aligned with grad_flat
                for d in b:
                    self._recv_region[d] = (base, stride, lo)
                cur = base + self.N * stride
            recv_len = cur
        self.recv = torch.zeros(max(1, recv_len), dtype=i16, device=dev)
        # the fp32 optimizer partition (master, momentum, variance) is one
        # allocation, each array starting on a 2 MiB boundary; offloaded, it
        # lives in pinned host memory ([codex] 6.1, 6.3)
        sa = (max(1, self.S) + (1 << 19) - 1) >> 19 << 19
        self.offload = bool(offload)
        if self.offload:
            # offload_chunk 0: Adam reads and writes the host state directly;
            # otherwise chunks of that many elements are staged through HBM
            self.state = torch.zeros(3 * sa, dtype=f32, pin_memory=True)
            self.stage_elems = 6 * (int(offload_chunk) + 8) if offload_chunk else 0
            self.stage = torch.empty(self.stage_elems, dtype=f32, device=dev) if offload_chunk else None
        else:
            self.state = torch.zeros(3 * sa, dtype=f32, device=dev)
        self.master = self.state[0:max(1, self.S)]
        self.exp_avg = self.state[sa:sa + max(1, self.S)]
        self.exp_avg_sq = self.state[2 * sa:2 * sa + max(1, self.S)]
        self.sumsq = torch.zeros(self.N + 1, dtype=torch.float64, device=dev)
        self.n_slots, _ = zs.zs3_layout_norm_slots(self.h)
        self.partials = torch.zeros(max(1, self.n_slots), dtype=torch.float64, device=dev)
        if reduce_path == "coalesced":
            self._coalesced_buffers()
        self.outs = torch.zeros(2, dtype=torch.float64, device=dev)   # norm | scale (f32), flag (i32)
        self.t = 0
        # independent gradient buckets are spread over a few streams so that
        # short reduce-scatter kernels overlap (default priority streams)
        # (the offloaded Adam's swap-in and swap-out copies use two of them:
        # a process has few hardware queues, and streams that share one
        # serialise, so no stream is created just for the copies)
        n_aux = max(0, max(rs_streams, gather_streams, 3 if self.offload and offload_chunk else 0) - 1)
        self.aux_streams = [torch.cuda.Stream(device=dev) for _ in range(n_aux)]
        if self.offload:
            self.copy_streams = self.aux_streams[:2]
        self.rs_streams = max(1, rs_streams)
        self.gather_streams = max(1, gather_streams)
        self._fork = torch.cuda.Event()
        self._joins = [torch.cuda.Event() for _ in self.aux_streams]
        self._marshal()

    # ------------------------------------------------------------ pointers
    def full_param_ptr(self, ds_id: int) -> int:
        p = self.by_id[ds_id]
        if p["persistent"]:
            return self.pers_full.data_ptr() + 2 * self.pers_off[ds_id]
        return self.full.data_ptr() + 2 * self.full_off[ds_id]

    def chunk_ptr(self, bucket: int, v: int) -> int:
        _, _, w, c = self.bucket_meta[bucket]
        return self.wire.data_ptr() + 2 * (w + v * c)

    def recv_index(self, v: int, ds_id: int) -> int:
        """Element offset in ``recv`` of virtual rank v's slice of parameter
        ds_id for this rank."""
        off = self.by_id[ds_id]["shard_offset"]
        if self.recv_layout == "rank":
            return v * self.recv_stride + off
        base, stride, lo = self._recv_region[ds_id]
        return base + v * stride + (off - lo)

    def recv_ptr(self, v: int, ds_id: int) -> int:
        """Where virtual rank v's slice of parameter ds_id for this rank lives."""
        return self.recv.data_ptr() + 2 * self.recv_index(v, ds_id)

    def _coalesced_buffers(self):
        """Own full gradients, per-bucket send buffers and received chunks.
        Every chunk the reduce reads starts at the byte address of its
        bucket's first grad_flat position modulo 16, so the reduce runs
        co-aligned."""
        torch = self.torch
        part = [p for p in self.params if not p["persistent"]]
        self.grad_off: Dict[int, int] = {}
        o = 0
        for p in part:
            self.grad_off[p["ds_id"]] = o
            o = (o + p["numel"] + 7) // 8 * 8
        self.own_grads = torch.zeros(max(1, o), dtype=torch.int16, device=self.device)
        gp = self.grad.data_ptr()
        buckets = []          # (ids_part, ids_pers, C, send_off, {v: chunk_off})
        cursor = 0

        def place(n, residue):              # element offset with (2*off) % 16 == residue
            nonlocal cursor
            off = cursor + ((residue // 2 - cursor) % 8)
            cursor = off + n
            return off

        for b in self.reduce_buckets:
            ids_part = sorted(d for d in b if not self.by_id[d]["persistent"])
            ids_pers = [d for d in b if self.by_id[d]["persistent"]]
            C = sum(self.by_id[d]["partition_size"] for d in ids_part)
            if not ids_part:
                buckets.append((ids_part, ids_pers, 0, 0, {}))
                continue
            res = (gp + 2 * self.by_id[ids_part[0]]["shard_offset"]) % 16
            send = place(self.N * C, (res - 2 * self.rank * C) % 16)
            chunks = {v: place(C, res) for v in range(self.N) if v != self.rank}
            buckets.append((ids_part, ids_pers, C, send, chunks))
        self.xbuf = torch.zeros(max(1, cursor), dtype=torch.int16, device=self.device)
        self.coalesced = buckets

    def grad_ptr(self, ds_id: int) -> int:
        """This rank's full gradient of a partitioned parameter (non-contiguous path)."""
        return self.own_grads.data_ptr() + 2 * self.grad_off[ds_id]

    def recv_chunk_ptr(self, bucket: int, v: int) -> int:
        """The chunk virtual rank v sends to this rank for a gradient bucket."""
        _, _, C, send, chunks = self.coalesced[bucket]
        if v == self.rank:
            return self.xbuf.data_ptr() + 2 * (send + v * C)
        return self.xbuf.data_ptr() + 2 * chunks[v]

    def send_ptr(self, bucket: int) -> int:
        return self.xbuf.data_ptr() + 2 * self.coalesced[bucket][3]

    @property
    def norm_ptr(self) -> int:
        return self.outs.data_ptr()

    @property
    def scale_ptr(self) -> int:
        return self.outs.data_ptr() + 8

    @property
    def flag_ptr(self) -> int:
        return self.outs.data_ptr() + 12

    def _marshal(self):
        """Pre-build the ctypes arguments of every call of the step."""
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        self._g = []
        for bi, b in enumerate(self.gather_buckets):
            ids = (I64 * len(b))(*b)
            chunks = (P * self.N)(*[self.chunk_ptr(bi, v) for v in range(self.N)])
            fo = self.bucket_meta[bi][0]
            self._g.append((len(b), ids, self.chunk_ptr(bi, self.rank), chunks,
                            self.full.data_ptr() + 2 * fo))
        self._r = []
        self._x = []
        for bi, b in enumerate(self.reduce_buckets):
            if self.reduce_path == "coalesced":
                ids_part, ids_pers, C, _, _ = self.coalesced[bi]
                b = ids_pers
                if ids_part:
                    self._x.append((len(ids_part), (I64 * len(ids_part))(*ids_part),
                                    (P * len(ids_part))(*[self.grad_ptr(d) for d in ids_part]),
                                    self.send_ptr(bi),
                                    (P * self.N)(*[self.recv_chunk_ptr(bi, v) for v in range(self.N)])))
                if not b:
                    continue
            ids = (I64 * len(b))(*b)
            src = (P * (len(b) * self.N))(*[self.recv_ptr(v, d) for d in b for v in range(self.N)])
            self._r.append((len(b), ids, src))
        all_ids = [p["ds_id"] for p in self.params]
        self._p = (len(all_ids), (I64 * len(all_ids))(*all_ids),
                   (P * len(all_ids))(*[self.full_param_ptr(d) for d in all_ids]))
        if self.single_gather:
            nb = len(self.gather_buckets)
            starts, flat = [0], []
            for b in self.gather_buckets:
                flat += b
                starts.append(len(flat))
            self._gm = (nb, (ctypes.c_int32 * (nb + 1))(*starts), (I64 * max(1, len(flat)))(*flat),
                        (P * max(1, nb))(*[self._g[bi][2] for bi in range(nb)]),
                        (P * max(1, nb * self.N))(*[self.chunk_ptr(bi, v) for bi in range(nb) for v in range(self.N)]),
                        (P * max(1, nb))(*[self._g[bi][4] for bi in range(nb)]))
        if self.single_reduce:
            rs_ids = [d for b in self.reduce_buckets for d in b]
            self._rm = (len(rs_ids), (I64 * len(rs_ids))(*rs_ids),
                        (P * (len(rs_ids) * self.N))(*[self.recv_ptr(v, d) for d in rs_ids for v in range(self.N)]))

    # ------------------------------------------------------------- phases
    def _stream(self) -> int:
        return int(self.torch.cuda.current_stream().cuda_stream)

    def _ok(self, st):
        if st != 0:
            raise zs.Zs3Error(st, zs.zs3_last_error())

    def gather(self, bi: int, stream=None):
        """Pack + unpack of one bucket (one launch: the wire's own slot is the pack output)."""
        n, ids, own, chunks, fullp = self._g[bi]
        self._ok(zs.lib().zs3_gather_coalesced(self.h, self.rank, self.dcode, zs.ZS3_PACK | zs.ZS3_UNPACK, n, ids,
                                               self.shard.data_ptr(), own, chunks, fullp, None,
                                               stream if stream is not None else self._stream()))

    def pack(self, bi: int, stream=None):
        n, ids, own, chunks, fullp = self._g[bi]
        self._ok(zs.lib().zs3_gather_coalesced(self.h, self.rank, self.dcode, zs.ZS3_PACK, n, ids,
                                               self.shard.data_ptr(), own, None, None, None,
                                               stream if stream is not None else self._stream()))

    def unpack(self, bi: int, stream=None):
        n, ids, own, chunks, fullp = self._g[bi]
        self._ok(zs.lib().zs3_gather_coalesced(self.h, self.rank, self.dcode, zs.ZS3_UNPACK, n, ids, None, None,
                                               chunks, fullp, None,
                                               stream if stream is not None else self._stream()))

    def _fanout(self, stream, k):
        """The main stream plus k-1 auxiliary streams that wait for it."""
        torch = self.torch
        main = torch.cuda.current_stream() if stream is None else stream
        aux = self.aux_streams[:k - 1]
        if aux:
            self._fork.record(main)
            for a in aux:
                a.wait_event(self._fork)
        return main, aux, [int(main.cuda_stream)] + [int(a.cuda_stream) for a in aux]

    def _join(self, main, aux):
        for a, e in zip(aux, self._joins):
            e.record(a)
            main.wait_event(e)

    def gather_pass(self, stream=None, timer=None, streams=None):
        """Every gather bucket; buckets are independent, so with several
        gather streams they are dealt round-robin and joined at the end
        (``streams`` overrides the step's count for this pass).
        ``timer()``, if given, returns a (start, stop) hipEvent_t pair that
        the bucket's kernel records its own start and end into."""
        lib = zs.lib()
        if self.single_gather:
            nb, starts, ids, owns, chunks, fulls = self._gm
            if timer is not None:
                lib.zs3_time_next_launch(*timer())
            self._ok(lib.zs3_gather_coalesced_buckets(self.h, self.rank, self.dcode, nb, starts, ids,
                                                      self.shard.data_ptr(), owns, chunks, fulls,
                                                      stream if stream is not None else self._stream()))
            return
        main, aux, handles = self._fanout(stream, self.gather_streams if streams is None else streams)
        for bi in range(len(self._g)):
            if timer is not None:
                lib.zs3_time_next_launch(*timer())
            self.gather(bi, handles[bi % len(handles)])
        self._join(main, aux)

    def reduce_scatter(self, stream=None):
        """Every gradient bucket, fanned out over the main and auxiliary
        streams and joined back into the main stream."""
        lib = zs.lib()
        partials = self.partials.data_ptr() if self.fuse_norm else None
        if self.single_reduce:
            n, ids, src = self._rm
            self._ok(lib.zs3_reduce_scatter_local(self.h, self.rank, self.dcode, n, ids, src, self.grad.data_ptr(),
                                                  partials, stream if stream is not None else self._stream()))
            return
        main, aux, handles = self._fanout(stream, self.rs_streams)
        for i, (n, ids, grads, send, recv) in enumerate(self._x):
            self._ok(lib.zs3_reduce_scatter_coalesced(self.h, self.rank, self.dcode, zs.ZS3_PACK | zs.ZS3_REDUCE,
                                                      n, ids, grads, send, recv, self.grad.data_ptr(), partials,
                                                      handles[i % len(handles)]))
        for i, (n, ids, src) in enumerate(self._r, start=len(self._x)):
            self._ok(lib.zs3_reduce_scatter_local(self.h, self.rank, self.dcode, n, ids, src,
                                                  self.grad.data_ptr(), partials, handles[i % len(handles)]))
        self._join(main, aux)

    def repartition(self, stream=None, dst=None):
        """The partition copy ([codex] 3.1): every full parameter's own range
        into the flat shard (or into ``dst``, a buffer of the shard's size).
        Set-up work: the step itself never copies parameters back."""
        n, ids, ptrs = self._p
        out = self.shard if dst is None else dst
        self._ok(zs.lib().zs3_partition(self.h, self.rank, self.dcode, n, ids, ptrs, out.data_ptr(),
                                        stream if stream is not None else self._stream()))

    def grad_norm(self, finalize: bool = True, stream=None):
        if self.fuse_norm:
            self._ok(zs.lib().zs3_grad_norm_partials(self.h, self.rank, self.partials.data_ptr(),
                                                     self.sumsq.data_ptr(), int(finalize), self.max_norm, 1.0,
                                                     self.norm_ptr, self.scale_ptr, self.flag_ptr,
                                                     stream if stream is not None else self._stream()))
            return
        self._ok(zs.lib().zs3_grad_norm(self.h, self.rank, self.dcode, self.grad.data_ptr(), self.sumsq.data_ptr(),
                                        int(finalize), self.max_norm, 1.0, self.norm_ptr, self.scale_ptr,
                                        self.flag_ptr, stream if stream is not None else self._stream()))

    def adam_step(self, t: int, stream=None):
        a = self.adam
        hp = zs.zs3_adam_params(a.lr, a.beta1, a.beta2, a.eps, a.weight_decay, int(t))
        s = stream if stream is not None else self._stream()
        if self.offload:
            cin, cout = (int(x.cuda_stream) for x in self.copy_streams) if self.stage is not None else (None, None)
            for b, e in self.sub_groups:
                self._ok(zs.lib().zs3_adam_step_offload(
                    self.h, self.rank, self.dcode, b, e, self.master.data_ptr(), self.exp_avg.data_ptr(),
                    self.exp_avg_sq.data_ptr(), self.stage.data_ptr() if self.stage is not None else None,
                    self.stage_elems, self.grad.data_ptr(),
                    self.shard.data_ptr(), self.scale_ptr, self.flag_ptr, ctypes.byref(hp), s, cin, cout))
            return
        for b, e in self.sub_groups:
            self._ok(zs.lib().zs3_adam_step(self.h, self.rank, self.dcode, b, e, self.master.data_ptr(),
                                            self.exp_avg.data_ptr(), self.exp_avg_sq.data_ptr(),
                                            self.grad.data_ptr(), self.shard.data_ptr(), self.scale_ptr,
                                            self.flag_ptr, ctypes.byref(hp), s))

    def step(self, stream=None, on_phase=None, gather_timer=None, trace_pass=None):
        """One whole shard step; ``on_phase(name)`` is called before each phase
        and with None at the end (for event timing).  With ``trace_pass`` (a
        TraceGatherPass) the forward and backward gathers follow the
        fetch/release coordinator instead of the static gather buckets."""
        self.t += 1
        mark = on_phase or (lambda name: None)
        if trace_pass is not None:
            mark("gather_trace")
            trace_pass.run(stream)
        else:
            mark("gather_fwd")
            self.gather_pass(stream, gather_timer)
            mark("gather_bwd")
            self.gather_pass(stream, gather_timer)
        mark("reduce_scatter")
        self.reduce_scatter(stream)
        # the pre-step pass ([codex] 6.3): the gathered views are dropped;
        # the shard already is the partitioned form, so nothing moves
        mark("grad_norm")
        self.grad_norm(True, stream)
        mark("adam")
        self.adam_step(self.t, stream)
        mark(None)

    # ------------------------------------------------------------ set-up
    def init_from_full(self):
        """Partition the gathered/persistent full parameters into the shard,
        fill every virtual rank's chunk of every wire buffer (what the
        all-gather would deliver), and build the fp32 optimizer partition
        from the shard ([codex] 6.1: master = the shard widened, padding 0;
        momentum and variance 0), all through the library's calls."""
        torch = self.torch
        tmp = torch.zeros_like(self.shard)
        n, ids, ptrs = self._p
        lib = zs.lib()
        s = self._stream()
        for v in range(self.N):
            target = self.shard if v == self.rank else tmp
            self._ok(lib.zs3_partition(self.h, v, self.dcode, n, ids, ptrs, target.data_ptr(), s))
            for bi, (bn, bids, _, _, _) in enumerate(self._g):
                self._ok(lib.zs3_gather_coalesced(self.h, v, self.dcode, zs.ZS3_PACK, bn, bids, target.data_ptr(),
                                                  self.chunk_ptr(bi, v), None, None, None, s))
        del tmp
        if self.offload:
            # built in HBM one sub-group at a time, then moved to the pinned host state
            big = max((e - b for b, e in self.sub_groups), default=0)
            w = torch.empty(max(1, big), dtype=torch.float32, device=self.device)
            for b, e in self.sub_groups:
                self._ok(lib.zs3_init_master(self.h, self.rank, self.dcode, b, e, self.shard.data_ptr(),
                                             w.data_ptr() - 4 * b, None, None, s))
                self.master[b:e].copy_(w[:e - b])
            torch.cuda.current_stream().synchronize()
            self.exp_avg.zero_()
            self.exp_avg_sq.zero_()
            return
        for b, e in self.sub_groups:
            self._ok(lib.zs3_init_master(self.h, self.rank, self.dcode, b, e, self.shard.data_ptr(),
                                         self.master.data_ptr(), self.exp_avg.data_ptr(),
                                         self.exp_avg_sq.data_ptr(), s))

    def fill_peer_norms(self):
        """Stand-in for the N-scalar all-reduce of the norm: after one partial
        on this rank, give every other rank the same partial sum."""
        self.grad_norm(finalize=False)
        self.sumsq[: self.N] = self.sumsq[self.rank].item()

    # --------------------------------------------------------- accounting
    def algorithmic_bytes(self) -> Dict[str, int]:
        """Bytes each part of the step must move (real elements only)."""
        N = self.N
        part_real = sum(p["own"][1] - p["own"][0] for p in self.params if not p["persistent"])
        own = self.own_real
        F = self.F
        out = {
            "pack": 2 * 4 * part_real,          # two passes, read + write of the real own shard elements
            "unpack": 2 * 4 * F,                # two passes, read N pieces + write the full parameters
            "reduce_scatter": 2 * N * own + 2 * own,
            "grad_norm": 0 if self.fuse_norm else 2 * own,    # fused: no second read of grad_flat
            "adam": 28 * own,
        }
        if self.reduce_path == "coalesced":
            # send side: read the own full gradients, write N chunks (padding zeros included)
            full_part = sum(p["numel"] for p in self.params if not p["persistent"])
            chunks = sum(C for _, _, C, _, _ in self.coalesced)
            out["scatter_pack"] = 2 * full_part + 2 * N * chunks
        return out

    def budget_bytes(self) -> int:
        """The step's fixed algorithmic byte budget: forward and backward
        gather (pack + unpack), the reduce-scatter, a norm that reads the
        flat gradient once, and Adam -- the same work for every variant of
        the step, so that effective bandwidth compares them at equal work."""
        N = self.N
        part_real = sum(p["own"][1] - p["own"][0] for p in self.params if not p["persistent"])
        own = self.own_real
        return 2 * 4 * part_real + 2 * 4 * self.F + (2 * N + 2) * own + 2 * own + 28 * own

    def partition_bytes(self) -> int:
        """The partition copy (set-up, not part of the step): read and write
        every real own element once."""
        return 4 * self.own_real

    def destroy(self):
        if self.h:
            zs.zs3_layout_destroy(self.h)
            self.h = None
