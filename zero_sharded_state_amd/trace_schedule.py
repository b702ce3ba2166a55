"""Forward and backward parameter gathers driven by the fetch/release
coordinator ([codex] 5): the module order of a step is fed to
``zs3_coord_fetch`` / ``zs3_coord_release``, and every gather it returns
(the current module's, and the prefetch bucket) runs as one fused
``zs3_gather_coalesced`` (pack + unpack) on the device.

One GPU holds the N ranks as virtual ranks, so the chunks the other ranks
would contribute to each gather are prepared once, per gather bucket, from
their own shards.  Each gather writes its bucket's parameters into a
buffer of its own in a per-step arena (the views the module computes on);
nothing else moves.  The coordinator's buckets repeat from step to step once
its trace is complete, so the arena places each bucket at a fixed offset,
found by its position in the step's sequence of gathers.
"""

from __future__ import annotations

import ctypes
from typing import Dict, List, Sequence, Tuple

import zero_sharded_state_amd as zs


class TraceGatherPass:
    def __init__(self, step, modules: Sequence[Sequence[int]], order: Sequence[int], cfg: dict):
        """step: a ShardStep (its layout, rank, dtype and shard); modules[m] =
        ds_ids of module m; order = modules fetched in one step (forward,
        then backward); cfg = zs3_coord_config fields."""
        self.step = step
        self.modules = [list(m) for m in modules]
        self.order = list(order)
        self.coord = zs.zs3_coord_create(step.h, self.modules, cfg)
        self.n_ids = max(1, sum(len(m) for m in self.modules))
        self._ids = (ctypes.c_int64 * self.n_ids)()
        self._kinds = (ctypes.c_int32 * 2)()
        self._starts = (ctypes.c_int32 * 3)()
        self._n = ctypes.c_int32()
        self.ops: List[List[int]] = []          # the complete trace's gathers, in order
        self.kinds: List[int] = []

    # ----------------------------------------------------------- host side
    def _fetch(self, m: int) -> List[Tuple[int, List[int]]]:
        lib = zs.lib()
        st = lib.zs3_coord_fetch(self.coord, m, ctypes.byref(self._n), self._kinds, self._starts, self._ids)
        if st != 0:
            raise zs.Zs3Error(st, zs.zs3_last_error())
        return [(self._kinds[g], list(self._ids[self._starts[g]:self._starts[g + 1]])) for g in range(self._n.value)]

    def _release(self, m: int) -> int:
        st = zs.lib().zs3_coord_release(self.coord, m, ctypes.byref(self._n), self._ids)
        if st != 0:
            raise zs.Zs3Error(st, zs.zs3_last_error())
        return self._n.value

    def _host_step(self) -> List[Tuple[int, List[int]]]:
        ops = []
        for m in self.order:
            ops += self._fetch(m)
            self._release(m)
        zs.zs3_coord_release_all(self.coord)
        zs.zs3_coord_reset_step(self.coord)
        return ops

    def plan(self):
        """Run the coordinator until its trace is complete, then record one
        step's gathers and lay out their buffers."""
        for _ in range(8):
            if zs.zs3_coord_info(self.coord)["mode"] == zs.ZS3_TRACE_COMPLETE:
                break
            self._host_step()
        if zs.zs3_coord_info(self.coord)["mode"] != zs.ZS3_TRACE_COMPLETE:
            raise RuntimeError("the coordinator's trace did not complete")
        ops = self._host_step()
        self.kinds = [k for k, _ in ops]
        self.ops = [g for _, g in ops]
        s = self.step
        N, r = s.N, s.rank
        self.meta = []          # (full offset, full numel, wire offset, chunk numel)
        f = w = 0
        for g in self.ops:
            c, n = zs.zs3_bucket_sizes(s.h, g)
            self.meta.append((f, n, w, c))
            f += (n + 127) // 128 * 128
            w += (N * c + 127) // 128 * 128
        torch = s.torch
        self.full = torch.empty(max(1, f), dtype=torch.int16, device=s.device)
        self.wire = torch.empty(max(1, w), dtype=torch.int16, device=s.device)
        P = ctypes.c_void_p
        self._args = []
        for g, (fo, n, wo, c) in zip(self.ops, self.meta):
            ids = (ctypes.c_int64 * len(g))(*g)
            chunks = (P * N)(*[self.wire.data_ptr() + 2 * (wo + v * c) for v in range(N)])
            self._args.append((len(g), ids, self.wire.data_ptr() + 2 * (wo + r * c), chunks,
                               self.full.data_ptr() + 2 * fo))
        self.gathered = sum(n for _, n, _, _ in self.meta)
        self.packed = sum(sum(s.by_id[d]["own"][1] - s.by_id[d]["own"][0] for d in g) for g in self.ops)

    def fill_peer_chunks(self):
        """What the other ranks contribute to every gather: their packs of
        the bucket, from their shards (each virtual rank's shard is the
        partition of the same full parameters)."""
        s = self.step
        tmp = s.torch.zeros_like(s.shard)
        n, ids, ptrs = s._p
        lib = zs.lib()
        st = s._stream()
        for v in range(s.N):
            if v == s.rank:
                continue
            s._ok(lib.zs3_partition(s.h, v, s.dcode, n, ids, ptrs, tmp.data_ptr(), st))
            for (bn, bids, _, chunks, _) in self._args:
                s._ok(lib.zs3_gather_coalesced(s.h, v, s.dcode, zs.ZS3_PACK, bn, bids, tmp.data_ptr(),
                                               chunks[v], None, None, None, st))
        del tmp

    # --------------------------------------------------------- device side
    def run(self, stream=None, streams=None):
        """One step's fetches and releases, each returned gather launched as
        it is returned.  Every gather writes a buffer of its own, so they are
        dealt round-robin over the step's gather streams (``streams``
        overrides the count) and joined into the launch stream at the end.
        Returns the number of gathers."""
        s = self.step
        lib = zs.lib()
        main, aux, handles = s._fanout(stream, s.gather_streams if streams is None else streams)
        i = 0
        for m in self.order:
            for kind, g in self._fetch(m):
                if i >= len(self.ops) or g != self.ops[i]:
                    raise RuntimeError("the coordinator's gathers changed from the planned step")
                n, ids, own, chunks, fullp = self._args[i]
                s._ok(lib.zs3_gather_coalesced(s.h, s.rank, s.dcode, zs.ZS3_PACK | zs.ZS3_UNPACK, n, ids,
                                               s.shard.data_ptr(), own, chunks, fullp, None,
                                               handles[i % len(handles)]))
                i += 1
            self._release(m)
        s._join(main, aux)
        zs.zs3_coord_release_all(self.coord)
        zs.zs3_coord_reset_step(self.coord)
        if i != len(self.ops):
            raise RuntimeError("the coordinator's gathers changed from the planned step")
        return i

    def algorithmic_bytes(self) -> int:
        """Pack reads and writes the real own elements; unpack reads the N
        pieces and writes the full parameters (real elements only)."""
        return 4 * self.packed + 4 * self.gathered

    def destroy(self):
        if self.coord:
            zs.zs3_coord_destroy(self.coord)
            self.coord = None
