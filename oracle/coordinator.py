"""The fetch/release coordinator of ZeRO-3, as a plain step-by-step
simulation (TEST INFRASTRUCTURE ONLY).

Page tags are defined in ``oracle/__init__.py``.  [codex] 5 describes the
coordinator in three parts, followed here in the pages' order:

* 5.1 trace: a state machine INVALID -> RECORD -> COMPLETE advanced at
  every end of step; the step after the first records the module order,
  the next end of step turns it into a parameter-level script, and from
  then on the script drives prefetching.  A module order that differs from
  the script drops the trace (prefetching stops) and it is recorded again
  ([codex] 5.1 and section 7, dynamic graphs).
* 5.2 fetch: (i) issue the all-gather of the current module's parameters,
  (ii) wait for them, (iii) with a complete trace, pop the following
  parameters from the script queue until prefetch_bucket_size elements are
  collected or max_live_parameters would be passed, and issue one more
  all-gather for them.
* 5.3 release: a module's parameters go back to partitioned form unless
  the prefetcher has marked a later use, or a module within
  max_reuse_distance elements further on uses them again; persistent
  parameters are never gathered or released.

Readings where the pages leave a step open (each stated again where it is
used): a parameter is live (counted against max_live_parameters) from the
issue of its gather to its release; the reuse distance of a later module
is the sum of the partitioned-parameter elements of the modules strictly
between; gathers list their parameters in ascending ds_id ([codex] 5.2, 7);
the end of step releases nothing by itself (the pre-step pass does, see
``release_all``).

Every call returns the operations it decided, so that two implementations
can be compared event by event.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

INVALID, RECORD, COMPLETE = 0, 1, 2
NOT_AVAILABLE, INFLIGHT, AVAILABLE = 0, 1, 2
CURRENT, PREFETCH = 0, 1


@dataclass
class CoordConfig:
    prefetch_bucket_size: int = int(5e7)
    max_live_parameters: int = int(1e9)
    max_reuse_distance: int = int(1e9)


def fnv1a64_bytes(data: bytes) -> int:
    """64-bit FNV-1a (offset basis 14695981039346656037, prime
    1099511628211): for each byte, xor it in, then multiply."""
    h = 14695981039346656037
    for byte in data:
        h ^= byte
        h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def fnv1a64(values: Sequence[int]) -> int:
    """FNV-1a over the little-endian bytes of each value as a 64-bit integer."""
    return fnv1a64_bytes(b"".join((int(v) & 0xFFFFFFFFFFFFFFFF).to_bytes(8, "little") for v in values))


@dataclass
class Coordinator:
    numel: Dict[int, int]
    persistent: Dict[int, bool]
    modules: List[List[int]]                 # module id -> its parameters (ds_ids, ascending)
    cfg: CoordConfig = field(default_factory=CoordConfig)

    def __post_init__(self):
        self.modules = [sorted(set(int(d) for d in m)) for m in self.modules]
        self.mode = INVALID
        self.status = {d: (AVAILABLE if self.persistent[d] else NOT_AVAILABLE) for d in self.numel}
        self.live = 0
        self.trace: List[int] = []
        self.script: List[Tuple[int, int]] = []
        self.step_pos = 0
        self.cursor = 0
        self.marked: Dict[int, int] = {}          # ds_id -> latest script position the prefetcher popped
        self.fetched_at: Dict[int, int] = {}      # module -> trace position of its latest fetch
        self.invalidations = 0

    # ------------------------------------------------------------ helpers
    def _partitioned(self, m: int) -> List[int]:
        return [d for d in self.modules[m] if not self.persistent[d]]

    def _size(self, m: int) -> int:
        return sum(self.numel[d] for d in self._partitioned(m))

    def _invalidate(self):
        self.mode = INVALID
        self.invalidations += 1

    # -------------------------------------------------------------- fetch
    def fetch(self, m: int) -> List[Tuple[int, List[int]]]:
        """Gathers to issue for module m, in order: (CURRENT, ids) then
        (PREFETCH, ids); empty ones are left out."""
        k = self.step_pos
        self.step_pos += 1
        self.fetched_at[m] = k
        # 5.1: record, or check the script
        if self.mode == RECORD:
            self.trace.append(m)
        elif self.mode == COMPLETE and (k >= len(self.trace) or self.trace[k] != m):
            self._invalidate()
        ops: List[Tuple[int, List[int]]] = []
        # 5.2 (i): the current module's parameters that are not live
        need = [d for d in self._partitioned(m) if self.status[d] == NOT_AVAILABLE]
        for d in need:
            self.status[d] = INFLIGHT
            self.live += self.numel[d]
        if need:
            ops.append((CURRENT, sorted(need)))
        # 5.2 (ii): wait -- every parameter of the module is now available
        for d in self._partitioned(m):
            self.status[d] = AVAILABLE
        # 5.2 (iii): prefetch along the script
        if self.mode == COMPLETE and self.cfg.prefetch_bucket_size > 0:
            while self.cursor < len(self.script) and self.script[self.cursor][0] <= k:
                self.cursor += 1
            bucket: List[int] = []
            filled = 0
            while self.cursor < len(self.script):
                pos, d = self.script[self.cursor]
                if self.status[d] != NOT_AVAILABLE:
                    # already live: mark the later use, keep going
                    self.marked[d] = max(self.marked.get(d, -1), pos)
                    self.cursor += 1
                    continue
                n = self.numel[d]
                if bucket and filled + n > self.cfg.prefetch_bucket_size:
                    break
                if self.live + n > self.cfg.max_live_parameters:
                    break
                bucket.append(d)
                filled += n
                self.live += n
                self.status[d] = INFLIGHT
                self.marked[d] = max(self.marked.get(d, -1), pos)
                self.cursor += 1
            if bucket:
                ops.append((PREFETCH, sorted(bucket)))
        return ops

    # ------------------------------------------------------------ release
    def _reused_soon(self, d: int, k: int) -> bool:
        """Some module within max_reuse_distance elements after trace
        position k uses d (the distance of a module is the sum of the sizes
        of the modules strictly between)."""
        dist = 0
        for k2 in range(k + 1, len(self.trace)):
            m2 = self.trace[k2]
            if d in self.modules[m2]:
                return True
            dist += self._size(m2)
            if dist > self.cfg.max_reuse_distance:
                return False
        return False

    def release(self, m: int) -> List[int]:
        if m not in self.fetched_at:
            raise ValueError(f"module {m} was not fetched in this step")
        k = self.fetched_at.pop(m)
        out = []
        for d in self._partitioned(m):
            if self.status[d] != AVAILABLE:
                continue
            if self.marked.get(d, -1) > k:
                continue
            if self.mode == COMPLETE and self._reused_soon(d, k):
                continue
            self.status[d] = NOT_AVAILABLE
            self.live -= self.numel[d]
            out.append(d)
        return sorted(out)

    def release_all(self) -> List[int]:
        """The pre-step pass ([codex] 6.3): every parameter back to
        partitioned form."""
        out = [d for d in sorted(self.numel) if not self.persistent[d] and self.status[d] != NOT_AVAILABLE]
        for d in out:
            self.status[d] = NOT_AVAILABLE
            self.live -= self.numel[d]
        self.fetched_at.clear()
        return out

    # ---------------------------------------------------------- end of step
    def reset_step(self) -> int:
        if self.mode == COMPLETE and self.step_pos != len(self.trace):
            self._invalidate()
        if self.mode == INVALID:
            self.mode = RECORD
            self.trace = []
            self.script = []
        elif self.mode == RECORD:
            self.mode = COMPLETE
            self.script = [(k, d) for k, m in enumerate(self.trace) for d in self._partitioned(m)]
        self.step_pos = 0
        self.cursor = 0
        self.marked = {}
        self.fetched_at = {}
        return self.mode

    def signature(self) -> Tuple[int, int, int]:
        """What ranks compare at the end of a recording step ([codex] 5.1:
        module order, parameter order, number of fetches)."""
        return fnv1a64(self.trace), fnv1a64([d for _, d in self.script]), len(self.trace)
