"""The ZeRO-3 shard step, written out as plain numpy (TEST INFRASTRUCTURE ONLY).

Page tags ([codex], [csdn], [llmnex]) are defined in ``oracle/__init__.py``.

16-bit values are carried as ``np.uint16`` bit patterns together with a
dtype tag (``"fp16"`` or ``"bf16"``); numpy has no bfloat16.  Every
floating-point step is one IEEE operation on ``np.float32`` (or ``float64``
where stated), so the sequence of roundings is the one written here and no
fused multiply-add can appear.

Where the pages leave a step open, the reading taken is stated in the
docstring (the list of readings is kept with the design notes).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

FP16 = "fp16"
BF16 = "bf16"
_DTYPES = (FP16, BF16)


# --------------------------------------------------------------------------
# 16-bit storage types
# --------------------------------------------------------------------------

def to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit bit patterns to fp32.

    fp16: IEEE binary16 -> binary32 (every binary16 value, subnormals
    included, is representable).  bf16: the bit pattern is the upper half of
    an fp32 pattern, so widening appends 16 zero bits.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def from_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 to the 16-bit type, to nearest with ties to even.

    fp16 uses numpy's IEEE conversion (round to nearest even, overflow to
    inf, subnormals kept).  bf16 keeps the upper 16 bits of the fp32 pattern
    and rounds by the discarded lower 16 bits: up when they exceed half, or
    equal half and the kept part is odd.  NaN stays NaN (quiet bit set).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == FP16:
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32).astype(np.uint64)
        hi = u >> np.uint64(16)
        lo = u & np.uint64(0xFFFF)
        half = np.uint64(0x8000)
        up = (lo > half) | ((lo == half) & ((hi & np.uint64(1)) == np.uint64(1)))
        out = hi + up.astype(np.uint64)
        nan = np.isnan(x)
        out[nan] = hi[nan] | np.uint64(0x40)
        return out.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# a1: flat partition layout
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class ParamSlot:
    ds_id: int
    numel: int
    persistent: bool
    partition_size: int   # elements every rank holds for this parameter
    shard_offset: int     # start of those elements in the rank's flat shard


@dataclass(frozen=True)
class Layout:
    world_size: int
    threshold: int
    params: Tuple[ParamSlot, ...]      # ascending ds_id
    shard_numel: int                   # S + P: elements of one rank's flat shard

    def slot(self, ds_id: int) -> ParamSlot:
        for p in self.params:
            if p.ds_id == ds_id:
                return p
        raise KeyError(ds_id)

    def own_range(self, p: ParamSlot, rank: int) -> Tuple[int, int]:
        """[lo, hi) of the flattened parameter that ``rank`` holds real data for."""
        if p.persistent:
            return 0, p.numel
        lo = rank * p.partition_size
        hi = min(lo + p.partition_size, p.numel)
        return lo, max(lo, hi)

    @property
    def bytes_per_rank(self) -> int:
        """16 bytes per held element: 16-bit param + 16-bit grad + fp32 master, m, v.

        [codex] section 1 (16 Psi / N per card) and [llmnex] section 1
        (2 + 2 + 12 bytes per parameter).
        """
        return 16 * self.shard_numel


def make_layout(world_size: int, threshold: int, ds_ids: Sequence[int],
                numels: Sequence[int]) -> Layout:
    """Per-parameter partition sizes and flat-shard offsets.

    [codex] 3.1: the partition routine gives rank r the elements
    [r * partition_size, (r + 1) * partition_size) of each flattened
    parameter.  [codex] 5.3: parameters below the persistence threshold are
    never partitioned and stay whole on every rank.  [codex] 5.2: the
    coalesced gather orders parameters by ds_id, so the flat shard is laid
    out in ascending ds_id.

    Readings: partition_size = ceil(numel / N) (the pages give only the
    range); positions >= numel are zero padding; "below" means numel <
    threshold.
    """
    if world_size < 1:
        raise ValueError("world_size must be >= 1")
    if len(ds_ids) != len(numels):
        raise ValueError("ds_ids and numels differ in length")
    if len(set(int(d) for d in ds_ids)) != len(ds_ids):
        raise ValueError("duplicate ds_id")
    order = sorted(range(len(ds_ids)), key=lambda i: int(ds_ids[i]))
    slots: List[ParamSlot] = []
    offset = 0
    for i in order:
        d, n = int(ds_ids[i]), int(numels[i])
        if d < 0:
            raise ValueError("ds_id must be >= 0")
        if n < 1:
            raise ValueError("numel must be >= 1")
        persistent = n < threshold
        ps = n if persistent else -(-n // world_size)
        slots.append(ParamSlot(d, n, persistent, ps, offset))
        offset += ps
    return Layout(int(world_size), int(threshold), tuple(slots), offset)


def partition(layout: Layout, rank: int, full: Dict[int, np.ndarray]) -> np.ndarray:
    """The rank's flat shard from the full (flattened) parameters.

    [codex] 3.1 (own element range copied into the rank's shard) and 5.3
    (persistent parameters copied whole).  Padding positions hold 0.
    """
    out = np.zeros(layout.shard_numel, dtype=np.uint16)
    for p in layout.params:
        flat = np.asarray(full[p.ds_id], dtype=np.uint16).reshape(-1)
        assert flat.size == p.numel
        lo, hi = layout.own_range(p, rank)
        out[p.shard_offset:p.shard_offset + (hi - lo)] = flat[lo:hi]
    return out


# --------------------------------------------------------------------------
# a2: all_gather_coalesced pack / unpack
# --------------------------------------------------------------------------

def _bucket(layout: Layout, ds_ids: Sequence[int], allow_persistent: bool) -> List[ParamSlot]:
    if len(set(int(d) for d in ds_ids)) != len(ds_ids):
        raise ValueError("duplicate ds_id in request")
    slots = sorted((layout.slot(int(d)) for d in ds_ids), key=lambda p: p.ds_id)
    if not allow_persistent and any(p.persistent for p in slots):
        raise ValueError("persistent parameter in a gather bucket")
    return slots


def bucket_sizes(layout: Layout, ds_ids: Sequence[int]) -> Tuple[int, int]:
    """(chunk elements per rank, full elements) of a gather bucket."""
    slots = _bucket(layout, ds_ids, allow_persistent=False)
    return sum(p.partition_size for p in slots), sum(p.numel for p in slots)


def pack(layout: Layout, rank: int, ds_ids: Sequence[int],
         shard_flat: np.ndarray) -> np.ndarray:
    """The rank's contribution to one coalesced all-gather.

    [codex] 5.2: the shards of the requested group are ordered by ds_id and
    joined into one flat buffer before the single collective; the request
    order does not matter.  Each shard is taken whole (padding included).
    """
    slots = _bucket(layout, ds_ids, allow_persistent=False)
    parts = [shard_flat[p.shard_offset:p.shard_offset + p.partition_size] for p in slots]
    return np.concatenate(parts).astype(np.uint16) if parts else np.zeros(0, np.uint16)


def wire(chunks: Sequence[np.ndarray]) -> np.ndarray:
    """What the all-gather delivers: the N chunks back to back, rank-major."""
    return np.concatenate([np.asarray(c, np.uint16) for c in chunks])


def unpack(layout: Layout, ds_ids: Sequence[int],
           chunks: Sequence[np.ndarray]) -> Tuple[np.ndarray, Dict[int, int]]:
    """Full parameters of a bucket from the N ranks' chunks.

    [codex] 5.2: after the collective, each parameter's data is a view of
    one flat buffer.  The view of parameter j starts at f_j (prefix sum of
    full sizes in ds_id order); element v * ps_j + k of it comes from chunk v
    at c_j + k (c_j = prefix sum of partition sizes); padding is dropped.
    Returns the flat buffer and {ds_id: view offset}.
    """
    slots = _bucket(layout, ds_ids, allow_persistent=False)
    N = layout.world_size
    assert len(chunks) == N
    total = sum(p.numel for p in slots)
    full = np.empty(total, dtype=np.uint16)
    offsets: Dict[int, int] = {}
    c = 0
    f = 0
    for p in slots:
        offsets[p.ds_id] = f
        for v in range(N):
            lo, hi = layout.own_range(p, v)
            full[f + lo:f + hi] = np.asarray(chunks[v], np.uint16)[c:c + (hi - lo)]
        c += p.partition_size
        f += p.numel
    return full, offsets


def _greedy(items: Sequence[ParamSlot], size_of, limit: int) -> List[List[int]]:
    """Greedy bucketing: close the bucket before an item that would take it
    past ``limit``, unless the bucket is empty (an oversize item gets one)."""
    buckets: List[List[int]] = []
    cur: List[int] = []
    fill = 0
    for p in items:
        s = size_of(p)
        if cur and fill + s > limit:
            buckets.append(cur)
            cur, fill = [], 0
        cur.append(p.ds_id)
        fill += s
    if cur:
        buckets.append(cur)
    return buckets


def gather_buckets(layout: Layout, prefetch_bucket_size: int) -> List[List[int]]:
    """Gather buckets: non-persistent parameters in ds_id order, filled up to
    ``prefetch_bucket_size`` full elements ([codex] 5.2 step 3; reading:
    greedy fill, count full numel)."""
    items = [p for p in layout.params if not p.persistent]
    return _greedy(items, lambda p: p.numel, int(prefetch_bucket_size))


def reduce_buckets(layout: Layout, reduce_bucket_size: int) -> List[List[int]]:
    """Gradient buckets in backward arrival order (reverse ds_id), all
    parameters, filled up to ``reduce_bucket_size`` full elements ([codex]
    6.2: gradients collect in a bucket that is reduced when full)."""
    items = list(reversed(layout.params))
    return _greedy(items, lambda p: p.numel, int(reduce_bucket_size))


def sub_groups(layout: Layout, sub_group_size: int) -> List[Tuple[int, int]]:
    """Sub-groups as [begin, end) ranges of the rank's flat shard ([codex] 6.1:
    parameters are split into sub-groups of at most sub_group_size elements;
    reading: counted in per-rank shard elements, greedy in ds_id order,
    never splitting a parameter)."""
    groups = _greedy(list(layout.params), lambda p: p.partition_size, int(sub_group_size))
    out = []
    for g in groups:
        first = layout.slot(g[0])
        last = layout.slot(g[-1])
        out.append((first.shard_offset, last.shard_offset + last.partition_size))
    return out


# --------------------------------------------------------------------------
# a3: local reduce-scatter into the flat gradient buffer
# --------------------------------------------------------------------------

def reduce_scatter(layout: Layout, rank: int, dtype: str, ds_ids: Sequence[int],
                   grads: Sequence[Dict[int, np.ndarray]], grad_flat: np.ndarray) -> None:
    """Average the N ranks' gradients and keep only the rank's own slice.

    [codex] 6.2: the contiguous path all-reduces the bucket and each rank
    keeps its own interval, written into the one contiguous flat gradient
    buffer; no rank ever holds the full averaged gradient.  [csdn] core
    algorithm step 3 and the worked example: the reduction is a sum followed
    by the average, and each GPU keeps only its part.

    ``grads[v][ds_id]`` is virtual rank v's full flattened 16-bit gradient.
    Reading of the arithmetic: fp32 sum starting at +0.0 over v = 0..N-1 in
    that order, then one fp32 division by N, then round to the 16-bit type.
    Padding positions of the slice are written as 0.  Writes in place.
    """
    N = layout.world_size
    assert len(grads) == N
    for p in _bucket(layout, ds_ids, allow_persistent=True):
        lo, hi = layout.own_range(p, rank)
        acc = np.zeros(hi - lo, dtype=np.float32)
        for v in range(N):
            g = np.asarray(grads[v][p.ds_id], np.uint16).reshape(-1)
            acc = acc + to_f32(g[lo:hi], dtype)
        avg = acc / np.float32(N)
        o = p.shard_offset
        grad_flat[o:o + (hi - lo)] = from_f32(avg, dtype)
        grad_flat[o + (hi - lo):o + p.partition_size] = 0


def scatter_pack(layout: Layout, ds_ids: Sequence[int],
                 grads: Dict[int, np.ndarray]) -> List[np.ndarray]:
    """One rank's send side of the non-contiguous gradient path.

    [codex] 6.2, second row of the reduce-path table: without a contiguous
    bucket the gradients go through reduce_scatter_coalesced, which
    scatters straight to the owners.  Reading: the wire mirrors
    all_gather_coalesced ([codex] 5.2, 7): the bucket's parameters in
    ascending ds_id, each split into N partitions of partition_size
    elements (zeros past numel); chunk d holds partition d of every
    parameter back to back, so chunk d goes to rank d.  ``grads[ds_id]`` is
    this rank's full flattened 16-bit gradient.  Persistent parameters are
    never partitioned ([codex] 5.3) and take the all-reduce path instead.
    Returns the N chunks.
    """
    slots = _bucket(layout, ds_ids, allow_persistent=False)
    N = layout.world_size
    chunks = []
    for d in range(N):
        parts = []
        for p in slots:
            g = np.asarray(grads[p.ds_id], np.uint16).reshape(-1)
            assert g.size == p.numel
            part = np.zeros(p.partition_size, dtype=np.uint16)
            lo, hi = layout.own_range(p, d)
            part[:hi - lo] = g[lo:hi]
            parts.append(part)
        chunks.append(np.concatenate(parts) if parts else np.zeros(0, np.uint16))
    return chunks


def scatter_reduce(layout: Layout, rank: int, dtype: str, ds_ids: Sequence[int],
                   received: Sequence[np.ndarray], grad_flat: np.ndarray) -> None:
    """The owner's side of the non-contiguous gradient path.

    ``received[v]`` is chunk ``rank`` of virtual rank v's ``scatter_pack``
    (what the reduce-scatter delivers from v).  Same arithmetic as
    ``reduce_scatter`` ([codex] 6.2; [csdn] step 3): fp32 sum from +0 over
    v = 0..N-1 in order, one fp32 division by N, round to the 16-bit type,
    written at the parameter's place in the flat gradient buffer; padding
    positions are written as 0 whatever the chunks hold there.
    """
    slots = _bucket(layout, ds_ids, allow_persistent=False)
    N = layout.world_size
    assert len(received) == N
    c = 0
    for p in slots:
        lo, hi = layout.own_range(p, rank)
        acc = np.zeros(hi - lo, dtype=np.float32)
        for v in range(N):
            acc = acc + to_f32(np.asarray(received[v], np.uint16)[c:c + (hi - lo)], dtype)
        avg = acc / np.float32(N)
        o = p.shard_offset
        grad_flat[o:o + (hi - lo)] = from_f32(avg, dtype)
        grad_flat[o + (hi - lo):o + p.partition_size] = 0
        c += p.partition_size


# --------------------------------------------------------------------------
# a4: shard-aware global gradient norm and shared clip coefficient
# --------------------------------------------------------------------------

def grad_norm_partial(layout: Layout, rank: int, dtype: str,
                      grad_flat: np.ndarray) -> Tuple[float, float]:
    """(sum of squares over the rank's real partitioned gradient elements,
    sum of squares over the persistent gradients), both in fp64.

    [llmnex] pitfall 1: each card sees only its own part of the norm, so
    the per-card sums must be combined before a clip coefficient is formed.
    Persistent gradients are held whole by every rank, so they form a second
    sum that is counted once globally.  Squares of 16-bit values are exact
    in fp64.
    """
    part = 0.0
    pers = 0.0
    for p in layout.params:
        lo, hi = layout.own_range(p, rank)
        seg = grad_flat[p.shard_offset:p.shard_offset + (hi - lo)]
        s = float(np.sum(to_f32(seg, dtype).astype(np.float64) ** 2))
        if p.persistent:
            pers += s
        else:
            part += s
    return part, pers


def grad_norm_finalize(partials: Sequence[float], persistent: float,
                       max_norm: float, loss_scale: float = 1.0):
    """Global norm, shared clip coefficient and the combined gradient scale.

    [codex] 6.3: every sub-group is unscaled and clipped with the one global
    norm.  [llmnex] pitfall 1: the coefficient must be the same on every
    card.  Reading: total = sum of the N per-rank partials in rank order plus
    the persistent sum; norm = sqrt(total) in fp64; coefficient =
    min(1, max_norm / (norm + 1e-6)); scale = fp32(coefficient / loss_scale).
    Returns (norm, coefficient, scale as np.float32, nonfinite flag).
    """
    total = 0.0
    for s in partials:
        total += float(s)
    total += float(persistent)
    nonfinite = not math.isfinite(total)
    norm = math.sqrt(total) if not nonfinite else float("nan")
    if nonfinite:
        return norm, float("nan"), np.float32(np.nan), True
    coef = min(1.0, float(max_norm) / (norm + 1e-6))
    scale = np.float32(coef / float(loss_scale))
    return norm, coef, scale, False


# --------------------------------------------------------------------------
# a5: fused mixed-precision Adam on the rank's fp32 partition, cast back
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class AdamHParams:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    step: int = 1            # t, starting at 1 for the first update


def adam_scalars(hp: AdamHParams) -> Dict[str, np.float32]:
    """The fp32 constants of one step, each rounded once from fp64."""
    t = int(hp.step)
    if t < 1:
        raise ValueError("step must be >= 1")
    f = np.float32
    return {
        "lr": f(hp.lr),
        "b1": f(hp.beta1),
        "b2": f(hp.beta2),
        "omb1": f(1.0 - hp.beta1),
        "omb2": f(1.0 - hp.beta2),
        "bc1": f(1.0 - hp.beta1 ** t),
        "bc2": f(1.0 - hp.beta2 ** t),
        "eps": f(hp.eps),
        "lrwd": f(hp.lr * hp.weight_decay),
    }


def init_state(shard_flat: np.ndarray, dtype: str):
    """fp32 master (exact widening of the 16-bit shard) and zero m, v.

    [codex] 6.1: each sub-group gets the rank's fp32 master partition.
    """
    master = to_f32(shard_flat, dtype).copy()
    return master, np.zeros_like(master), np.zeros_like(master)


def padding_mask(layout: Layout, rank: int) -> np.ndarray:
    """True at the rank's flat-shard positions that are padding."""
    mask = np.zeros(layout.shard_numel, dtype=bool)
    for p in layout.params:
        lo, hi = layout.own_range(p, rank)
        mask[p.shard_offset + (hi - lo):p.shard_offset + p.partition_size] = True
    return mask


def adam_step(layout: Layout, rank: int, dtype: str, begin: int, end: int,
              master: np.ndarray, exp_avg: np.ndarray, exp_avg_sq: np.ndarray,
              grad_flat: np.ndarray, shard_flat: np.ndarray, scale: np.float32,
              nonfinite: bool, hp: AdamHParams) -> None:
    """One Adam step on the flat range [begin, end) of the rank's partition.

    [codex] 6.3: per sub-group, unscale and clip with the global norm, run
    the real optimizer on the rank's fp32 partition only, then write the
    fp32 values back into the 16-bit shard.  [llmnex] section 1: the
    optimizer state is fp32 master weight, momentum and variance.

    The update is Kingma & Ba's Adam with bias correction and eps added
    outside the square root (the pages name Adam's momentum and variance but
    print no formula).  Each line below is one fp32 operation:

        g   = f32(grad16) * scale
        w   = w - lrwd * w               (only if weight_decay != 0: decoupled, as in AdamW)
        m   = b1 * m + omb1 * g
        v   = b2 * v + omb2 * (g * g)
        mh  = m / bc1 ;  vh = v / bc2
        den = sqrt(vh) + eps
        w   = w - lr * (mh / den)
        shard16 = round_to_nearest_even(w)

    Padding positions are skipped (they stay 0).  If ``nonfinite`` is set the
    whole step is skipped and nothing changes.  Works in place.
    """
    if nonfinite:
        return
    c = adam_scalars(hp)
    real = ~padding_mask(layout, rank)[begin:end]
    idx = np.nonzero(real)[0] + begin
    w = master[idx]
    m = exp_avg[idx]
    v = exp_avg_sq[idx]
    g = to_f32(grad_flat[idx], dtype) * np.float32(scale)
    if hp.weight_decay != 0.0:
        w = w - c["lrwd"] * w
    m = c["b1"] * m + c["omb1"] * g
    v = c["b2"] * v + c["omb2"] * (g * g)
    mh = m / c["bc1"]
    vh = v / c["bc2"]
    den = np.sqrt(vh) + c["eps"]
    w = w - c["lr"] * (mh / den)
    master[idx] = w
    exp_avg[idx] = m
    exp_avg_sq[idx] = v
    shard_flat[idx] = from_f32(w, dtype)


# --------------------------------------------------------------------------
# Unsharded reference of a whole step (for the sharding invariants)
# --------------------------------------------------------------------------

def dense_reference_step(dtype: str, params: Dict[int, np.ndarray],
                         grads: Sequence[Dict[int, np.ndarray]],
                         state: Optional[Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]]],
                         max_norm: float, hp: AdamHParams):
    """One data-parallel step with nothing sharded: average every full
    gradient over the N ranks, take the L2 norm of the whole averaged
    gradient, clip, and run the same Adam on every full parameter.

    [llmnex] section 2: the step that ZeRO-3 shards must give what plain
    data parallelism gives; concatenating the ranks' shards of the result
    must reproduce this.  Returns (new params, new state, norm, scale).
    """
    N = len(grads)
    avg = {}
    for d in params:
        acc = np.zeros(np.asarray(params[d]).size, dtype=np.float32)
        for v in range(N):
            acc = acc + to_f32(np.asarray(grads[v][d]).reshape(-1), dtype)
        avg[d] = from_f32(acc / np.float32(N), dtype)
    total = 0.0
    for d in sorted(avg):
        total += float(np.sum(to_f32(avg[d], dtype).astype(np.float64) ** 2))
    norm = math.sqrt(total)
    coef = min(1.0, float(max_norm) / (norm + 1e-6))
    scale = np.float32(coef)
    c = adam_scalars(hp)
    new_params, new_state = {}, {}
    for d in sorted(params):
        if state is None or d not in state:
            w = to_f32(np.asarray(params[d]).reshape(-1), dtype).copy()
            m = np.zeros_like(w)
            v = np.zeros_like(w)
        else:
            w, m, v = (a.copy() for a in state[d])
        g = to_f32(avg[d], dtype) * scale
        if hp.weight_decay != 0.0:
            w = w - c["lrwd"] * w
        m = c["b1"] * m + c["omb1"] * g
        v = c["b2"] * v + c["omb2"] * (g * g)
        mh = m / c["bc1"]
        vh = v / c["bc2"]
        den = np.sqrt(vh) + c["eps"]
        w = w - c["lr"] * (mh / den)
        new_state[d] = (w, m, v)
        new_params[d] = from_f32(w, dtype)
    return new_params, new_state, norm, scale
