"""Planted mistakes in the CPU oracle, for checking that its pins bite.

Each entry replaces one oracle function (or method) with a copy that makes
one plausible slip: an off-by-one, a dropped term, a swapped constant, a
wrong order or stride, a transposed index.  ``install(name)`` applies it in
this process, on the CPU only.  The test suite's ``conftest.py`` calls it
when ``ZS3_ORACLE_MUTANT`` names a mutant, and ``test_oracle_mutants.py``
runs the oracle's pin tests once per mutant and requires them to fail.
Nothing here touches the HIP library.
"""

from __future__ import annotations

import math

import numpy as np

import oracle
import oracle.zero3 as z


def _set(attr, fn):
    setattr(z, attr, fn)
    if hasattr(oracle, attr):
        setattr(oracle, attr, fn)


# ---- layout -----------------------------------------------------------------

def _own_range_short(self, p, rank):
    """Slice end taken as inclusive: each rank loses its last element."""
    if p.persistent:
        return 0, p.numel
    lo = rank * p.partition_size
    hi = min(lo + p.partition_size - 1, p.numel)
    return lo, max(lo, hi)


def _persistent_le(orig):
    def make_layout(world_size, threshold, ds_ids, numels):
        """numel <= threshold counted as persistent (should be <)."""
        L = orig(world_size, threshold, ds_ids, numels)
        slots, off = [], 0
        for p in L.params:
            pers = p.numel <= threshold
            ps = p.numel if pers else -(-p.numel // world_size)
            slots.append(z.ParamSlot(p.ds_id, p.numel, pers, ps, off))
            off += ps
        return z.Layout(L.world_size, L.threshold, tuple(slots), off)
    return make_layout


def _ps_floor(orig):
    def make_layout(world_size, threshold, ds_ids, numels):
        """partition_size = numel // N + 1 instead of ceil(numel / N)."""
        L = orig(world_size, threshold, ds_ids, numels)
        slots, off = [], 0
        for p in L.params:
            ps = p.numel if p.persistent else p.numel // world_size + 1
            slots.append(z.ParamSlot(p.ds_id, p.numel, p.persistent, ps, off))
            off += ps
        return z.Layout(L.world_size, L.threshold, tuple(slots), off)
    return make_layout


# ---- gather -----------------------------------------------------------------

def _pack_request_order(layout, rank, ds_ids, shard_flat):
    """Chunks joined in request order instead of ascending ds_id."""
    z._bucket(layout, ds_ids, allow_persistent=False)
    slots = [layout.slot(int(d)) for d in ds_ids]
    parts = [shard_flat[p.shard_offset:p.shard_offset + p.partition_size] for p in slots]
    return np.concatenate(parts).astype(np.uint16) if parts else np.zeros(0, np.uint16)


def _unpack_with(chunk_step, place):
    def unpack(layout, ds_ids, chunks):
        slots = z._bucket(layout, ds_ids, allow_persistent=False)
        N = layout.world_size
        total = sum(p.numel for p in slots)
        full = np.zeros(total, dtype=np.uint16)
        offsets = {}
        c = f = 0
        for p in slots:
            offsets[p.ds_id] = f
            for v in range(N):
                lo, hi = layout.own_range(p, v)
                src = np.asarray(chunks[v], np.uint16)[c:c + (hi - lo)]
                place(full, f, p, N, v, lo, hi, src)
            c += chunk_step(p, N)
            f += p.numel
        return full, offsets
    return unpack


def _place_plain(full, f, p, N, v, lo, hi, src):
    full[f + lo:f + hi] = src


def _place_rank_minor(full, f, p, N, v, lo, hi, src):
    """Element k of chunk v written to position k * N + v (transposed)."""
    for k, x in enumerate(src):
        j = k * N + v
        if j < p.numel:
            full[f + j] = x


# ---- reduce-scatter ---------------------------------------------------------

def _reduce_scatter_with(order, divide, zero_padding, seeded=False):
    def reduce_scatter(layout, rank, dtype, ds_ids, grads, grad_flat):
        N = layout.world_size
        for p in z._bucket(layout, ds_ids, allow_persistent=True):
            lo, hi = layout.own_range(p, rank)
            acc = None if seeded else np.zeros(hi - lo, dtype=np.float32)
            for v in order(N):
                g = np.asarray(grads[v][p.ds_id], np.uint16).reshape(-1)
                x = z.to_f32(g[lo:hi], dtype)
                acc = x.copy() if acc is None else acc + x
            avg = acc / np.float32(N) if divide else acc
            o = p.shard_offset
            grad_flat[o:o + (hi - lo)] = z.from_f32(avg, dtype)
            if zero_padding:
                grad_flat[o + (hi - lo):o + p.partition_size] = 0
    return reduce_scatter


def _scatter_pack_rotated(layout, ds_ids, grads):
    """Chunk d filled from partition d + 1 (mod N)."""
    slots = z._bucket(layout, ds_ids, allow_persistent=False)
    N = layout.world_size
    chunks = []
    for d in range(N):
        parts = []
        for p in slots:
            g = np.asarray(grads[p.ds_id], np.uint16).reshape(-1)
            part = np.zeros(p.partition_size, dtype=np.uint16)
            lo, hi = layout.own_range(p, (d + 1) % N)
            part[:hi - lo] = g[lo:hi]
            parts.append(part)
        chunks.append(np.concatenate(parts) if parts else np.zeros(0, np.uint16))
    return chunks


def _scatter_reduce_stride(layout, rank, dtype, ds_ids, received, grad_flat):
    """The chunk cursor advances by the real length, not partition_size."""
    slots = z._bucket(layout, ds_ids, allow_persistent=False)
    N = layout.world_size
    c = 0
    for p in slots:
        lo, hi = layout.own_range(p, rank)
        acc = np.zeros(hi - lo, dtype=np.float32)
        for v in range(N):
            acc = acc + z.to_f32(np.asarray(received[v], np.uint16)[c:c + (hi - lo)], dtype)
        o = p.shard_offset
        grad_flat[o:o + (hi - lo)] = z.from_f32(acc / np.float32(N), dtype)
        grad_flat[o + (hi - lo):o + p.partition_size] = 0
        c += hi - lo


# ---- norm -------------------------------------------------------------------

def _norm_partial_with(persistent_separate, accum):
    def grad_norm_partial(layout, rank, dtype, grad_flat):
        part = pers = 0.0
        for p in layout.params:
            lo, hi = layout.own_range(p, rank)
            seg = grad_flat[p.shard_offset:p.shard_offset + (hi - lo)]
            s = float(accum(z.to_f32(seg, dtype)))
            if p.persistent and persistent_separate:
                pers += s
            else:
                part += s
        return part, pers
    return grad_norm_partial


def _finalize_with(coef_of):
    def grad_norm_finalize(partials, persistent, max_norm, loss_scale=1.0):
        total = sum(float(s) for s in partials) + float(persistent)
        if not math.isfinite(total):
            return float("nan"), float("nan"), np.float32(np.nan), True
        norm = math.sqrt(total)
        coef = coef_of(float(max_norm), norm)
        return norm, coef, np.float32(coef / float(loss_scale)), False
    return grad_norm_finalize


# ---- Adam -------------------------------------------------------------------

def _adam_with(slip):
    def adam_step(layout, rank, dtype, begin, end, master, exp_avg, exp_avg_sq, grad_flat, shard_flat, scale,
                  nonfinite, hp):
        if nonfinite:
            return
        c = z.adam_scalars(hp)
        if slip == "padding":
            idx = np.arange(begin, end)
        else:
            idx = np.nonzero(~z.padding_mask(layout, rank)[begin:end])[0] + begin
        w, m, v = master[idx], exp_avg[idx], exp_avg_sq[idx]
        g = z.to_f32(grad_flat[idx], dtype)
        if slip != "unscaled":
            g = g * np.float32(scale)
        if hp.weight_decay != 0.0:
            if slip == "wd_coupled":
                g = g + np.float32(hp.weight_decay) * w
            elif slip == "wd_without_lr":
                w = w - np.float32(hp.weight_decay) * w
            else:
                w = w - c["lrwd"] * w
        if slip == "beta_swap":
            m = c["b2"] * m + c["omb2"] * g
        elif slip == "fma":
            m = (c["b1"].astype(np.float64) * m + c["omb1"].astype(np.float64) * g).astype(np.float32)
        else:
            m = c["b1"] * m + c["omb1"] * g
        v = c["b2"] * v + c["omb2"] * (g * g)
        if slip == "no_bias_correction":
            mh, vh = m, v
        else:
            mh, vh = m / c["bc1"], v / c["bc2"]
        den = np.sqrt(vh + c["eps"]) if slip == "eps_inside" else np.sqrt(vh) + c["eps"]
        if slip == "reordered":
            w = w - (c["lr"] * mh) / den
        else:
            w = w - c["lr"] * (mh / den)
        master[idx], exp_avg[idx], exp_avg_sq[idx] = w, m, v
        shard_flat[idx] = z.from_f32(w, dtype)
    return adam_step


# ---- conversions ------------------------------------------------------------

def _from_f32_bf16_truncate(orig):
    def from_f32(x, dtype):
        """bf16 by truncation instead of round-to-nearest-even."""
        if dtype != z.BF16:
            return orig(x, dtype)
        x = np.ascontiguousarray(x, np.float32)
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return from_f32


def _to_f32_fp16_flush(orig):
    def to_f32(bits, dtype):
        """fp16 subnormals flushed to zero."""
        out = orig(bits, dtype)
        if dtype == z.FP16:
            out = np.where(np.abs(out) < np.float32(2.0 ** -14), np.float32(0.0) * np.sign(out), out)
        return out.astype(np.float32)
    return to_f32


def _install_layout(name):
    if name == "own_range_short":
        z.Layout.own_range = _own_range_short
    elif name == "persistent_le":
        _set("make_layout", _persistent_le(z.make_layout))
    elif name == "partition_size_floor_plus_one":
        _set("make_layout", _ps_floor(z.make_layout))


MUTANTS = {
    "own_range_short": _install_layout,
    "persistent_le": _install_layout,
    "partition_size_floor_plus_one": _install_layout,
    "pack_request_order": lambda n: _set("pack", _pack_request_order),
    "unpack_chunk_stride_numel_div_n": lambda n: _set(
        "unpack", _unpack_with(lambda p, N: p.numel // N, _place_plain)),
    "unpack_rank_minor": lambda n: _set("unpack", _unpack_with(lambda p, N: p.partition_size, _place_rank_minor)),
    "reduce_scatter_no_average": lambda n: _set(
        "reduce_scatter", _reduce_scatter_with(lambda N: range(N), False, True)),
    "reduce_scatter_reverse_rank_order": lambda n: _set(
        "reduce_scatter", _reduce_scatter_with(lambda N: reversed(range(N)), True, True)),
    "reduce_scatter_seeded_with_rank_0": lambda n: _set(
        "reduce_scatter", _reduce_scatter_with(lambda N: range(N), True, True, seeded=True)),
    "reduce_scatter_padding_not_zeroed": lambda n: _set(
        "reduce_scatter", _reduce_scatter_with(lambda N: range(N), True, False)),
    "scatter_pack_rotated": lambda n: _set("scatter_pack", _scatter_pack_rotated),
    "scatter_reduce_stride": lambda n: _set("scatter_reduce", _scatter_reduce_stride),
    "norm_persistent_counted_per_rank": lambda n: _set(
        "grad_norm_partial", _norm_partial_with(False, lambda x: np.sum(x.astype(np.float64) ** 2))),
    "norm_squares_in_fp32": lambda n: _set(
        "grad_norm_partial", _norm_partial_with(True, lambda x: np.sum(x * x, dtype=np.float32))),
    "norm_coefficient_without_eps": lambda n: _set(
        "grad_norm_finalize", _finalize_with(lambda mx, norm: min(1.0, mx / norm) if norm > 0 else 1.0)),
    "norm_coefficient_without_min": lambda n: _set(
        "grad_norm_finalize", _finalize_with(lambda mx, norm: mx / (norm + 1e-6))),
    "adam_eps_inside_sqrt": lambda n: _set("adam_step", _adam_with("eps_inside")),
    "adam_no_bias_correction": lambda n: _set("adam_step", _adam_with("no_bias_correction")),
    "adam_beta1_beta2_swapped": lambda n: _set("adam_step", _adam_with("beta_swap")),
    "adam_gradient_not_scaled": lambda n: _set("adam_step", _adam_with("unscaled")),
    "adam_updates_padding": lambda n: _set("adam_step", _adam_with("padding")),
    "adam_fused_multiply_add": lambda n: _set("adam_step", _adam_with("fma")),
    "adam_reordered_update": lambda n: _set("adam_step", _adam_with("reordered")),
    "adam_weight_decay_coupled_into_gradient": lambda n: _set("adam_step", _adam_with("wd_coupled")),
    "adam_weight_decay_without_lr": lambda n: _set("adam_step", _adam_with("wd_without_lr")),
    "bf16_rounding_by_truncation": lambda n: _set("from_f32", _from_f32_bf16_truncate(z.from_f32)),
    "fp16_subnormals_flushed": lambda n: _set("to_f32", _to_f32_fp16_flush(z.to_f32)),
}


def install(name: str) -> None:
    if name not in MUTANTS:
        raise KeyError(f"unknown oracle mutant {name!r}")
    MUTANTS[name](name)


# ---- the coordinator (oracle/coordinator.py) -------------------------------

import oracle.coordinator as oc  # noqa: E402


def _fetch_with(slip):
    def fetch(self, m):
        k = self.step_pos
        self.step_pos += 1
        self.fetched_at[m] = k
        if self.mode == oc.RECORD:
            self.trace.append(m)
        elif self.mode == oc.COMPLETE and slip != "no_order_check" and (k >= len(self.trace) or self.trace[k] != m):
            self._invalidate()
        ops = []
        need = [d for d in self._partitioned(m) if self.status[d] == oc.NOT_AVAILABLE]
        for d in need:
            self.status[d] = oc.INFLIGHT
            self.live += self.numel[d]
        if need:
            ops.append((oc.CURRENT, sorted(need)))
        for d in self._partitioned(m):
            self.status[d] = oc.AVAILABLE
        if self.mode == oc.COMPLETE and self.cfg.prefetch_bucket_size > 0:
            while self.cursor < len(self.script) and self.script[self.cursor][0] <= k:
                self.cursor += 1
            bucket, filled = [], 0
            while self.cursor < len(self.script):
                pos, d = self.script[self.cursor]
                if self.status[d] != oc.NOT_AVAILABLE:
                    if slip != "no_marks":
                        self.marked[d] = max(self.marked.get(d, -1), pos)
                    self.cursor += 1
                    continue
                n = self.numel[d]
                if slip == "bucket_overfill":
                    if bucket and filled > self.cfg.prefetch_bucket_size:
                        break
                elif bucket and filled + n > self.cfg.prefetch_bucket_size:
                    break
                if slip == "live_limit_ge":
                    if self.live + n >= self.cfg.max_live_parameters:
                        break
                elif self.live + n > self.cfg.max_live_parameters:
                    break
                bucket.append(d)
                filled += n
                self.live += n
                self.status[d] = oc.INFLIGHT
                self.marked[d] = max(self.marked.get(d, -1), pos)
                self.cursor += 1
            if bucket:
                ops.append((oc.PREFETCH, sorted(bucket)))
        return ops
    return fetch


def _reused_soon_inclusive(self, d, k):
    """The using module's own size counted into the distance."""
    dist = 0
    for k2 in range(k + 1, len(self.trace)):
        m2 = self.trace[k2]
        dist += self._size(m2)
        if d in self.modules[m2]:
            return dist <= self.cfg.max_reuse_distance
        if dist > self.cfg.max_reuse_distance:
            return False
    return False


def _release_ignoring_reuse(orig):
    def release(self, m):
        saved = self.mode
        self.mode = oc.RECORD if self.mode == oc.COMPLETE else self.mode   # skips the reuse test
        try:
            return orig(self, m)
        finally:
            self.mode = saved
    return release


def _release_ignoring_marks(orig):
    def release(self, m):
        """A parameter the prefetcher marked for a later use is released anyway."""
        saved = self.marked
        self.marked = {}
        try:
            return orig(self, m)
        finally:
            self.marked = saved
    return release


def _reset_step_records_forever(self):
    """The recording step never completes the trace."""
    if self.mode == oc.INVALID or self.mode == oc.RECORD:
        self.mode = oc.RECORD
        self.trace = []
        self.script = []
    self.step_pos = 0
    self.cursor = 0
    self.marked = {}
    self.fetched_at = {}
    return self.mode


def _fnv1_bytes(data):
    """FNV-1 (multiply, then xor) instead of FNV-1a."""
    h = 14695981039346656037
    for byte in data:
        h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
        h ^= byte
    return h


def _set_coord(attr, fn):
    setattr(oc.Coordinator, attr, fn)


COORD_MUTANTS = {
    "coord_prefetch_live_limit_off_by_one": lambda n: _set_coord("fetch", _fetch_with("live_limit_ge")),
    "coord_prefetch_bucket_overfilled": lambda n: _set_coord("fetch", _fetch_with("bucket_overfill")),
    "coord_prefetch_does_not_mark_live": lambda n: _set_coord("fetch", _fetch_with("no_marks")),
    "coord_release_ignores_marks": lambda n: _set_coord("release", _release_ignoring_marks(oc.Coordinator.release)),
    "coord_no_trace_check": lambda n: _set_coord("fetch", _fetch_with("no_order_check")),
    "coord_reuse_distance_counts_user": lambda n: _set_coord("_reused_soon", _reused_soon_inclusive),
    "coord_release_ignores_reuse": lambda n: _set_coord("release", _release_ignoring_reuse(oc.Coordinator.release)),
    "coord_never_completes_trace": lambda n: _set_coord("reset_step", _reset_step_records_forever),
    "coord_fnv1_not_fnv1a": lambda n: setattr(oc, "fnv1a64_bytes", _fnv1_bytes),
}
MUTANTS.update(COORD_MUTANTS)
