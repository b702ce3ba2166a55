"""Python binding of libzs3, the ZeRO-3 shard-step library for MI355X.

Argument marshalling only: every function below has the name of a C entry
point in ``include/zs3.h`` and forwards to it through ctypes.  Device
buffers may be given as torch tensors (their data pointers are passed) or as
raw integer device addresses; ``stream`` may be a ``torch.cuda.Stream``, a
raw ``hipStream_t`` integer, or ``None`` for torch's current stream.  A
non-zero status raises ``Zs3Error``.  If the shared library has not been
built, the first call raises ``RuntimeError`` -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzs3.so")

ZS3_OK = 0
ZS3_EINVAL = -1
ZS3_EDTYPE = -2
ZS3_EDUPID = -3
ZS3_ENOTFOUND = -4
ZS3_EPERSIST = -5
ZS3_EALIAS = -6
ZS3_EHIP = -7
ZS3_ENOMEM = -8

ZS3_FP16 = 1
ZS3_BF16 = 2
ZS3_PACK = 1
ZS3_UNPACK = 2
ZS3_REDUCE = 4
ZS3_GATHER_BUCKETS = 1
ZS3_REDUCE_BUCKETS = 2
ZS3_TRACE_INVALID, ZS3_TRACE_RECORD, ZS3_TRACE_COMPLETE = 0, 1, 2
ZS3_PARAM_NOT_AVAILABLE, ZS3_PARAM_INFLIGHT, ZS3_PARAM_AVAILABLE = 0, 1, 2
ZS3_GATHER_CURRENT, ZS3_GATHER_PREFETCH = 0, 1

DTYPES = {"fp16": ZS3_FP16, "bf16": ZS3_BF16}

# Every exported symbol of include/zs3.h.
EXPORTS = (
    "zs3_abi_version", "zs3_status_str", "zs3_last_error", "zs3_time_next_launch",
    "zs3_layout_create", "zs3_layout_destroy", "zs3_layout_info", "zs3_layout_totals", "zs3_layout_param_at",
    "zs3_layout_param", "zs3_layout_own_range", "zs3_plan_buckets", "zs3_sub_groups",
    "zs3_bucket_sizes", "zs3_partition", "zs3_gather_coalesced", "zs3_gather_coalesced_buckets",
    "zs3_reduce_scatter_local",
    "zs3_layout_norm_slots", "zs3_reduce_scatter_coalesced", "zs3_grad_norm", "zs3_grad_norm_partials",
    "zs3_grad_norm_partials_noalloc",
    "zs3_adam_step", "zs3_adam_step_offload", "zs3_init_master", "zs3_coord_create", "zs3_coord_destroy",
    "zs3_coord_fetch", "zs3_coord_release",
    "zs3_coord_release_all", "zs3_coord_reset_step", "zs3_coord_info", "zs3_coord_param_status",
    "zs3_coord_trace_signature",
)


class Zs3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"zs3 status {status}: {message}")
        self.status = status
        self.message = message


class zs3_coord_config(ctypes.Structure):
    _fields_ = [
        ("prefetch_bucket_size", ctypes.c_int64),
        ("max_live_parameters", ctypes.c_int64),
        ("max_reuse_distance", ctypes.c_int64),
    ]


class zs3_adam_params(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_double),
        ("beta1", ctypes.c_double),
        ("beta2", ctypes.c_double),
        ("eps", ctypes.c_double),
        ("weight_decay", ctypes.c_double),
        ("step", ctypes.c_int64),
    ]


_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_p_i64 = ctypes.POINTER(ctypes.c_int64)
_p_i32 = ctypes.POINTER(ctypes.c_int32)

_p_u64 = ctypes.POINTER(ctypes.c_uint64)

_SIGNATURES = {
    "zs3_abi_version": (_c_i32, []),
    "zs3_status_str": (ctypes.c_char_p, [_c_i32]),
    "zs3_last_error": (ctypes.c_char_p, []),
    "zs3_time_next_launch": (_c_i32, [_c_p, _c_p]),
    "zs3_layout_create": (_c_i32, [_c_i32, _c_i64, _c_i32, _p_i64, _p_i64, ctypes.POINTER(_c_p)]),
    "zs3_layout_destroy": (None, [_c_p]),
    "zs3_layout_info": (_c_i32, [_c_p, _p_i32, _p_i64, _p_i32, _p_i64, _p_i64]),
    "zs3_layout_totals": (_c_i32, [_c_p, _p_i64, _p_i64]),
    "zs3_layout_param_at": (_c_i32, [_c_p, _c_i32, _p_i64, _p_i64, _p_i64, _p_i32, _p_i64]),
    "zs3_layout_param": (_c_i32, [_c_p, _c_i64, _p_i64, _p_i64, _p_i32, _p_i64]),
    "zs3_layout_own_range": (_c_i32, [_c_p, _c_i64, _c_i32, _p_i64, _p_i64]),
    "zs3_plan_buckets": (_c_i32, [_c_p, _c_i32, _c_i64, _c_i32, _p_i32, _p_i32, _p_i64]),
    "zs3_sub_groups": (_c_i32, [_c_p, _c_i64, _c_i32, _p_i32, _p_i64]),
    "zs3_bucket_sizes": (_c_i32, [_c_p, _c_i32, _p_i64, _p_i64, _p_i64]),
    "zs3_partition": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _p_i64, ctypes.POINTER(_c_p), _c_p, _c_p]),
    "zs3_gather_coalesced": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _p_i64, _c_p, _c_p,
                                      ctypes.POINTER(_c_p), _c_p, _p_i64, _c_p]),
    "zs3_gather_coalesced_buckets": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _p_i32, _p_i64, _c_p,
                                              ctypes.POINTER(_c_p), ctypes.POINTER(_c_p), ctypes.POINTER(_c_p), _c_p]),
    "zs3_reduce_scatter_local": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _p_i64, ctypes.POINTER(_c_p),
                                          _c_p, _c_p, _c_p]),
    "zs3_layout_norm_slots": (_c_i32, [_c_p, _p_i64, _p_i64]),
    "zs3_reduce_scatter_coalesced": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i32, _c_i32, _p_i64, ctypes.POINTER(_c_p),
                                              _c_p, ctypes.POINTER(_c_p), _c_p, _c_p, _c_p]),
    "zs3_grad_norm_partials": (_c_i32, [_c_p, _c_i32, _c_p, _c_p, _c_i32, ctypes.c_double, ctypes.c_double,
                                        _c_p, _c_p, _c_p, _c_p]),
    "zs3_grad_norm_partials_noalloc": (_c_i32, [_c_p, _c_i32, _c_p, _c_p, _c_i32, ctypes.c_double, ctypes.c_double,
                                                _c_p, _c_p, _c_p, _c_p]),
    "zs3_grad_norm": (_c_i32, [_c_p, _c_i32, _c_i32, _c_p, _c_p, _c_i32, ctypes.c_double,
                               ctypes.c_double, _c_p, _c_p, _c_p, _c_p]),
    "zs3_adam_step": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                               _c_p, _c_p, ctypes.POINTER(zs3_adam_params), _c_p]),
    "zs3_adam_step_offload": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                       _c_p, _c_p, _c_p, _c_p, ctypes.POINTER(zs3_adam_params), _c_p, _c_p, _c_p]),
    "zs3_init_master": (_c_i32, [_c_p, _c_i32, _c_i32, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "zs3_coord_create": (_c_i32, [_c_p, _c_i32, _p_i32, _p_i64, ctypes.POINTER(zs3_coord_config),
                                  ctypes.POINTER(_c_p)]),
    "zs3_coord_destroy": (None, [_c_p]),
    "zs3_coord_fetch": (_c_i32, [_c_p, _c_i32, _p_i32, _p_i32, _p_i32, _p_i64]),
    "zs3_coord_release": (_c_i32, [_c_p, _c_i32, _p_i32, _p_i64]),
    "zs3_coord_release_all": (_c_i32, [_c_p, _p_i32, _p_i64]),
    "zs3_coord_reset_step": (_c_i32, [_c_p, _p_i32]),
    "zs3_coord_info": (_c_i32, [_c_p, _p_i32, _p_i64, _p_i32, _p_i32]),
    "zs3_coord_param_status": (_c_i32, [_c_p, _c_i64, _p_i32]),
    "zs3_coord_trace_signature": (_c_i32, [_c_p, _p_u64, _p_u64, _p_i32]),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libzs3.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m zero_sharded_state_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


# ------------------------------------------------------------- marshalling

def _check(status: int) -> None:
    if status != ZS3_OK:
        raise Zs3Error(status, lib().zs3_last_error().decode(errors="replace"))


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _i64s(vals: Sequence[int]):
    arr = (ctypes.c_int64 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


def _ptrs(vals: Sequence) -> ctypes.Array:
    return (ctypes.c_void_p * max(1, len(vals)))(*[_ptr(v) for v in vals])


def _dtype(d) -> int:
    return DTYPES[d] if isinstance(d, str) else int(d)


def _hp(hp) -> zs3_adam_params:
    if isinstance(hp, zs3_adam_params):
        return hp
    if isinstance(hp, dict):
        return zs3_adam_params(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp.get("weight_decay", 0.0),
                               int(hp["step"]))
    return zs3_adam_params(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, int(hp.step))


# ------------------------------------------------------------------- calls

def zs3_abi_version() -> int:
    return lib().zs3_abi_version()


def zs3_status_str(status: int) -> str:
    return lib().zs3_status_str(status).decode()


def zs3_last_error() -> str:
    return lib().zs3_last_error().decode(errors="replace")


def zs3_time_next_launch(start_event, stop_event) -> None:
    """The calling thread's next zs3 kernel launch records its start/end
    timestamps into these hipEvent_t handles (integers)."""
    _check(lib().zs3_time_next_launch(start_event, stop_event))


def zs3_layout_create(world_size: int, persistence_threshold: int, ds_ids: Sequence[int],
                      numels: Sequence[int]) -> int:
    h = ctypes.c_void_p()
    _check(lib().zs3_layout_create(world_size, int(persistence_threshold), len(ds_ids), _i64s(ds_ids),
                                   _i64s(numels), ctypes.byref(h)))
    return h.value


def zs3_layout_destroy(layout: int) -> None:
    lib().zs3_layout_destroy(layout)


def zs3_layout_info(layout: int) -> dict:
    w, np_ = ctypes.c_int32(), ctypes.c_int32()
    t, s, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zs3_layout_info(layout, ctypes.byref(w), ctypes.byref(t), ctypes.byref(np_),
                                 ctypes.byref(s), ctypes.byref(b)))
    return {"world_size": w.value, "persistence_threshold": t.value, "n_params": np_.value,
            "shard_numel": s.value, "bytes_per_rank": b.value}


def zs3_layout_totals(layout: int) -> Tuple[int, int]:
    """(shard_numel, bytes_per_rank)."""
    s, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zs3_layout_totals(layout, ctypes.byref(s), ctypes.byref(b)))
    return s.value, b.value


def zs3_layout_param_at(layout: int, index: int) -> dict:
    d, n, ps, off = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    pers = ctypes.c_int32()
    _check(lib().zs3_layout_param_at(layout, index, ctypes.byref(d), ctypes.byref(n), ctypes.byref(ps),
                                     ctypes.byref(pers), ctypes.byref(off)))
    return {"ds_id": d.value, "numel": n.value, "partition_size": ps.value, "persistent": bool(pers.value),
            "shard_offset": off.value}


def zs3_layout_param(layout: int, ds_id: int) -> dict:
    n, ps, off = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    pers = ctypes.c_int32()
    _check(lib().zs3_layout_param(layout, ds_id, ctypes.byref(n), ctypes.byref(ps), ctypes.byref(pers),
                                  ctypes.byref(off)))
    return {"ds_id": ds_id, "numel": n.value, "partition_size": ps.value, "persistent": bool(pers.value),
            "shard_offset": off.value}


def zs3_layout_own_range(layout: int, ds_id: int, rank: int) -> Tuple[int, int]:
    lo, hi = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zs3_layout_own_range(layout, ds_id, rank, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def zs3_plan_buckets(layout: int, kind: int, limit: int) -> List[List[int]]:
    n_params = zs3_layout_info(layout)["n_params"]
    cap = n_params + 1
    nb = ctypes.c_int32()
    starts = (ctypes.c_int32 * cap)()
    ids = (ctypes.c_int64 * max(1, n_params))()
    _check(lib().zs3_plan_buckets(layout, kind, int(limit), cap, ctypes.byref(nb), starts, ids))
    return [list(ids[starts[b]:starts[b + 1]]) for b in range(nb.value)]


def zs3_sub_groups(layout: int, sub_group_size: int) -> List[Tuple[int, int]]:
    cap = max(1, zs3_layout_info(layout)["n_params"])
    ng = ctypes.c_int32()
    be = (ctypes.c_int64 * (2 * cap))()
    _check(lib().zs3_sub_groups(layout, int(sub_group_size), cap, ctypes.byref(ng), be))
    return [(be[2 * g], be[2 * g + 1]) for g in range(ng.value)]


def zs3_bucket_sizes(layout: int, ds_ids: Sequence[int]) -> Tuple[int, int]:
    c, f = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zs3_bucket_sizes(layout, len(ds_ids), _i64s(ds_ids), ctypes.byref(c), ctypes.byref(f)))
    return c.value, f.value


def zs3_partition(layout: int, rank: int, dtype, ds_ids: Sequence[int], full_params: Sequence,
                  shard_flat, stream=None) -> None:
    _check(lib().zs3_partition(layout, rank, _dtype(dtype), len(ds_ids), _i64s(ds_ids), _ptrs(full_params),
                               _ptr(shard_flat), _stream(stream)))


def zs3_gather_coalesced(layout: int, rank: int, dtype, mode: int, ds_ids: Sequence[int], shard_flat=None,
                         own_chunk=None, rank_chunks: Optional[Sequence] = None, full_flat=None,
                         stream=None) -> List[int]:
    n = len(ds_ids)
    offs = (ctypes.c_int64 * max(1, n))()
    chunks = _ptrs(rank_chunks) if rank_chunks is not None else None
    _check(lib().zs3_gather_coalesced(layout, rank, _dtype(dtype), mode, n, _i64s(ds_ids), _ptr(shard_flat),
                                      _ptr(own_chunk), chunks, _ptr(full_flat), offs, _stream(stream)))
    return list(offs[:n])


def zs3_gather_coalesced_buckets(layout: int, rank: int, dtype, buckets: Sequence[Sequence[int]], shard_flat,
                                 own_chunks: Sequence, rank_chunks: Sequence[Sequence], full_flats: Sequence,
                                 stream=None) -> None:
    """buckets[b] = ds_ids of bucket b; rank_chunks[b] = its N chunk pointers."""
    starts = [0]
    flat: List[int] = []
    for b in buckets:
        flat += [int(d) for d in b]
        starts.append(len(flat))
    chunks = [c for per in rank_chunks for c in per]
    _check(lib().zs3_gather_coalesced_buckets(layout, rank, _dtype(dtype), len(buckets),
                                              (ctypes.c_int32 * len(starts))(*starts), _i64s(flat), _ptr(shard_flat),
                                              _ptrs(own_chunks), _ptrs(chunks), _ptrs(full_flats), _stream(stream)))


def zs3_reduce_scatter_local(layout: int, rank: int, dtype, ds_ids: Sequence[int], src: Sequence,
                             grad_flat, partials=None, stream=None) -> None:
    _check(lib().zs3_reduce_scatter_local(layout, rank, _dtype(dtype), len(ds_ids), _i64s(ds_ids), _ptrs(src),
                                          _ptr(grad_flat), _ptr(partials), _stream(stream)))


def zs3_layout_norm_slots(layout: int) -> Tuple[int, int]:
    """(n_slots, n_part_slots) of the layout's norm slot array."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().zs3_layout_norm_slots(layout, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def zs3_reduce_scatter_coalesced(layout: int, rank: int, dtype, mode: int, ds_ids: Sequence[int],
                                 grads: Optional[Sequence] = None, send=None,
                                 recv_chunks: Optional[Sequence] = None, grad_flat=None, partials=None,
                                 stream=None) -> None:
    g = _ptrs(grads) if grads is not None else None
    r = _ptrs(recv_chunks) if recv_chunks is not None else None
    _check(lib().zs3_reduce_scatter_coalesced(layout, rank, _dtype(dtype), mode, len(ds_ids), _i64s(ds_ids), g,
                                              _ptr(send), r, _ptr(grad_flat), _ptr(partials), _stream(stream)))


def zs3_grad_norm(layout: int, rank: int, dtype, grad_flat, sumsq, finalize: bool, max_norm: float = 1.0,
                  loss_scale: float = 1.0, norm_out=None, scale_out=None, nonfinite=None, stream=None) -> None:
    _check(lib().zs3_grad_norm(layout, rank, _dtype(dtype), _ptr(grad_flat), _ptr(sumsq), int(bool(finalize)),
                               float(max_norm), float(loss_scale), _ptr(norm_out), _ptr(scale_out),
                               _ptr(nonfinite), _stream(stream)))


def zs3_grad_norm_partials(layout: int, rank: int, partials, sumsq, finalize: bool, max_norm: float = 1.0,
                           loss_scale: float = 1.0, norm_out=None, scale_out=None, nonfinite=None,
                           stream=None) -> None:
    _check(lib().zs3_grad_norm_partials(layout, rank, _ptr(partials), _ptr(sumsq), int(bool(finalize)),
                                        float(max_norm), float(loss_scale), _ptr(norm_out), _ptr(scale_out),
                                        _ptr(nonfinite), _stream(stream)))


def zs3_grad_norm_partials_noalloc(layout: int, rank: int, partials, sumsq, finalize: bool, max_norm: float = 1.0,
                                   loss_scale: float = 1.0, norm_out=None, scale_out=None, nonfinite=None,
                                   stream=None) -> None:
    _check(lib().zs3_grad_norm_partials_noalloc(layout, rank, _ptr(partials), _ptr(sumsq), int(bool(finalize)),
                                                float(max_norm), float(loss_scale), _ptr(norm_out), _ptr(scale_out),
                                                _ptr(nonfinite), _stream(stream)))


def zs3_adam_step(layout: int, rank: int, dtype, begin: int, end: int, master, exp_avg, exp_avg_sq, grad_flat,
                  shard_flat, scale, nonfinite, hp, stream=None) -> None:
    p = _hp(hp)
    _check(lib().zs3_adam_step(layout, rank, _dtype(dtype), int(begin), int(end), _ptr(master), _ptr(exp_avg),
                               _ptr(exp_avg_sq), _ptr(grad_flat), _ptr(shard_flat), _ptr(scale), _ptr(nonfinite),
                               ctypes.byref(p), _stream(stream)))


def zs3_adam_step_offload(layout: int, rank: int, dtype, begin: int, end: int, host_master, host_exp_avg,
                          host_exp_avg_sq, stage, stage_elems: int, grad_flat, shard_flat, scale, nonfinite, hp,
                          stream=None, copy_in_stream=None, copy_out_stream=None) -> None:
    p = _hp(hp)
    _check(lib().zs3_adam_step_offload(layout, rank, _dtype(dtype), int(begin), int(end), _ptr(host_master),
                                       _ptr(host_exp_avg), _ptr(host_exp_avg_sq), _ptr(stage), int(stage_elems),
                                       _ptr(grad_flat), _ptr(shard_flat), _ptr(scale), _ptr(nonfinite),
                                       ctypes.byref(p), _stream(stream),
                                       _stream(copy_in_stream) if copy_in_stream is not None else None,
                                       _stream(copy_out_stream) if copy_out_stream is not None else None))


def zs3_init_master(layout: int, rank: int, dtype, begin: int, end: int, shard_flat, master, exp_avg=None,
                    exp_avg_sq=None, stream=None) -> None:
    _check(lib().zs3_init_master(layout, rank, _dtype(dtype), int(begin), int(end), _ptr(shard_flat), _ptr(master),
                                 _ptr(exp_avg), _ptr(exp_avg_sq), _stream(stream)))


# ------------------------------------------------------------- coordinator

_coord_cap = {}


def _coord_cfg(cfg) -> zs3_coord_config:
    if isinstance(cfg, zs3_coord_config):
        return cfg
    if isinstance(cfg, dict):
        return zs3_coord_config(int(cfg["prefetch_bucket_size"]), int(cfg["max_live_parameters"]),
                                int(cfg["max_reuse_distance"]))
    return zs3_coord_config(int(cfg.prefetch_bucket_size), int(cfg.max_live_parameters), int(cfg.max_reuse_distance))


def zs3_coord_create(layout: int, modules: Sequence[Sequence[int]], cfg) -> int:
    """modules[m] = the ds_ids module m owns."""
    starts = [0]
    flat: List[int] = []
    for m in modules:
        flat += [int(d) for d in m]
        starts.append(len(flat))
    h = ctypes.c_void_p()
    c = _coord_cfg(cfg)
    _check(lib().zs3_coord_create(layout, len(modules), (ctypes.c_int32 * len(starts))(*starts), _i64s(flat),
                                  ctypes.byref(c), ctypes.byref(h)))
    _coord_cap[h.value] = max(1, len(flat))
    return h.value


def zs3_coord_destroy(coord: int) -> None:
    _coord_cap.pop(coord, None)
    lib().zs3_coord_destroy(coord)


def zs3_coord_fetch(coord: int, module: int) -> List[Tuple[int, List[int]]]:
    """[(kind, ds_ids), ...]: the gathers to issue, in order."""
    n = ctypes.c_int32()
    kinds = (ctypes.c_int32 * 2)()
    starts = (ctypes.c_int32 * 3)()
    ids = (ctypes.c_int64 * _coord_cap[coord])()
    _check(lib().zs3_coord_fetch(coord, module, ctypes.byref(n), kinds, starts, ids))
    return [(kinds[g], list(ids[starts[g]:starts[g + 1]])) for g in range(n.value)]


def zs3_coord_release(coord: int, module: int) -> List[int]:
    n = ctypes.c_int32()
    ids = (ctypes.c_int64 * _coord_cap[coord])()
    _check(lib().zs3_coord_release(coord, module, ctypes.byref(n), ids))
    return list(ids[:n.value])


def zs3_coord_release_all(coord: int) -> List[int]:
    n = ctypes.c_int32()
    ids = (ctypes.c_int64 * _coord_cap[coord])()
    _check(lib().zs3_coord_release_all(coord, ctypes.byref(n), ids))
    return list(ids[:n.value])


def zs3_coord_reset_step(coord: int) -> int:
    m = ctypes.c_int32()
    _check(lib().zs3_coord_reset_step(coord, ctypes.byref(m)))
    return m.value


def zs3_coord_info(coord: int) -> dict:
    m, t, inv = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    live = ctypes.c_int64()
    _check(lib().zs3_coord_info(coord, ctypes.byref(m), ctypes.byref(live), ctypes.byref(t), ctypes.byref(inv)))
    return {"mode": m.value, "live_numel": live.value, "trace_len": t.value, "invalidations": inv.value}


def zs3_coord_param_status(coord: int, ds_id: int) -> int:
    st = ctypes.c_int32()
    _check(lib().zs3_coord_param_status(coord, int(ds_id), ctypes.byref(st)))
    return st.value


def zs3_coord_trace_signature(coord: int) -> Tuple[int, int, int]:
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    n = ctypes.c_int32()
    _check(lib().zs3_coord_trace_signature(coord, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)))
    return a.value, b.value, n.value
