"""Invariants on the device: the results do not depend on how the work is
split into calls.

* gather: one bucket of every partitioned parameter, or one bucket per
  parameter, requested in a shuffled order -> the same gathered views;
* reduce-scatter: one call per parameter in ascending ds_id, or one call of
  all parameters in a shuffled order -> the same flat gradient and the same
  fused norm partials (and so the same sum of squares);
* Adam: one sub-group over the whole shard, or one per parameter -> the same
  fp32 state and 16-bit shard, bit for bit.

Ragged sizes, padding, persistent parameters, N in {3, 8, 64}.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_state_amd as zs
from synth.gen import random_bits16, to16_host

from gpu_util import Buf16, Buf32, note, require_gpu, sync

pytestmark = pytest.mark.gpu

CASES = [  # seed, N, threshold, n_params, max numel
    (31, 3, 40, 9, 50000),
    (32, 8, 300, 12, 70001),
    (33, 64, 200, 6, 90000),
]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _case(seed, N, T, n, mx):
    rng = np.random.default_rng(seed)
    ids = [int(x) for x in rng.permutation(n) * 5 + 1]
    numels = [int(x) for x in rng.integers(1, mx + 1, n)]
    full = {d: random_bits16(seed, nm, "bf16", 0.02, 1, d) for d, nm in zip(ids, numels)}
    return rng, ids, numels, full


@pytest.mark.parametrize("case", CASES)
def test_gather_does_not_depend_on_bucketing_or_request_order(case):
    seed, N, T, n, mx = case
    rng, ids, numels, full = _case(*case)
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        part = [p.ds_id for p in L.params if not p.persistent]
        r = N - 1
        shards = [Buf16(L.shard_numel, fill=oracle.partition(L, v, full)) for v in range(N)]
        views = {}
        for label, buckets in (("one bucket", [list(rng.permutation(part))]), ("per parameter", [[d] for d in part])):
            got = {}
            for b in buckets:
                b = [int(x) for x in b]
                chunk_n, full_n = oracle.bucket_sizes(L, b)
                chunks = [Buf16(chunk_n) for _ in range(N)]
                for v in range(N):
                    zs.zs3_gather_coalesced(h, v, "bf16", zs.ZS3_PACK, b, shards[v].ptr(), chunks[v].ptr())
                fl = Buf16(full_n)
                note(f"invariance gather N={N} {label} bucket={len(b)}")
                offs = zs.zs3_gather_coalesced(h, r, "bf16", zs.ZS3_PACK | zs.ZS3_UNPACK, b, shards[r].ptr(),
                                               chunks[r].ptr(), [c.ptr() for c in chunks], fl.ptr())
                sync()
                host = fl.host()
                for d, o in zip(b, offs):
                    got[d] = host[o:o + L.slot(d).numel].copy()
            views[label] = got
        for d in part:
            assert np.array_equal(views["one bucket"][d], views["per parameter"][d]), f"ds_id {d}"
            assert np.array_equal(views["one bucket"][d], full[d]), f"ds_id {d} round trip"
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("case", CASES)
def test_reduce_scatter_and_norm_partials_do_not_depend_on_bucketing(case):
    seed, N, T, n, mx = case
    rng, ids, numels, _ = _case(*case)
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        r = N // 2
        srcs = {}
        keep = []
        for p in L.params:
            lo, hi = L.own_range(p, r)
            for v in range(N):
                g = to16_host((rng.standard_normal(max(hi - lo, 0)) * 1e-3).astype(np.float32), "bf16")
                b = Buf16(hi - lo, shift=v % 8, fill=g) if hi > lo else None
                keep.append(b)
                srcs[(p.ds_id, v)] = b.ptr() if b is not None else 0
        outs = {}
        for label, buckets in (("per parameter", [[d] for d in sorted(ids)]),
                               ("one call, shuffled", [[int(x) for x in rng.permutation(ids)]])):
            out = Buf16(L.shard_numel, fill=np.full(L.shard_numel, 0x7FC0, np.uint16))
            partials = torch.full((max(1, n_slots),), float("nan"), dtype=torch.float64, device="cuda")
            note(f"invariance reduce-scatter N={N} {label}")
            for b in buckets:
                src = [srcs[(d, v)] for d in b for v in range(N)]
                zs.zs3_reduce_scatter_local(h, r, "bf16", b, src, out.ptr(), partials)
            sumsq = torch.zeros(N + 1, dtype=torch.float64, device="cuda")
            zs.zs3_grad_norm_partials(h, r, partials, sumsq, False)
            sync()
            outs[label] = (out.host(), partials.cpu().numpy().view(np.uint64).copy(),
                           sumsq.cpu().numpy().view(np.uint64).copy())
        a, b = outs["per parameter"], outs["one call, shuffled"]
        assert np.array_equal(a[0], b[0]), "flat gradient"
        assert np.array_equal(a[1], b[1]), "norm partials"
        assert np.array_equal(a[2], b[2]), "sum of squares"
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("case", CASES)
def test_adam_does_not_depend_on_sub_groups(case):
    seed, N, T, n, mx = case
    rng, ids, numels, full = _case(*case)
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        r = 0
        shard0 = oracle.partition(L, r, full)
        grads = [random_bits16(seed * 13 + t, L.shard_numel, "bf16", 1e-3, 7) for t in range(1, 6)]
        scal = torch.tensor([0.75, 0.0], dtype=torch.float32, device="cuda")
        res = {}
        for label, groups in (("whole shard", [(0, L.shard_numel)]), ("per parameter", oracle.sub_groups(L, 1))):
            W, M, V = Buf32(L.shard_numel), Buf32(L.shard_numel), Buf32(L.shard_numel)
            S = Buf16(L.shard_numel, fill=shard0)
            zs.zs3_init_master(h, r, "bf16", 0, L.shard_numel, S.ptr(), W.ptr(), M.ptr(), V.ptr())
            note(f"invariance adam N={N} {label} groups={len(groups)}")
            for t, g in enumerate(grads, start=1):
                G = Buf16(L.shard_numel, fill=g)
                hp = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.0, "step": t}
                for b, e in groups:
                    zs.zs3_adam_step(h, r, "bf16", b, e, W.ptr(), M.ptr(), V.ptr(), G.ptr(), S.ptr(),
                                     scal.data_ptr(), scal.data_ptr() + 4, hp)
                sync()
            res[label] = [x.host().view(np.uint32 if isinstance(x, Buf32) else np.uint16).copy() for x in (W, M, V, S)]
        for name, a, b in zip(("master", "exp_avg", "exp_avg_sq", "shard"), res["whole shard"], res["per parameter"]):
            assert np.array_equal(a, b), name
    finally:
        zs.zs3_layout_destroy(h)


# ------------------------------------------------------- one launch per phase

@pytest.mark.parametrize("seed", range(30))
def test_gather_buckets_in_one_launch(seed):
    """zs3_gather_coalesced_buckets: random layouts split into random
    buckets (shuffled inside), each bucket's wire and gathered buffer at its
    own misaligned place: every packed chunk and gathered buffer equals the
    per-bucket calls' and the oracle's pack + unpack, bit for bit; canaries
    intact."""
    rng = np.random.default_rng(700 + seed)
    N = int(rng.choice([1, 2, 3, 5, 8, 16, 64]))
    T = int(rng.choice([0, 50, 500]))
    n = int(rng.integers(1, 40))
    numels = [int(rng.integers(1, 300)) if k < 0.5 else int(rng.integers(300, 60_000)) for k in rng.random(n)]
    ids = [int(x) for x in rng.choice(8 * n + 3, n, replace=False)]
    dtype = "bf16" if rng.random() < 0.5 else "fp16"
    r = int(rng.integers(0, N))
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        full = {d: random_bits16(seed, nm, dtype, 0.02, 3, d) for d, nm in zip(ids, numels)}
        shards = [oracle.partition(L, v, full) for v in range(N)]
        part = [int(x) for x in rng.permutation([p.ds_id for p in L.params if not p.persistent])]
        if not part:
            return
        cuts = sorted(set(int(x) for x in rng.integers(1, len(part) + 1, int(rng.integers(0, 6)))) | {len(part)})
        buckets, a = [], 0
        for c in cuts:
            buckets.append(part[a:c])
            a = c
        sh = Buf16(L.shard_numel, shift=int(rng.integers(0, 8)), fill=shards[r])
        tag = f"gather buckets seed={seed} N={N} {dtype} rank={r} buckets={[len(b) for b in buckets]}"
        res = {}
        for label in ("per bucket", "one launch"):
            owns, fulls, chunks, keep = [], [], [], []
            for b in buckets:
                chunk_n, full_n = oracle.bucket_sizes(L, b)
                ref_chunks = [oracle.pack(L, v, b, shards[v]) for v in range(N)]
                cb = [Buf16(chunk_n, shift=int(rng.integers(0, 8)), fill=ref_chunks[v]) for v in range(N)]
                own = Buf16(chunk_n, shift=int(rng.integers(0, 8)))
                fl = Buf16(full_n, shift=int(rng.integers(0, 8)))
                ptrs = [c.ptr() for c in cb]
                ptrs[r] = own.ptr()
                owns.append(own)
                fulls.append(fl)
                chunks.append(ptrs)
                keep.append(cb)
            note(f"{tag}: {label}")
            if label == "per bucket":
                for b, own, ptrs, fl in zip(buckets, owns, chunks, fulls):
                    zs.zs3_gather_coalesced(h, r, dtype, zs.ZS3_PACK | zs.ZS3_UNPACK, b, sh.ptr(), own.ptr(), ptrs,
                                            fl.ptr())
            else:
                zs.zs3_gather_coalesced_buckets(h, r, dtype, buckets, sh.ptr(), [o.ptr() for o in owns], chunks,
                                                [f.ptr() for f in fulls])
            sync()
            res[label] = [(o.host(), f.host()) for o, f in zip(owns, fulls)]
            for buf in owns + fulls:
                buf.check_guards()
        for bi, b in enumerate(buckets):
            ref_chunks = [oracle.pack(L, v, b, shards[v]) for v in range(N)]
            ref_full, _ = oracle.unpack(L, b, ref_chunks)
            for label in res:
                own, fl = res[label][bi]
                assert np.array_equal(own, ref_chunks[r]), f"{label}: packed chunk of bucket {bi}"
                assert np.array_equal(fl, ref_full), f"{label}: gathered bucket {bi}"
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rank", [("c2", 0), ("c3", 7), ("c1", 2)])
def test_single_launch_step_equals_per_bucket_step(name, rank):
    """A whole step with one gather launch per pass and one reduce-scatter
    launch for every gradient bucket gives the bits of the per-bucket step:
    every gathered buffer, the flat gradient, the fused norm's partial sums,
    the norm and the fp32 state and 16-bit shard after two steps."""
    import bench
    from synth import get_config

    cfg = get_config(name)
    out = {}
    for single in (False, True):
        note(f"single-launch step {name} rank={rank} single={single}")
        step = bench.make_step(cfg, rank, rs_streams=3, fuse_norm=True, single_launch=single)
        try:
            bench.fill_inputs(step, cfg)
            for _ in range(2):
                step.step()
            sync()
            out[single] = {k: getattr(step, k).cpu().numpy().view(np.uint8).copy()
                           for k in ("full", "wire", "grad", "partials", "sumsq", "outs", "master", "exp_avg",
                                     "exp_avg_sq", "shard")}
        finally:
            step.destroy()
    for k in out[False]:
        assert np.array_equal(out[False][k], out[True][k]), f"{k} differs between the two launch modes"
