"""The library's aliasing checks against a brute-force pairwise test (host
logic, no GPU).

zs3_reduce_scatter_local and zs3_gather_coalesced_buckets reject a call in
which a range they write overlaps any other range of the call (a source,
another output) with ZS3_EALIAS, using one sort-and-sweep over every byte
range.  Here the buffers are fake addresses in an empty address space,
drawn so that about half of the calls overlap somewhere (a source placed
inside a written range, two outputs that touch, a source inside the norm
partials); the expected answer comes from testing every pair of ranges.
A call that passes the checks goes on to allocate or launch, which fails
without a GPU (ZS3_EHIP or ZS3_ENOMEM), so nothing ever runs on a device:
the test runs only where no device is visible.
"""

import ctypes

import numpy as np
import pytest

import zero_sharded_state_amd as zs

I64, P = ctypes.c_int64, ctypes.c_void_p
BF16 = zs.DTYPES["bf16"]
BASE = 1 << 40


@pytest.fixture(scope="module", autouse=True)
def _no_device():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("fake addresses must never reach a device: host-only test")
    zs.lib()


def _overlap_pairs(ranges):
    """True if a written range overlaps any other non-empty range (every pair)."""
    for i, (a0, a1, wa) in enumerate(ranges):
        if a1 <= a0:
            continue
        for j, (b0, b1, wb) in enumerate(ranges):
            if j <= i or b1 <= b0 or not (wa or wb):
                continue
            if a0 < b1 and b0 < a1:
                return True
    return False


def _layout(rng):
    N = int(rng.integers(1, 10))
    n = int(rng.integers(1, 9))
    T = int(rng.choice([0, 40]))
    numels = [int(rng.integers(1, 60)) if k < 0.3 else int(rng.integers(60, 5000)) for k in rng.random(n)]
    ids = [int(x) for x in rng.choice(4 * n + 3, n, replace=False)]
    return N, T, ids, numels


def _params(h, ids):
    info = {}
    for i in range(len(ids)):
        p = zs.zs3_layout_param_at(h, i)
        info[p["ds_id"]] = p
    return info


@pytest.mark.parametrize("seed", range(150))
def test_reduce_scatter_alias_check_matches_pairwise(seed):
    rng = np.random.default_rng(4000 + seed)
    N, T, ids, numels = _layout(rng)
    h = zs.zs3_layout_create(N, T, ids, numels)
    try:
        info = _params(h, ids)
        rank = int(rng.integers(0, N))
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        grad = BASE + 2 * int(rng.integers(0, 1 << 16))
        partials = BASE + (1 << 30) + 8 * int(rng.integers(0, 1 << 12))
        call = [d for d in ids if rng.random() < 0.8] or [ids[0]]
        rng.shuffle(call)
        ranges = [(partials, partials + 8 * n_slots, True)]
        written = []
        for d in call:
            p = info[d]
            w0 = grad + 2 * p["shard_offset"]
            ranges.append((w0, w0 + 2 * p["partition_size"], True))
            written.append((w0, w0 + 2 * p["partition_size"]))
        src = []
        aliased = rng.random() < 0.5
        for d in call:
            lo, hi = zs.zs3_layout_own_range(h, d, rank)
            real = hi - lo
            for v in range(N):
                # sources far from everything, except, sometimes, one placed
                # at or near a written range (partials included)
                a = BASE + (1 << 33) + 2 * int(rng.integers(0, 1 << 28))
                if aliased and rng.random() < 0.15:
                    tgt = written[int(rng.integers(0, len(written)))] if rng.random() < 0.8 else \
                        (partials, partials + 8 * n_slots)
                    a = tgt[0] + 2 * int(rng.integers(-max(1, real), (tgt[1] - tgt[0]) // 2 + 2))
                    a = max(BASE, a)
                src.append(a)
                if real > 0:
                    ranges.append((a, a + 2 * real, False))
        want = _overlap_pairs(ranges)
        st = zs.lib().zs3_reduce_scatter_local(h, rank, BF16, len(call), (I64 * len(call))(*call),
                                               (P * len(src))(*src), grad, partials, None)
        msg = zs.zs3_last_error()
        if want:
            assert st == zs.ZS3_EALIAS, (st, msg)
        else:
            assert st in (zs.ZS3_EHIP, zs.ZS3_ENOMEM), (st, msg)
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("seed", range(150))
def test_gather_buckets_alias_check_matches_pairwise(seed):
    rng = np.random.default_rng(5000 + seed)
    N, T, ids, numels = _layout(rng)
    h = zs.zs3_layout_create(N, T, ids, numels)
    try:
        info = _params(h, ids)
        part = [d for d in ids if not info[d]["persistent"]]
        if not part:
            pytest.skip("every parameter is persistent")
        rank = int(rng.integers(0, N))
        rng.shuffle(part)
        nb = int(rng.integers(1, len(part) + 1))
        cuts = sorted(int(x) for x in rng.choice(np.arange(1, len(part)), nb - 1, replace=False)) if nb > 1 else []
        buckets = [part[a:b] for a, b in zip([0] + cuts, cuts + [len(part)])]
        S = sum(p["partition_size"] for p in info.values())
        shard = BASE + 2 * int(rng.integers(0, 1 << 16))
        ranges = [(shard, shard + 2 * S, False)]
        aliased = rng.random() < 0.5
        outs = []            # (own_chunk, full) per bucket
        others = []          # per bucket, N chunk pointers
        placed = []
        for b in buckets:
            chunk = sum(info[d]["partition_size"] for d in b)
            full = sum(info[d]["numel"] for d in b)

            def pick(nbytes):
                a = BASE + (1 << 34) + 16 * int(rng.integers(0, 1 << 27))
                if aliased and placed and rng.random() < 0.12:
                    t0, t1 = placed[int(rng.integers(0, len(placed)))]
                    a = max(BASE, t0 + 2 * int(rng.integers(-(nbytes // 2), (t1 - t0) // 2 + 2)))
                placed.append((a, a + nbytes))
                return a

            own = pick(2 * chunk)
            fl = pick(2 * full)
            ranges += [(own, own + 2 * chunk, True), (fl, fl + 2 * full, True)]
            ch = []
            for v in range(N):
                if v == rank:
                    ch.append(own)
                    continue
                a = pick(2 * chunk)
                ch.append(a)
                ranges.append((a, a + 2 * chunk, False))
            outs.append((own, fl))
            others.append(ch)
        if aliased and rng.random() < 0.2:
            # an output inside the shard
            own, fl = outs[0]
            outs[0] = (shard + 2 * int(rng.integers(0, max(1, S))), fl)
            others[0][rank] = outs[0][0]
            chunk = sum(info[d]["partition_size"] for d in buckets[0])
            ranges = [r for r in ranges if r[0] != own or not r[2]] + [(outs[0][0], outs[0][0] + 2 * chunk, True)]
        want = _overlap_pairs(ranges)
        flat = [d for b in buckets for d in b]
        starts = [0]
        for b in buckets:
            starts.append(starts[-1] + len(b))
        st = zs.lib().zs3_gather_coalesced_buckets(
            h, rank, BF16, len(buckets), (ctypes.c_int32 * len(starts))(*starts), (I64 * len(flat))(*flat), shard,
            (P * len(buckets))(*[o for o, _ in outs]), (P * (len(buckets) * N))(*[a for ch in others for a in ch]),
            (P * len(buckets))(*[f for _, f in outs]), None)
        msg = zs.zs3_last_error()
        if want:
            assert st == zs.ZS3_EALIAS, (st, msg)
        else:
            assert st in (zs.ZS3_EHIP, zs.ZS3_ENOMEM), (st, msg)
    finally:
        zs.zs3_layout_destroy(h)
