"""GPU parity on seeded random layouts: each case draws a world size (1 to
64; 128 to 1000 in a few more), a persistence threshold, up to 16 parameters with ragged sizes (mostly
tiny, some spanning many workgroup pieces), a dtype, a rank, base-pointer
misalignments and bucket limits, then runs the whole chain through the C
ABI -- partition, fused gather of every gather bucket (shuffled requests),
slice-only reduce-scatter of every reduce bucket, the norm (the other
ranks' partial sums filled in from the oracle), two Adam steps on the
reduced gradient -- and compares every output with the oracle: bit-exact
for the 16-bit outputs and the fp32 state, 1e-12 for the norm's sums.  More
random layouts take the non-contiguous gradient path with the fused norm,
and Adam on state held in pinned host memory."""

import numpy as np
import pytest

import oracle
import zero_sharded_state_amd as zs
from synth.gen import random_bits16

from gpu_util import Buf16, Buf32, note, require_gpu, sync

pytestmark = pytest.mark.gpu

WORLD = [1, 2, 3, 4, 5, 7, 8, 13, 16, 31, 64]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _case(seed):
    rng = np.random.default_rng(10_000 + seed)
    N = int(rng.choice(WORLD))
    T = int(rng.choice([0, 10, 100, 1000]))
    n = int(rng.integers(1, 17))
    kind = rng.random(n)
    numels = [int(rng.integers(1, 300)) if k < 0.6 else int(rng.integers(300, 20_000)) if k < 0.9
              else int(rng.integers(20_000, 120_000)) for k in kind]
    ids = [int(x) for x in rng.choice(10 * n + 5, n, replace=False)]
    dtype = "bf16" if rng.random() < 0.5 else "fp16"
    r = int(rng.integers(0, N))
    shifts = [int(x) for x in rng.integers(0, 8, 6)]
    return rng, N, T, ids, numels, dtype, r, shifts


@pytest.mark.parametrize("seed", range(200))
def test_random_layout_chain(seed):
    _chain(seed, *_case(seed))


def _large_world_case(seed):
    """Many ranks (128 to 1000): every parameter split over more ranks than
    it has elements in places (ranks holding only padding), the gathers'
    and reduce-scatter's work lists far past what fits in kernel arguments."""
    rng = np.random.default_rng(40_000 + seed)
    N = int(rng.choice([128, 256, 1000]))
    T = int(rng.choice([0, 50]))
    n = int(rng.integers(1, 7))
    numels = [int(rng.integers(1, 200)) if k < 0.4 else int(rng.integers(200, 6000)) for k in rng.random(n)]
    ids = [int(x) for x in rng.choice(10 * n + 5, n, replace=False)]
    dtype = "bf16" if rng.random() < 0.5 else "fp16"
    r = int(rng.choice([0, N - 1, int(rng.integers(0, N))]))
    shifts = [int(x) for x in rng.integers(0, 8, 6)]
    return rng, N, T, ids, numels, dtype, r, shifts


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", range(6))
def test_large_world_chain(seed):
    _chain(1000 + seed, *_large_world_case(seed))


def _chain(seed, rng, N, T, ids, numels, dtype, r, sh):
    import torch
    tag = f"random seed={seed} N={N} T={T} params={len(ids)} {dtype} rank={r}"
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        S = L.shard_numel
        full = {d: random_bits16(seed, nm, dtype, 0.02, 1, d) for d, nm in zip(ids, numels)}

        # partition
        note(f"{tag}: partition")
        srcs = {d: Buf16(full[d].size, shift=(d + sh[0]) % 8, fill=full[d]) for d in ids}
        order = [int(x) for x in rng.permutation(ids)]
        shard = Buf16(S, shift=sh[1], fill=np.full(S, 0x7777, np.uint16))
        zs.zs3_partition(h, r, dtype, order, [srcs[d].ptr() for d in order], shard.ptr())
        sync()
        ref_shard = oracle.partition(L, r, full)
        assert np.array_equal(shard.host(), ref_shard), "partition"
        shard.check_guards()

        # fused gather of every gather bucket
        shards = [oracle.partition(L, v, full) for v in range(N)]
        limit = int(rng.integers(1, sum(numels) + 2))
        for bi, bucket in enumerate(oracle.gather_buckets(L, limit)):
            chunk_n, full_n = oracle.bucket_sizes(L, bucket)
            ref_chunks = [oracle.pack(L, v, bucket, shards[v]) for v in range(N)]
            ref_full, ref_offs = oracle.unpack(L, bucket, ref_chunks)
            req = [int(x) for x in rng.permutation(bucket)]
            note(f"{tag}: gather bucket {bi} ({len(bucket)} params)")
            chunks = [Buf16(chunk_n, shift=(sh[2] + v) % 8, fill=ref_chunks[v]) for v in range(N)]
            own = Buf16(chunk_n, shift=sh[2])
            fl = Buf16(full_n, shift=sh[3])
            ptrs = [c.ptr() for c in chunks]
            ptrs[r] = own.ptr()
            offs = zs.zs3_gather_coalesced(h, r, dtype, zs.ZS3_PACK | zs.ZS3_UNPACK, req, shard.ptr(), own.ptr(),
                                           ptrs, fl.ptr())
            sync()
            assert np.array_equal(own.host(), ref_chunks[r]), f"packed chunk of bucket {bi}"
            assert np.array_equal(fl.host(), ref_full), f"gathered bucket {bi}"
            assert offs == [ref_offs[d] for d in req]
            own.check_guards()
            fl.check_guards()

        # slice-only reduce-scatter of every reduce bucket
        grads = [{d: random_bits16(seed * 97 + v, nm, dtype, 1e-3, 2, d) for d, nm in zip(ids, numels)}
                 for v in range(N)]
        rlimit = int(rng.integers(1, sum(numels) + 2))
        buckets = oracle.reduce_buckets(L, rlimit)
        ref_grad = np.zeros(S, np.uint16)
        gflat = Buf16(S, shift=sh[4], fill=np.full(S, 0x3C3C, np.uint16))
        keep = []
        for bi, b in enumerate(buckets):
            oracle.reduce_scatter(L, r, dtype, b, grads, ref_grad)
            src = []
            for d in b:
                lo, hi = L.own_range(L.slot(d), r)
                for v in range(N):
                    buf = Buf16(hi - lo, shift=(v + sh[5]) % 8, fill=grads[v][d][lo:hi]) if hi > lo else None
                    keep.append(buf)
                    src.append(buf.ptr() if buf is not None else 0)
            note(f"{tag}: reduce-scatter bucket {bi} ({len(b)} params)")
            zs.zs3_reduce_scatter_local(h, r, dtype, b, src, gflat.ptr())
        sync()
        assert np.array_equal(gflat.host(), ref_grad), "reduce-scatter"
        gflat.check_guards()
        del keep

        # norm: the other ranks' partial sums from the oracle, this rank's from the GPU
        parts = []
        for v in range(N):
            gv = ref_grad if v == r else np.zeros(S, np.uint16)
            if v != r:
                for b in buckets:
                    oracle.reduce_scatter(L, v, dtype, b, grads, gv)
            parts.append(oracle.grad_norm_partial(L, v, dtype, gv))
        max_norm = float(rng.choice([1e-3, 1.0, 1e3]))
        norm, coef, scale, bad = oracle.grad_norm_finalize([a for a, _ in parts], parts[0][1], max_norm)
        sumsq = torch.tensor([a for a, _ in parts] + [0.0], dtype=torch.float64, device="cuda")
        sumsq[r] = -1.0
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        note(f"{tag}: norm")
        zs.zs3_grad_norm(h, r, dtype, gflat.ptr(), sumsq, True, max_norm, 1.0, outs.data_ptr(),
                         outs.data_ptr() + 8, outs.data_ptr() + 12)
        sync()
        s = sumsq.cpu().numpy()
        assert s[r] == pytest.approx(parts[r][0], rel=1e-12, abs=0)
        assert s[N] == pytest.approx(parts[0][1], rel=1e-12, abs=0)
        o = outs.cpu().numpy()
        assert float(o[0]) == pytest.approx(norm, rel=1e-12, abs=1e-300)
        assert int(o[1:2].view(np.int32)[1]) == int(bad) == 0

        # the fp32 state from the library's init of the GPU shard, then two
        # Adam steps on the reduced gradient with the oracle's scale
        w, m, v_ = oracle.init_state(ref_shard, dtype)
        W, M, V = (Buf32(S, sh[i], np.full(S, 7.0, np.float32)) for i in range(3))
        note(f"{tag}: fp32 master partition")
        zs.zs3_init_master(h, r, dtype, 0, S, shard.ptr(), W.ptr(), M.ptr(), V.ptr())
        sync()
        for name, got, ref in (("master", W.host(), w), ("exp_avg", M.host(), m), ("exp_avg_sq", V.host(), v_)):
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{name} after init"
        sub = oracle.sub_groups(L, int(rng.integers(1, S + 2)))
        scal = torch.tensor([float(scale), 0.0], dtype=torch.float32, device="cuda")
        out16 = ref_shard.copy()
        for t in (1, 2):
            hp = oracle.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.0, t)
            note(f"{tag}: adam step {t} over {len(sub)} sub-groups")
            for b, e in sub:
                oracle.adam_step(L, r, dtype, b, e, w, m, v_, ref_grad, out16, scale, False, hp)
                zs.zs3_adam_step(h, r, dtype, b, e, W.ptr(), M.ptr(), V.ptr(), gflat.ptr(), shard.ptr(),
                                 scal.data_ptr(), scal.data_ptr() + 4, hp)
        sync()
        for name, got, ref in (("master", W.host(), w), ("exp_avg", M.host(), m), ("exp_avg_sq", V.host(), v_)):
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{name} not bit-exact"
        assert np.array_equal(shard.host(), out16), "16-bit shard after Adam"
        for b in (W, M, V, shard):
            b.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("seed", range(100))
def test_random_layout_gradient_paths(seed):
    """The non-contiguous gradient path on random layouts: for every reduce
    bucket, the rank packs its own full gradients of the bucket's
    partitioned parameters into the N-chunk send buffer and reduces the N
    chunks addressed to it (its own read back from the send buffer, the
    peers' from the oracle's pack) in one call; persistent parameters take
    the contiguous call.  Both write the fused norm's partial sums into
    slots that start as NaN.  The flat gradient equals the oracle's
    reduce-scatter bit for bit, the norm its shard-aware norm."""
    import torch
    rng, N, T, ids, numels, dtype, r, sh = _case(5_000 + seed)
    tag = f"random paths seed={seed} N={N} T={T} params={len(ids)} {dtype} rank={r}"
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        S = L.shard_numel
        grads = [{d: random_bits16(seed * 89 + v, nm, dtype, 1e-3, 3, d) for d, nm in zip(ids, numels)}
                 for v in range(N)]
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        partials = torch.full((max(1, n_slots),), float("nan"), dtype=torch.float64, device="cuda")
        out = Buf16(S, shift=sh[0], fill=np.full(S, 0x2B2B, np.uint16))
        ref = np.zeros(S, np.uint16)
        buckets = oracle.reduce_buckets(L, int(rng.integers(1, sum(numels) + 2)))
        keep = []
        for bi, b in enumerate(buckets):
            oracle.reduce_scatter(L, r, dtype, b, grads, ref)
            pb = [int(x) for x in rng.permutation([d for d in b if not L.slot(d).persistent])]
            qb = [d for d in b if L.slot(d).persistent]
            if pb:
                peers = [oracle.scatter_pack(L, pb, grads[v])[r] for v in range(N)]
                C = peers[0].size
                own = {d: Buf16(L.slot(d).numel, shift=(d + sh[1]) % 8, fill=grads[r][d]) for d in pb}
                send = Buf16(N * C, shift=sh[2])
                bufs = [Buf16(C, shift=(v + sh[3]) % 8, fill=peers[v]) for v in range(N)]
                keep += [send, *own.values(), *bufs]
                recv = [x.ptr() for x in bufs]
                recv[r] = send.ptr() + 2 * r * C
                note(f"{tag}: bucket {bi} pack+reduce ({len(pb)} params)")
                zs.zs3_reduce_scatter_coalesced(h, r, dtype, zs.ZS3_PACK | zs.ZS3_REDUCE, pb,
                                                grads=[own[d].ptr() for d in pb], send=send.ptr(),
                                                recv_chunks=recv, grad_flat=out.ptr(), partials=partials.data_ptr())
            if qb:
                src = []
                for d in qb:
                    for v in range(N):
                        buf = Buf16(L.slot(d).numel, shift=(v + sh[4]) % 8, fill=grads[v][d])
                        keep.append(buf)
                        src.append(buf.ptr())
                note(f"{tag}: bucket {bi} persistent ({len(qb)} params)")
                zs.zs3_reduce_scatter_local(h, r, dtype, qb, src, out.ptr(), partials=partials.data_ptr())
        sync()
        assert np.array_equal(out.host(), ref), "flat gradient"
        out.check_guards()
        del keep
        # the norm from the fused partial sums, the other ranks' sums from the oracle
        parts = []
        for v in range(N):
            gv = ref if v == r else np.zeros(S, np.uint16)
            if v != r:
                for b in buckets:
                    oracle.reduce_scatter(L, v, dtype, b, grads, gv)
            parts.append(oracle.grad_norm_partial(L, v, dtype, gv))
        max_norm = float(rng.choice([1e-3, 1.0, 1e3]))
        norm, coef, scale, bad = oracle.grad_norm_finalize([a for a, _ in parts], parts[0][1], max_norm)
        sumsq = torch.tensor([a for a, _ in parts] + [-1.0], dtype=torch.float64, device="cuda")
        sumsq[r] = -1.0
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        note(f"{tag}: norm from the fused partials")
        zs.zs3_grad_norm_partials(h, r, partials, sumsq, True, max_norm, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                                  outs.data_ptr() + 12)
        sync()
        s = sumsq.cpu().numpy()
        assert s[r] == pytest.approx(parts[r][0], rel=1e-12, abs=0)
        assert s[N] == pytest.approx(parts[0][1], rel=1e-12, abs=0)
        o = outs.cpu().numpy()
        assert float(o[0]) == pytest.approx(norm, rel=1e-12, abs=1e-300)
        assert int(o[1:2].view(np.int32)[1]) == int(bad) == 0
        got_scale = float(o[1:2].view(np.float32)[0])
        assert abs(got_scale - float(scale)) <= float(np.spacing(np.float32(scale)))
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("seed", range(40))
def test_random_layout_offloaded_adam(seed):
    """Adam on fp32 state in pinned host memory (read through the device
    mapping, or staged through a small device buffer in chunks of a random
    size) on random layouts and sub-groups: the same bits as the device
    Adam and the oracle after two steps."""
    import torch
    rng, N, T, ids, numels, dtype, r, sh = _case(9_000 + seed)
    chunk = None if rng.random() < 0.4 else int(rng.integers(8, 70_000))
    tag = f"random offload seed={seed} N={N} params={len(ids)} {dtype} rank={r} chunk={chunk}"
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        S = L.shard_numel
        pad = oracle.padding_mask(L, r)
        shard0 = random_bits16(seed, S, dtype, 0.02, 4)
        shard0[pad] = 0
        m0 = (rng.standard_normal(S) * 1e-4).astype(np.float32)
        v0 = (rng.random(S) * 1e-7).astype(np.float32)
        m0[pad] = 0
        v0[pad] = 0
        ds = Buf16(S, shift=sh[3], fill=shard0)
        dw = Buf32(S, sh[0], np.full(S, 7.0, np.float32))
        zs.zs3_init_master(h, r, dtype, 0, S, ds.ptr(), dw.ptr())       # the master from the library
        sync()
        w0 = dw.host()
        assert np.array_equal(w0.view(np.uint32), oracle.init_state(shard0, dtype)[0].view(np.uint32))
        dm, dv = Buf32(S, sh[1], m0), Buf32(S, sh[2], v0)
        hw, hm, hv = (torch.from_numpy(x.copy()).pin_memory() for x in (w0, m0, v0))
        hs = Buf16(S, shift=sh[4], fill=shard0)
        stage = torch.full((6 * (chunk + 8),), float("nan"), dtype=torch.float32, device="cuda") if chunk else None
        scale = np.float32(rng.choice([1.0, 0.37]))
        scal = torch.tensor([float(scale), 0.0], dtype=torch.float32, device="cuda")
        cin, cout = torch.cuda.Stream(), torch.cuda.Stream()
        groups = oracle.sub_groups(L, int(rng.integers(1, S + 2)))
        ow, om, ov, osh = w0.copy(), m0.copy(), v0.copy(), shard0.copy()
        for t in (1, 2):
            g = random_bits16(seed * 13 + t, S, dtype, 1e-3, 6)
            g[pad] = 0
            gb = Buf16(S, shift=sh[5], fill=g)
            hp = oracle.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.0, t)
            note(f"{tag}: step {t} over {len(groups)} sub-groups")
            for b, e in groups:
                zs.zs3_adam_step(h, r, dtype, b, e, dw.ptr(), dm.ptr(), dv.ptr(), gb.ptr(), ds.ptr(),
                                 scal.data_ptr(), scal.data_ptr() + 4, hp)
                zs.zs3_adam_step_offload(h, r, dtype, b, e, hw, hm, hv, stage, stage.numel() if chunk else 0,
                                         gb.ptr(), hs.ptr(), scal.data_ptr(), scal.data_ptr() + 4, hp,
                                         copy_in_stream=cin, copy_out_stream=cout)
                oracle.adam_step(L, r, dtype, b, e, ow, om, ov, g, osh, scale, False, hp)
            sync()
        for name, got, dev, ref in (("master", hw, dw, ow), ("exp_avg", hm, dm, om), ("exp_avg_sq", hv, dv, ov)):
            assert np.array_equal(got.numpy().view(np.uint32), dev.host().view(np.uint32)), f"{name}: offload"
            assert np.array_equal(got.numpy().view(np.uint32), ref.view(np.uint32)), f"{name}: oracle"
        assert np.array_equal(hs.host(), ds.host()) and np.array_equal(hs.host(), osh), "16-bit shard"
        for b in (dw, dm, dv, ds, hs):
            b.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("seed", range(60))
def test_random_layout_init_master(seed):
    """zs3_init_master ([codex] 6.1: the fp32 partition made from the 16-bit
    shard) over a random sub-range of a random layout: the exact widening at
    real positions and 0 at padding (whatever the shard holds there), m and
    v zero, nothing outside the range or the buffers touched; bit-exact
    against the oracle's initial state."""
    rng, N, T, ids, numels, dtype, r, sh = _case(20_000 + seed)
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        S = L.shard_numel
        full = {d: random_bits16(seed, nm, dtype, 0.02, 8, d) for d, nm in zip(ids, numels)}
        ref_shard = oracle.partition(L, r, full)
        w, m, v = oracle.init_state(ref_shard, dtype)
        # the shard as the library's partition writes it, then garbage in its padding
        shard_in = ref_shard.copy()
        pad = oracle.padding_mask(L, r)
        shard_in[pad] = random_bits16(seed + 1, int(pad.sum()), dtype, 1.0, 9) if pad.any() else shard_in[pad]
        a, b = sorted(int(x) for x in rng.integers(0, S + 1, 2))
        if rng.random() < 0.3:
            a, b = 0, S
        tag = f"init master seed={seed} N={N} params={len(ids)} {dtype} rank={r} range=[{a}, {b}) of {S}"
        sb = Buf16(S, shift=sh[0], fill=shard_in)
        fill = np.full(S, 7.0, np.float32)
        W, M, V = Buf32(S, sh[1], fill), Buf32(S, sh[2], fill), Buf32(S, sh[3], fill)
        note(tag)
        zs.zs3_init_master(h, r, dtype, a, b, sb.ptr(), W.ptr(), M.ptr(), V.ptr())
        sync()
        for name, got, ref in (("master", W.host(), w), ("exp_avg", M.host(), m), ("exp_avg_sq", V.host(), v)):
            assert np.array_equal(got[a:b].view(np.uint32), ref[a:b].view(np.uint32)), f"{name} inside the range"
            assert np.all(got[:a] == 7.0) and np.all(got[b:] == 7.0), f"{name} outside the range"
        assert np.array_equal(sb.host(), shard_in), "the shard is read only"
        for buf in (W, M, V, sb):
            buf.check_guards()
        # NULL moments: only the master is written
        W2, M2 = Buf32(S, sh[4], fill), Buf32(S, sh[5], fill)
        zs.zs3_init_master(h, r, dtype, 0, S, sb.ptr(), W2.ptr(), None, None)
        sync()
        assert np.array_equal(W2.host().view(np.uint32), w.view(np.uint32))
        assert np.all(M2.host() == 7.0)
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("seed", range(40))
def test_random_layout_wide_reduce_scatter(seed):
    """Many ranks (16 to 100) with every source co-aligned with its
    destination modulo 16 bytes (the layout the wide reduce-scatter kernel
    takes): random ragged layouts and buckets, both gradient paths, the
    fused norm's slots pre-filled with NaN.  The flat gradient equals the
    oracle's reduce-scatter bit for bit and the partial sums of squares its
    shard-aware partials within 1e-12."""
    import torch
    rng = np.random.default_rng(30_000 + seed)
    N = int(rng.choice([16, 17, 31, 64, 64, 100]))
    T = int(rng.choice([0, 100, 5000]))
    n = int(rng.integers(1, 12))
    numels = [int(rng.integers(1, 3000)) if k < 0.4 else int(rng.integers(3000, 400_000)) if k < 0.9
              else int(rng.integers(400_000, 4_000_000)) for k in rng.random(n)]
    ids = [int(x) for x in rng.choice(6 * n + 5, n, replace=False)]
    dtype = "bf16" if rng.random() < 0.5 else "fp16"
    r = int(rng.choice([0, N - 1, int(rng.integers(0, N))]))
    path = "coalesced" if rng.random() < 0.35 else "contiguous"
    tag = f"wide reduce seed={seed} N={N} T={T} params={n} {dtype} rank={r} {path}"
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        S = L.shard_numel
        n_slots, n_part = zs.zs3_layout_norm_slots(h)
        # each virtual rank's gradients: only the slice this rank receives is
        # ever read, so only that slice is drawn (the rest stays zero)
        grads = []
        for v in range(N):
            g = {}
            for p in L.params:
                lo, hi = L.own_range(p, r)
                a = np.zeros(p.numel, np.uint16)
                if hi > lo:
                    a[lo:hi] = random_bits16(seed * 101 + v, hi - lo, dtype, 1e-3, 11, p.ds_id)
                g[p.ds_id] = a
            grads.append(g)
        shift = int(rng.integers(0, 8))
        gflat = Buf16(S, shift=shift, fill=np.full(S, 0x3C3C, np.uint16))
        partials = torch.full((n_slots,), float("nan"), dtype=torch.float64, device="cuda")
        ref = np.zeros(S, np.uint16)
        keep = []
        pers = [p.ds_id for p in L.params if p.persistent]
        part = [p.ds_id for p in L.params if not p.persistent]
        if path == "contiguous" or not part:
            # slice-only sources: rank v's slices laid out like the flat shard, stride a multiple of 8
            stride = (S + 7) // 8 * 8
            host = np.zeros(N * stride, np.uint16)
            for v in range(N):
                for p in L.params:
                    lo, hi = L.own_range(p, r)
                    host[v * stride + p.shard_offset:v * stride + p.shard_offset + hi - lo] = grads[v][p.ds_id][lo:hi]
            recv = Buf16(N * stride, shift=shift, fill=host)
            keep.append(recv)
            for bi, b in enumerate(oracle.reduce_buckets(L, int(rng.integers(1, sum(numels) + 2)))):
                oracle.reduce_scatter(L, r, dtype, b, grads, ref)
                req = [int(x) for x in rng.permutation(b)]
                src = [recv.ptr() + 2 * (v * stride + L.slot(d).shard_offset) for d in req for v in range(N)]
                note(f"{tag}: bucket {bi} ({len(b)} params)")
                zs.zs3_reduce_scatter_local(h, r, dtype, req, src, gflat.ptr(), partials)
        else:
            # the chunks each rank sends this rank, each at the address of its
            # bucket's first grad_flat position modulo 16
            if pers:
                oracle.reduce_scatter(L, r, dtype, pers, grads, ref)
                stride = (S + 7) // 8 * 8
                host = np.zeros(N * stride, np.uint16)
                for v in range(N):
                    for d in pers:
                        p = L.slot(d)
                        host[v * stride + p.shard_offset:v * stride + p.shard_offset + p.numel] = grads[v][d]
                recv = Buf16(N * stride, shift=shift, fill=host)
                keep.append(recv)
                src = [recv.ptr() + 2 * (v * stride + L.slot(d).shard_offset) for d in pers for v in range(N)]
                zs.zs3_reduce_scatter_local(h, r, dtype, pers, src, gflat.ptr(), partials)
            limit = int(rng.integers(1, sum(L.slot(d).numel for d in part) + 2))
            for bi, b in enumerate(oracle.gather_buckets(L, limit)):
                C = sum(L.slot(d).partition_size for d in b)
                chunks = []          # chunk r of every rank's send buffer (the wire of the pack)
                for v in range(N):
                    parts = []
                    for d in sorted(b):
                        p = L.slot(d)
                        lo, hi = L.own_range(p, r)
                        part = np.zeros(p.partition_size, np.uint16)
                        part[:hi - lo] = grads[v][d][lo:hi]
                        parts.append(part)
                    chunks.append(np.concatenate(parts))
                oracle.scatter_reduce(L, r, dtype, b, chunks, ref)
                first = min(L.slot(d).shard_offset for d in b)
                want = (gflat.ptr() + 2 * first) % 16
                bufs = []
                for v in range(N):
                    buf = Buf16(C + 8, shift=0)
                    off = ((want - buf.ptr() % 16) % 16) // 2
                    buf.view[off:off + C].copy_(torch.from_numpy(chunks[v].view(np.int16)).cuda())
                    bufs.append((buf, buf.ptr() + 2 * off))
                keep.append(bufs)
                req = [int(x) for x in rng.permutation(b)]
                note(f"{tag}: coalesced bucket {bi} ({len(b)} params)")
                zs.zs3_reduce_scatter_coalesced(h, r, dtype, zs.ZS3_REDUCE, req, recv_chunks=[p for _, p in bufs],
                                                grad_flat=gflat.ptr(), partials=partials)
        sync()
        assert np.array_equal(gflat.host(), ref), "flat gradient"
        gflat.check_guards()
        sumsq = torch.zeros(N + 1, dtype=torch.float64, device="cuda")
        zs.zs3_grad_norm_partials(h, r, partials, sumsq, False)
        sync()
        a, q = oracle.grad_norm_partial(L, r, dtype, ref)
        s = sumsq.cpu().numpy()
        assert s[r] == pytest.approx(a, rel=1e-12, abs=0), "partitioned sum of squares"
        assert s[N] == pytest.approx(q, rel=1e-12, abs=0), "persistent sum of squares"
        del keep
    finally:
        zs.zs3_layout_destroy(h)
