"""GPU parity of the five entry points against the CPU oracle, on seeded
inputs that span several workgroup pieces, ragged tails, padding, every
source/destination misalignment, N from 1 to 64, and the pages' worked
example.  Every call goes through the C ABI; every output buffer is
guarded by canaries."""

import numpy as np
import pytest

import oracle
import zero_sharded_state_amd as zs
from synth import get_config
from synth.gen import grad_host, random_bits16, to16_host, weights_host

from gpu_util import Buf16, Buf32, assert_f32_close, note, ordinal16, require_gpu, sync

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _problem(seed, N, T, n_params, max_numel, dtype="bf16"):
    rng = np.random.default_rng(seed)
    ids = [int(x) for x in rng.permutation(n_params) * 7 + 2]
    numels = [int(x) for x in rng.integers(1, max_numel + 1, n_params)]
    full = {d: random_bits16(seed, n, dtype, 0.02, 1, d) for d, n in zip(ids, numels)}
    return ids, numels, full


PROBLEMS = [
    # seed, N, threshold, n_params, max numel
    (1, 1, 0, 5, 3000),
    (2, 2, 50, 9, 40000),
    (3, 3, 100, 12, 70000),
    (4, 4, 0, 7, 20011),
    (5, 8, 1000, 14, 90000),
    (6, 64, 500, 10, 60000),
    (7, 5, 0, 30, 700),
]


def _layout(ids, numels, N, T):
    return zs.zs3_layout_create(N, T, ids, numels), oracle.make_layout(N, T, ids, numels)


# --------------------------------------------------------------- partition

@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("shift", [0, 3])
def test_partition_bit_exact(prob, shift):
    seed, N, T, n, mx = prob
    ids, numels, full = _problem(seed, N, T, n, mx)
    h, L = _layout(ids, numels, N, T)
    try:
        srcs = {d: Buf16(full[d].size, shift=(d + shift) % 8, fill=full[d]) for d in ids}
        for r in sorted({0, N - 1, N // 2}):
            note(f"partition seed={seed} N={N} rank={r} shift={shift}")
            out = Buf16(L.shard_numel, shift=shift, fill=np.full(L.shard_numel, 0x7777, np.uint16))
            order = ids[::-1]
            zs.zs3_partition(h, r, "bf16", order, [srcs[d].ptr() for d in order], out.ptr())
            sync()
            assert np.array_equal(out.host(), oracle.partition(L, r, full))
            out.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


# ----------------------------------------------------------- pack / unpack

@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("shifts", [(0, 0, 0), (1, 5, 2), (7, 0, 3)])
@pytest.mark.parametrize("fused", [True, False])
def test_gather_pack_unpack_bit_exact(prob, shifts, fused):
    """fused: the wire's own slot is the pack output (one launch); otherwise
    the own slot is a separate, already-filled chunk (pack, then unpack)."""
    seed, N, T, n, mx = prob
    s_shard, s_chunk, s_full = shifts
    ids, numels, full = _problem(seed, N, T, n, mx)
    h, L = _layout(ids, numels, N, T)
    try:
        shards = [oracle.partition(L, r, full) for r in range(N)]
        limit = max(1, sum(numels) // 3)
        for bucket in oracle.gather_buckets(L, limit):
            chunk_n, full_n = oracle.bucket_sizes(L, bucket)
            req = list(np.random.default_rng(seed).permutation(bucket))
            ref_chunks = [oracle.pack(L, v, bucket, shards[v]) for v in range(N)]
            ref_full, ref_offs = oracle.unpack(L, bucket, ref_chunks)
            r = (seed * 7) % N
            note(f"gather seed={seed} N={N} rank={r} bucket={len(bucket)} params shifts={shifts} fused={fused}")
            sh = Buf16(L.shard_numel, shift=s_shard, fill=shards[r])
            chunks = [Buf16(chunk_n, shift=(s_chunk + v) % 8, fill=ref_chunks[v]) for v in range(N)]
            own = Buf16(chunk_n, shift=s_chunk)
            fl = Buf16(full_n, shift=s_full)
            rank_ptrs = [c.ptr() for c in chunks]
            if fused:
                rank_ptrs[r] = own.ptr()
            offs = zs.zs3_gather_coalesced(h, r, "bf16", zs.ZS3_PACK | zs.ZS3_UNPACK, req, sh.ptr(), own.ptr(),
                                           rank_ptrs, fl.ptr())
            sync()
            assert np.array_equal(own.host(), ref_chunks[r])
            assert np.array_equal(fl.host(), ref_full)
            assert offs == [ref_offs[d] for d in req]
            for d in bucket:
                assert np.array_equal(fl.host()[ref_offs[d]:ref_offs[d] + full[d].size], full[d])
            own.check_guards()
            fl.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


def test_partition_then_gather_round_trip_c1():
    cfg = get_config("c1")
    N = cfg.world_size
    h, L = _layout(cfg.ds_ids, cfg.numels, N, cfg.threshold)
    try:
        full = {d: weights_host(cfg, d) for d in cfg.ds_ids}
        srcs = {d: Buf16(full[d].size, fill=full[d]) for d in cfg.ds_ids}
        shards = []
        for r in range(N):
            s = Buf16(L.shard_numel)
            zs.zs3_partition(h, r, cfg.dtype, cfg.ds_ids, [srcs[d].ptr() for d in cfg.ds_ids], s.ptr())
            shards.append(s)
        chunk_n, full_n = oracle.bucket_sizes(L, cfg.ds_ids)
        chunks = [Buf16(chunk_n) for _ in range(N)]
        for r in range(N):
            zs.zs3_gather_coalesced(h, r, cfg.dtype, zs.ZS3_PACK, cfg.ds_ids, shards[r].ptr(), chunks[r].ptr())
        fl = Buf16(full_n)
        offs = zs.zs3_gather_coalesced(h, 0, cfg.dtype, zs.ZS3_UNPACK, cfg.ds_ids, None, None,
                                       [c.ptr() for c in chunks], fl.ptr())
        sync()
        got = fl.host()
        for d, o in zip(cfg.ds_ids, offs):
            assert np.array_equal(got[o:o + full[d].size], full[d])
    finally:
        zs.zs3_layout_destroy(h)


# ---------------------------------------------------------- reduce-scatter

def _rs_case(seed, N, T, n, mx, dtype, slice_only, shift):
    ids, numels, _ = _problem(seed, N, T, n, mx, dtype)
    h, L = _layout(ids, numels, N, T)
    rng = np.random.default_rng(seed + 100)
    grads = [{d: to16_host((rng.standard_normal(nm) * 1e-3).astype(np.float32), dtype)
              for d, nm in zip(ids, numels)} for _ in range(N)]
    return h, L, ids, grads


@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("slice_only,shift", [(False, 0), (True, 0), (False, 5), (True, 3)])
def test_reduce_scatter_bit_exact(prob, dtype, slice_only, shift):
    seed, N, T, n, mx = prob
    h, L, ids, grads = _rs_case(seed, N, T, n, mx, dtype, slice_only, shift)
    try:
        for r in sorted({0, N - 1}):
            ref = np.zeros(L.shard_numel, np.uint16)
            buckets = oracle.reduce_buckets(L, max(1, sum(p.numel for p in L.params) // 4))
            for b in buckets:
                oracle.reduce_scatter(L, r, dtype, b, grads, ref)
            note(f"reduce_scatter seed={seed} N={N} rank={r} {dtype} slice_only={slice_only} shift={shift}")
            out = Buf16(L.shard_numel, shift=shift, fill=np.full(L.shard_numel, 0x3C3C, np.uint16))
            keep = []
            for b in buckets:
                src = []
                for d in b:
                    p = L.slot(d)
                    lo, hi = L.own_range(p, r)
                    for v in range(N):
                        g = grads[v][d]
                        if slice_only:      # only the slice rank r receives from v
                            buf = Buf16(hi - lo, shift=(v + shift) % 8, fill=g[lo:hi]) if hi > lo else None
                            keep.append(buf)
                            src.append(buf.ptr() if buf is not None else 0)
                        else:               # v's whole gradient, pointer at element lo
                            buf = Buf16(g.size, shift=(v * 3 + shift) % 8, fill=g)
                            keep.append(buf)
                            src.append(buf.ptr() + 2 * lo)
                zs.zs3_reduce_scatter_local(h, r, dtype, b, src, out.ptr())
            sync()
            got = out.host()
            assert np.array_equal(got, ref), f"mismatch at {np.nonzero(got != ref)[0][:10]}"
            out.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


# Gradient values whose fp32 sums depend on the order of the adds (sums
# reach past 24 significant bits and round, often on ties): the kernel's
# rank-order sum must match the oracle's bit for bit.
ORDER_VALUES = {
    "bf16": [0x4B80, 0xCB80, 0x3F80, 0xBF80, 0x4B00, 0xCB00, 0x3F00, 0x4C00, 0xCC00, 0x0000, 0x8000, 0x3E80],
    "fp16": [0x7800, 0xF800, 0x1800, 0x9800, 0x3C00, 0xBC00, 0x7400, 0xF400, 0x1400, 0x0001, 0x8000, 0x6800],
}


@pytest.mark.parametrize("N", [3, 8, 9, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_reduce_scatter_order_sensitive_values(N, dtype):
    from oracle import brute
    ids, numels, T = [4, 9, 13], [3 * 32768 + 13, 40000, 999], 0
    rng = np.random.default_rng(N)
    vals = np.array(ORDER_VALUES[dtype], np.uint16)
    grads = [{d: rng.choice(vals, nm) for d, nm in zip(ids, numels)} for _ in range(N)]
    h, L = _layout(ids, numels, N, T)
    try:
        for r in sorted({0, N - 1}):
            p0 = L.slot(ids[0])
            lo, hi = L.own_range(p0, r)
            sample = [[int(grads[v][ids[0]][lo + k]) for v in range(N)] for k in range(min(200, hi - lo))]
            flips = sum(brute.reduce_scatter_elem(x, dtype) != brute.reduce_scatter_elem(x[::-1], dtype)
                        for x in sample)
            assert flips > 0, "the input does not depend on the order of the adds"
            ref = np.zeros(L.shard_numel, np.uint16)
            oracle.reduce_scatter(L, r, dtype, ids, grads, ref)
            note(f"reduce_scatter order-sensitive N={N} rank={r} {dtype}")
            out = Buf16(L.shard_numel, fill=np.full(L.shard_numel, 0x3C3C, np.uint16))
            keep, src = [], []
            for d in ids:
                lo, hi = L.own_range(L.slot(d), r)
                for v in range(N):
                    buf = Buf16(hi - lo, shift=v % 8, fill=grads[v][d][lo:hi]) if hi > lo else None
                    keep.append(buf)
                    src.append(buf.ptr() if buf is not None else 0)
            zs.zs3_reduce_scatter_local(h, r, dtype, ids, src, out.ptr())
            sync()
            got = out.host()
            assert np.array_equal(got, ref), f"mismatch at {np.nonzero(got != ref)[0][:10]}"
            out.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


def test_reduce_scatter_worked_example():
    """The csdn page's 4-GPU example: grads 0.5, 1, 1.5, 2 on every rank;
    GPU r keeps the averaged unit it owns (GPU0: 0.5)."""
    h = zs.zs3_layout_create(4, 0, [0], [4])
    try:
        g = to16_host(np.array([0.5, 1, 1.5, 2], np.float32), "fp16")
        bufs = [Buf16(4, fill=g) for _ in range(4)]
        for r in range(4):
            out = Buf16(1)
            zs.zs3_reduce_scatter_local(h, r, "fp16", [0], [b.ptr() + 2 * r for b in bufs], out.ptr())
            sync()
            assert float(oracle.to_f32(out.host(), "fp16")[0]) == [0.5, 1.0, 1.5, 2.0][r]
    finally:
        zs.zs3_layout_destroy(h)


# --------------------------------------------------------------- grad norm

@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shift", [0, 5])
def test_grad_norm(prob, dtype, shift):
    import torch
    seed, N, T, n, mx = prob
    ids, numels, _ = _problem(seed, N, T, n, mx, dtype)
    h, L = _layout(ids, numels, N, T)
    try:
        flats, parts = [], []
        for r in range(N):
            g = random_bits16(seed + r, L.shard_numel, dtype, 1e-2, 9)
            g[oracle.padding_mask(L, r)] = 0
            flats.append(g)
            parts.append(oracle.grad_norm_partial(L, r, dtype, g))
        norm, coef, scale, bad = oracle.grad_norm_finalize([a for a, _ in parts], parts[0][1], 0.5)
        sumsq = torch.zeros(N + 1, dtype=torch.float64, device="cuda")
        outs = torch.zeros(4, dtype=torch.float64, device="cuda")
        norm_p, scale_p, flag_p = outs.data_ptr(), outs.data_ptr() + 8, outs.data_ptr() + 12
        for r in range(N):
            note(f"grad_norm seed={seed} N={N} rank={r} {dtype} shift={shift}")
            gb = Buf16(L.shard_numel, shift=shift, fill=flats[r])
            zs.zs3_grad_norm(h, r, dtype, gb.ptr(), sumsq, r == N - 1, 0.5, 1.0, norm_p, scale_p, flag_p)
            sync()
        s = sumsq.cpu().numpy()
        for r in range(N):
            assert s[r] == pytest.approx(parts[r][0], rel=1e-12, abs=0)
        assert s[N] == pytest.approx(parts[0][1], rel=1e-12, abs=0)
        o = outs.cpu().numpy()
        got_norm = float(o[0])
        got_scale = float(o[1:2].view(np.float32)[0])
        got_flag = int(o[1:2].view(np.int32)[1])
        assert got_norm == pytest.approx(norm, rel=1e-5)
        assert abs(got_norm - norm) <= 1e-12 * norm
        assert got_flag == 0
        assert np.float32(got_scale) == scale or abs(got_scale - scale) <= np.spacing(np.float32(scale))
    finally:
        zs.zs3_layout_destroy(h)


def test_grad_norm_nonfinite_flag():
    import torch
    h = zs.zs3_layout_create(2, 0, [0], [5000])
    try:
        g = random_bits16(3, 2500, "fp16", 1e-2, 1)
        g[1234] = 0x7C00   # +inf
        gb = Buf16(2500, fill=g)
        sumsq = torch.zeros(3, dtype=torch.float64, device="cuda")
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        zs.zs3_grad_norm(h, 0, "fp16", gb.ptr(), sumsq, True, 1.0, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                         outs.data_ptr() + 12)
        sync()
        assert int(outs.cpu().numpy()[1:2].view(np.int32)[1]) == 1
    finally:
        zs.zs3_layout_destroy(h)


# -------------------------------------------------------------------- Adam

@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shift", [0, 1])
def test_adam_ten_steps(prob, dtype, shift):
    _adam_chain(prob, dtype, shift, 0.0)


@pytest.mark.parametrize("prob", [PROBLEMS[2], PROBLEMS[4], PROBLEMS[5]])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_adam_ten_steps_with_weight_decay(prob, dtype):
    _adam_chain(prob, dtype, 1, 0.05)


def _adam_chain(prob, dtype, shift, wd):
    import torch
    seed, N, T, n, mx = prob
    ids, numels, full = _problem(seed, N, T, n, mx, dtype)
    h, L = _layout(ids, numels, N, T)
    try:
        r = N - 1
        shard = oracle.partition(L, r, full)
        w, m, v = oracle.init_state(shard, dtype)
        # the GPU side starts from the library's partition and fp32 init
        srcs = [Buf16(full[d].size, fill=full[d]) for d in ids]
        S = Buf16(L.shard_numel, shift, np.full(L.shard_numel, 0x7777, np.uint16))
        zs.zs3_partition(h, r, dtype, ids, [b.ptr() for b in srcs], S.ptr())
        W, M, V = (Buf32(L.shard_numel, shift, np.full(L.shard_numel, 7.0, np.float32)) for _ in range(3))
        zs.zs3_init_master(h, r, dtype, 0, L.shard_numel, S.ptr(), W.ptr(), M.ptr(), V.ptr())
        sync()
        assert np.array_equal(S.host(), shard), "partition"
        for name, got, ref in (("master", W.host(), w), ("m", M.host(), m), ("v", V.host(), v)):
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{name} after init"
        pad = oracle.padding_mask(L, r)
        groups = oracle.sub_groups(L, max(1, L.shard_numel // 3))
        scal = torch.zeros(2, dtype=torch.float32, device="cuda")
        for t in range(1, 11):
            g = random_bits16(seed * 31 + t, L.shard_numel, dtype, 1e-3, 5)
            g[pad] = 0
            G = Buf16(L.shard_numel, shift, g)
            scale = np.float32(0.8 if t % 2 else 1.0)
            scal[0] = float(scale)
            hp = oracle.AdamHParams(1e-3, 0.9, 0.999, 1e-8, wd, t)
            note(f"adam seed={seed} N={N} rank={r} {dtype} shift={shift} wd={wd} step={t}")
            for b, e in groups:
                oracle.adam_step(L, r, dtype, b, e, w, m, v, g, shard, scale, False, hp)
                zs.zs3_adam_step(h, r, dtype, b, e, W.ptr(), M.ptr(), V.ptr(), G.ptr(), S.ptr(),
                                 scal.data_ptr(), scal.data_ptr() + 4, hp)
        sync()
        for name, got, ref in (("master", W.host(), w), ("m", M.host(), m), ("v", V.host(), v)):
            assert_f32_close(got, ref, 2e-6, name)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{name} not bit-exact"
        d = np.abs(ordinal16(S.host()) - ordinal16(shard))
        assert d.max() <= 1
        assert np.array_equal(S.host(), shard)
        for b in (W, M, V, S):
            b.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


def test_adam_nonfinite_flag_skips_everything():
    import torch
    h = zs.zs3_layout_create(1, 0, [0], [10000])
    try:
        w = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
        W, M, V = Buf32(10000, 0, w), Buf32(10000, 0, w * 0), Buf32(10000, 0, w * 0)
        S = Buf16(10000, 0, oracle.from_f32(w, "bf16"))
        G = Buf16(10000, 0, random_bits16(1, 10000, "bf16", 1e-3, 1))
        scal = torch.tensor([1.0], device="cuda")
        flag = torch.tensor([1], dtype=torch.int32, device="cuda")
        zs.zs3_adam_step(h, 0, "bf16", 0, 10000, W.ptr(), M.ptr(), V.ptr(), G.ptr(), S.ptr(), scal.data_ptr(),
                         flag.data_ptr(), oracle.AdamHParams(step=1))
        sync()
        assert np.array_equal(W.host(), w) and np.all(M.host() == 0) and np.all(V.host() == 0)
    finally:
        zs.zs3_layout_destroy(h)


# ------------------------------------------------------------- edge cases

def test_empty_requests_are_noops():
    h = zs.zs3_layout_create(4, 0, [0, 1], [10, 20])
    try:
        out = Buf16(8)
        zs.zs3_partition(h, 0, "bf16", [], [], out.ptr())
        assert zs.zs3_gather_coalesced(h, 0, "bf16", zs.ZS3_PACK | zs.ZS3_UNPACK, [], out.ptr(), out.ptr(),
                                       [out.ptr()] * 4, out.ptr()) == []
        zs.zs3_reduce_scatter_local(h, 0, "bf16", [], [], out.ptr())
        import torch
        st = torch.zeros(4, dtype=torch.float32, device="cuda")
        zs.zs3_adam_step(h, 0, "bf16", 3, 3, st.data_ptr(), st.data_ptr(), st.data_ptr(), out.ptr(), out.ptr(),
                         st.data_ptr(), None, oracle.AdamHParams(step=1))
        sync()
        out.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


def test_empty_layout_norm_is_zero():
    import torch
    h = zs.zs3_layout_create(2, 0, [], [])
    try:
        sumsq = torch.full((3,), 7.0, dtype=torch.float64, device="cuda")
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        g = Buf16(1)
        sumsq[1] = 4.0
        zs.zs3_grad_norm(h, 0, "fp16", g.ptr(), sumsq, True, 1.0, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                         outs.data_ptr() + 12)
        sync()
        s = sumsq.cpu().numpy()
        assert s[0] == 0.0 and s[2] == 0.0 and float(outs.cpu().numpy()[0]) == 2.0
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_ranks_holding_only_padding(dtype):
    """numel 3 over N = 8: ranks 3..7 hold only padding, and 1-element
    parameters leave every rank but 0 empty."""
    N = 8
    ids, numels = [0, 1, 2], [3, 1, 17]
    h, L = _layout(ids, numels, N, 0)
    try:
        full = {d: random_bits16(d, n, dtype, 0.5, 3) for d, n in zip(ids, numels)}
        srcs = {d: Buf16(numels[i], fill=full[d]) for i, d in enumerate(ids)}
        grads = [{d: random_bits16(10 + v, n, dtype, 0.1, d) for d, n in zip(ids, numels)} for v in range(N)]
        gbufs = [{d: Buf16(numels[i], fill=grads[v][d]) for i, d in enumerate(ids)} for v in range(N)]
        for r in range(N):
            note(f"padding-only ranks {dtype} rank={r}")
            sh = Buf16(L.shard_numel, fill=np.full(L.shard_numel, 0x1111, np.uint16))
            zs.zs3_partition(h, r, dtype, ids, [srcs[d].ptr() for d in ids], sh.ptr())
            gf = Buf16(L.shard_numel, fill=np.full(L.shard_numel, 0x2222, np.uint16))
            src = []
            for d in ids:
                lo, hi = L.own_range(L.slot(d), r)
                src += [gbufs[v][d].ptr() + 2 * lo if hi > lo else 0 for v in range(N)]
            zs.zs3_reduce_scatter_local(h, r, dtype, ids, src, gf.ptr())
            sync()
            assert np.array_equal(sh.host(), oracle.partition(L, r, full))
            ref = np.zeros(L.shard_numel, np.uint16)
            oracle.reduce_scatter(L, r, dtype, ids, grads, ref)
            assert np.array_equal(gf.host(), ref)
            sh.check_guards()
            gf.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


def test_fp16_overflow_sets_flag_and_adam_skips():
    """Averaging fp16 gradients near the top of the range still fits, but a
    gradient of inf makes the norm non-finite and the step is skipped."""
    import torch
    N = 4
    h = zs.zs3_layout_create(N, 0, [0], [4096])
    try:
        g = np.full(4096, 0x7BFF, np.uint16)           # 65504, the largest fp16
        g[100] = 0x7C00                                  # +inf
        bufs = [Buf16(4096, fill=g) for _ in range(N)]
        gf = Buf16(1024)
        zs.zs3_reduce_scatter_local(h, 0, "fp16", [0], [b.ptr() for b in bufs], gf.ptr())
        ref = np.zeros(1024, np.uint16)
        oracle.reduce_scatter(oracle.make_layout(N, 0, [0], [4096]), 0, "fp16", [0], [{0: g}] * N, ref)
        sync()
        assert np.array_equal(gf.host(), ref)
        assert gf.host()[0] == 0x7BFF and gf.host()[100] == 0x7C00
        sumsq = torch.zeros(N + 1, dtype=torch.float64, device="cuda")
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        zs.zs3_grad_norm(h, 0, "fp16", gf.ptr(), sumsq, True, 1.0, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                         outs.data_ptr() + 12)
        W = Buf32(1024, 0, np.ones(1024, np.float32))
        M, V = Buf32(1024, 0, np.zeros(1024, np.float32)), Buf32(1024, 0, np.zeros(1024, np.float32))
        S = Buf16(1024, 0, np.full(1024, 0x3C00, np.uint16))
        zs.zs3_adam_step(h, 0, "fp16", 0, 1024, W.ptr(), M.ptr(), V.ptr(), gf.ptr(), S.ptr(), outs.data_ptr() + 8,
                         outs.data_ptr() + 12, oracle.AdamHParams(step=1))
        sync()
        assert int(outs.cpu().numpy()[1:2].view(np.int32)[1]) == 1
        assert np.all(W.host() == 1.0) and np.all(M.host() == 0) and np.all(S.host() == 0x3C00)
    finally:
        zs.zs3_layout_destroy(h)


def test_repeated_calls_reuse_plans_and_stay_exact():
    """The second and third identical calls take the cached work list."""
    seed, N, T, n, mx = PROBLEMS[4]
    ids, numels, full = _problem(seed, N, T, n, mx)
    h, L = _layout(ids, numels, N, T)
    try:
        srcs = {d: Buf16(full[d].size, fill=full[d]) for d in ids}
        ref = oracle.partition(L, 3, full)
        for k in range(3):
            out = Buf16(L.shard_numel)
            zs.zs3_partition(h, 3, "bf16", ids, [srcs[d].ptr() for d in ids], out.ptr())
            sync()
            assert np.array_equal(out.host(), ref)
    finally:
        zs.zs3_layout_destroy(h)


def test_time_next_launch_records_kernel_timestamps():
    """The instrumentation hook times exactly the next launch."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(a)) == 0 and hip.hipEventCreate(ctypes.byref(b)) == 0
    h = zs.zs3_layout_create(1, 0, [0], [1 << 24])
    try:
        src, dst = Buf16(1 << 24), Buf16(1 << 24)
        zs.zs3_time_next_launch(a.value, b.value)
        zs.zs3_partition(h, 0, "bf16", [0], [src.ptr()], dst.ptr())
        zs.zs3_partition(h, 0, "bf16", [0], [src.ptr()], dst.ptr())     # not timed
        sync()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        assert 0.0 < ms.value < 50.0
    finally:
        zs.zs3_layout_destroy(h)
        hip.hipEventDestroy(a)
        hip.hipEventDestroy(b)
