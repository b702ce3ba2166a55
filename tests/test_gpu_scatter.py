"""GPU parity of the non-contiguous gradient path (reduce_scatter_coalesced:
send-side pack and owner-side reduce) and of the norm fused into both
reduce paths, against the CPU oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
import zero_sharded_state_amd as zs
from synth.gen import random_bits16, to16_host

from gpu_util import Buf16, note, require_gpu, sync
from test_gpu_parity import PROBLEMS, _layout, _problem

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _grads(seed, L, ids, dtype):
    rng = np.random.default_rng(seed + 200)
    out = []
    for _ in range(L.world_size):
        out.append({d: to16_host((rng.standard_normal(L.slot(d).numel) * 1e-3).astype(np.float32), dtype)
                    for d in ids})
    return out


def _part_buckets(L, limit):
    """Reduce buckets with the persistent parameters taken out."""
    out = []
    for b in oracle.reduce_buckets(L, limit):
        p = [d for d in b if not L.slot(d).persistent]
        if p:
            out.append(p)
    return out


def _poison_padding(L, bucket, rank, chunk, rng):
    """Nonzero garbage at the padding positions of a received chunk."""
    c = 0
    for p in sorted((L.slot(d) for d in bucket), key=lambda q: q.ds_id):
        lo, hi = L.own_range(p, rank)
        n_pad = p.partition_size - (hi - lo)
        if n_pad:
            chunk[c + (hi - lo):c + p.partition_size] = rng.integers(0x3000, 0x3c00, n_pad).astype(np.uint16)
        c += p.partition_size


@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("shifts", [(0, 0), (3, 5), (7, 1)])
def test_scatter_pack_bit_exact(prob, shifts):
    seed, N, T, n, mx = prob
    s_grad, s_send = shifts
    ids, numels, _ = _problem(seed, N, T, n, mx)
    h, L = _layout(ids, numels, N, T)
    try:
        grads = _grads(seed, L, ids, "bf16")
        r = (seed * 5) % N
        for b in _part_buckets(L, max(1, sum(numels) // 3)):
            C = sum(L.slot(d).partition_size for d in b)
            ref = np.concatenate(oracle.scatter_pack(L, b, grads[r]))
            note(f"scatter pack seed={seed} N={N} rank={r} bucket={len(b)} C={C} shifts={shifts}")
            gb = {d: Buf16(L.slot(d).numel, shift=(d + s_grad) % 8, fill=grads[r][d]) for d in b}
            send = Buf16(N * C, shift=s_send, fill=np.full(N * C, 0x7A7A, np.uint16))
            req = b[::-1]
            zs.zs3_reduce_scatter_coalesced(h, r, "bf16", zs.ZS3_PACK, req, grads=[gb[d].ptr() for d in req],
                                            send=send.ptr())
            sync()
            assert np.array_equal(send.host(), ref)
            send.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shift", [0, 3])
def test_scatter_reduce_bit_exact(prob, dtype, shift):
    seed, N, T, n, mx = prob
    ids, numels, _ = _problem(seed, N, T, n, mx, dtype)
    h, L = _layout(ids, numels, N, T)
    rng = np.random.default_rng(seed + 300)
    try:
        grads = _grads(seed, L, ids, dtype)
        buckets = _part_buckets(L, max(1, sum(numels) // 4))
        for r in sorted({0, N - 1}):
            ref = np.full(L.shard_numel, 0x3C3C, np.uint16)
            out = Buf16(L.shard_numel, shift=shift, fill=ref)
            keep = []
            for b in buckets:
                sends = [oracle.scatter_pack(L, b, grads[v]) for v in range(N)]
                recv = [sends[v][r].copy() for v in range(N)]
                for ch in recv:
                    _poison_padding(L, b, r, ch, rng)
                oracle.scatter_reduce(L, r, dtype, b, recv, ref)
                bufs = [Buf16(ch.size, shift=(v + shift) % 8, fill=ch) for v, ch in enumerate(recv)]
                keep += bufs
                note(f"scatter reduce seed={seed} N={N} rank={r} {dtype} bucket={len(b)} shift={shift}")
                zs.zs3_reduce_scatter_coalesced(h, r, dtype, zs.ZS3_REDUCE, b, recv_chunks=[x.ptr() for x in bufs],
                                                grad_flat=out.ptr())
            sync()
            got = out.host()
            assert np.array_equal(got, ref), f"mismatch at {np.nonzero(got != ref)[0][:10]}"
            out.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("N", [1, 4, 8])
def test_scatter_pack_and_reduce_in_one_call(N):
    """Both bits: the own chunk is read from the send buffer the pack just
    wrote; the result equals the contiguous path's."""
    ids = [3, 1, 4, 9, 2]
    numels = [70001, 33, 4096 * 3 + 5, 17, 129]
    h, L = _layout(ids, numels, N, 0)
    try:
        grads = _grads(11, L, ids, "bf16")
        r = N - 1
        C = sum(L.slot(d).partition_size for d in ids)
        peers = [oracle.scatter_pack(L, ids, grads[v])[r] for v in range(N)]
        gb = {d: Buf16(L.slot(d).numel, shift=d % 8, fill=grads[r][d]) for d in ids}
        send = Buf16(N * C, shift=2)
        bufs = [Buf16(C, fill=peers[v]) for v in range(N)]
        recv = [b.ptr() for b in bufs]
        recv[r] = send.ptr() + 2 * r * C
        out = Buf16(L.shard_numel, shift=1, fill=np.full(L.shard_numel, 0x1111, np.uint16))
        note(f"scatter pack+reduce N={N}")
        zs.zs3_reduce_scatter_coalesced(h, r, "bf16", zs.ZS3_PACK | zs.ZS3_REDUCE, ids,
                                        grads=[gb[d].ptr() for d in ids], send=send.ptr(), recv_chunks=recv,
                                        grad_flat=out.ptr())
        sync()
        ref = np.full(L.shard_numel, 0x1111, np.uint16)
        oracle.reduce_scatter(L, r, "bf16", ids, grads, ref)
        assert np.array_equal(out.host(), ref)
        out.check_guards()
        send.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


# ------------------------------------------------- norm fused into the reduce

def _norm_from_partials(h, L, r, partials, peer_parts, pers, max_norm):
    import torch
    N = L.world_size
    sumsq = torch.zeros(N + 1, dtype=torch.float64, device="cuda")
    sumsq[:N] = torch.tensor(peer_parts, dtype=torch.float64)
    outs = torch.zeros(2, dtype=torch.float64, device="cuda")
    zs.zs3_grad_norm_partials(h, r, partials, sumsq, True, max_norm, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                              outs.data_ptr() + 12)
    sync()
    o = outs.cpu().numpy()
    return sumsq.cpu().numpy(), float(o[0]), float(o[1:2].view(np.float32)[0]), int(o[1:2].view(np.int32)[1])


@pytest.mark.parametrize("prob", PROBLEMS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("path", ["contiguous", "coalesced"])
def test_fused_norm_matches_oracle(prob, dtype, path):
    """Every slot starts as NaN: a slot the reduce fails to write poisons the
    norm.  The fused sums equal the oracle's shard-aware partials."""
    import torch
    seed, N, T, n, mx = prob
    ids, numels, _ = _problem(seed, N, T, n, mx, dtype)
    h, L = _layout(ids, numels, N, T)
    try:
        grads = _grads(seed, L, ids, dtype)
        n_slots, n_part = zs.zs3_layout_norm_slots(h)
        assert 0 < n_part <= n_slots or (n_part == 0 and all(p.persistent for p in L.params))
        r = (seed * 3) % N
        ref = np.zeros(L.shard_numel, np.uint16)
        limit = max(1, sum(numels) // 4)
        for b in oracle.reduce_buckets(L, limit):
            oracle.reduce_scatter(L, r, dtype, b, grads, ref)
        part, pers = oracle.grad_norm_partial(L, r, dtype, ref)
        partials = torch.full((n_slots,), float("nan"), dtype=torch.float64, device="cuda")
        out = Buf16(L.shard_numel, shift=seed % 8)
        keep = []
        for b in oracle.reduce_buckets(L, limit):
            pb = [d for d in b if not L.slot(d).persistent]
            qb = [d for d in b if L.slot(d).persistent] if path == "coalesced" else b
            if path == "coalesced" and pb:
                recv = [oracle.scatter_pack(L, pb, grads[v])[r] for v in range(N)]
                bufs = [Buf16(ch.size, shift=v % 8, fill=ch) for v, ch in enumerate(recv)]
                keep += bufs
                zs.zs3_reduce_scatter_coalesced(h, r, dtype, zs.ZS3_REDUCE, pb, recv_chunks=[x.ptr() for x in bufs],
                                                grad_flat=out.ptr(), partials=partials.data_ptr())
            if qb:
                src = []
                for d in qb:
                    lo, _ = L.own_range(L.slot(d), r)
                    for v in range(N):
                        buf = Buf16(L.slot(d).numel, shift=(v + d) % 8, fill=grads[v][d])
                        keep.append(buf)
                        src.append(buf.ptr() + 2 * lo)
                zs.zs3_reduce_scatter_local(h, r, dtype, qb, src, out.ptr(), partials=partials.data_ptr())
        note(f"fused norm seed={seed} N={N} rank={r} {dtype} {path}")
        sync()
        assert np.array_equal(out.host(), ref)
        peers = [part * (1 + 0.1 * v) if v != r else 0.0 for v in range(N)]
        s, norm_got, scale_got, flag = _norm_from_partials(h, L, r, partials, peers, pers, 0.5)
        assert s[r] == pytest.approx(part, rel=1e-12, abs=0)
        assert s[N] == pytest.approx(pers, rel=1e-12, abs=0)
        all_parts = list(peers)
        all_parts[r] = part
        norm, coef, scale, bad = oracle.grad_norm_finalize(all_parts, pers, 0.5)
        assert flag == 0 and not bad
        assert norm_got == pytest.approx(norm, rel=1e-12)
        assert abs(scale_got - float(scale)) <= float(np.spacing(np.float32(scale)))
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("shift", range(8))
def test_fused_norm_every_slot_written_at_piece_edges(shift):
    """Slices one element either side of the piece size, at every
    destination alignment: the spare slot group is zeroed when the aligned
    split needs one piece fewer than the bound."""
    import torch
    P = 256 * 2 * 8 * 8     # elements of one reduce-scatter piece (256 threads x 2 vectors x 8 x 8 workgroups)
    numels = [1, 7, 8, 9, P - 1, P, P + 1, P + 2, P + 7, P + 8, 2 * P + 3, 3 * P - 1]
    ids = list(range(len(numels)))
    h, L = _layout(ids, numels, 1, 0)
    try:
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        g = {d: random_bits16(d + 40, numels[d], "fp16", 1e-2, 1) for d in ids}
        partials = torch.full((n_slots,), float("nan"), dtype=torch.float64, device="cuda")
        out = Buf16(L.shard_numel, shift=shift)
        bufs = [Buf16(numels[d], shift=(d + shift) % 8, fill=g[d]) for d in ids]
        note(f"fused norm piece edges shift={shift}")
        for d in ids:     # one call per parameter: every slice in its own launch
            zs.zs3_reduce_scatter_local(h, 0, "fp16", [d], [bufs[d].ptr()], out.ptr(), partials=partials.data_ptr())
        sync()
        ref = np.zeros(L.shard_numel, np.uint16)
        oracle.reduce_scatter(L, 0, "fp16", ids, [g], ref)
        assert np.array_equal(out.host(), ref)
        p = partials.cpu().numpy()
        assert np.all(np.isfinite(p))
        part, _ = oracle.grad_norm_partial(L, 0, "fp16", ref)
        assert float(p.sum()) == pytest.approx(part, rel=1e-12)
    finally:
        zs.zs3_layout_destroy(h)


def test_fused_norm_nonfinite_flag():
    import torch
    h = zs.zs3_layout_create(2, 0, [0], [5000])
    try:
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        g = random_bits16(3, 5000, "fp16", 1e-2, 1)
        g[1234] = 0x7C00   # +inf in rank 0's slice; the average stays inf
        bufs = [Buf16(5000, fill=g) for _ in range(2)]
        out = Buf16(2500)
        partials = torch.zeros(n_slots, dtype=torch.float64, device="cuda")
        zs.zs3_reduce_scatter_local(h, 0, "fp16", [0], [b.ptr() for b in bufs], out.ptr(),
                                    partials=partials.data_ptr())
        sumsq = torch.zeros(3, dtype=torch.float64, device="cuda")
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        zs.zs3_grad_norm_partials(h, 0, partials, sumsq, True, 1.0, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                                  outs.data_ptr() + 12)
        sync()
        assert int(outs.cpu().numpy()[1:2].view(np.int32)[1]) == 1
    finally:
        zs.zs3_layout_destroy(h)


def test_fused_norm_on_an_empty_layout():
    """No parameters: no slots; the partial sums are 0 and the peers' sums
    alone make the norm."""
    import torch
    h = zs.zs3_layout_create(2, 0, [], [])
    try:
        assert zs.zs3_layout_norm_slots(h) == (0, 0)
        partials = torch.zeros(1, dtype=torch.float64, device="cuda")
        sumsq = torch.full((3,), 7.0, dtype=torch.float64, device="cuda")
        sumsq[1] = 4.0
        outs = torch.zeros(2, dtype=torch.float64, device="cuda")
        zs.zs3_grad_norm_partials(h, 0, partials, sumsq, True, 1.0, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
                                  outs.data_ptr() + 12)
        sync()
        s = sumsq.cpu().numpy()
        assert s[0] == 0.0 and s[2] == 0.0 and float(outs.cpu().numpy()[0]) == 2.0
    finally:
        zs.zs3_layout_destroy(h)


def test_scatter_empty_request_and_padding_only_rank():
    """An empty bucket is a no-op; a rank whose ranges are all padding
    writes zeros (and zero partial sums) whatever the chunks hold."""
    import torch
    h = zs.zs3_layout_create(64, 0, [0, 1], [5, 70])      # rank 63: padding of both (ps 1 and 2)
    try:
        zs.zs3_reduce_scatter_coalesced(h, 63, "fp16", zs.ZS3_PACK | zs.ZS3_REDUCE, [], grads=[], send=Buf16(8).ptr(),
                                        recv_chunks=[Buf16(8).ptr()] * 64, grad_flat=Buf16(8).ptr())
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        partials = torch.full((n_slots,), float("nan"), dtype=torch.float64, device="cuda")
        chunks = [Buf16(3, fill=np.array([0x3C00, 0x3C00, 0x3C00], np.uint16)) for _ in range(64)]
        out = Buf16(3, fill=np.full(3, 0x1234, np.uint16))
        zs.zs3_reduce_scatter_coalesced(h, 63, "fp16", zs.ZS3_REDUCE, [1, 0], recv_chunks=[c.ptr() for c in chunks],
                                        grad_flat=out.ptr(), partials=partials.data_ptr())
        sync()
        assert out.host().tolist() == [0, 0, 0]
        assert np.all(partials.cpu().numpy() == 0.0)
        out.check_guards()
    finally:
        zs.zs3_layout_destroy(h)
