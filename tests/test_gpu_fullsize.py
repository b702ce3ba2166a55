"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (ShardStep: per-bucket calls, fused gathers, gradient buckets
over three streams).

* c2 (GPT-2-small set) and c3 (one Llama-3-8B layer): the whole step chained
  for 10 steps on the GPU against the oracle's own 10-step chain from the
  same synthetic inputs (weights, per-step gradients, the peers' norm
  partials); every output compared.  Variants: the norm fused into the
  reduce, the non-contiguous gradient path (reduce_scatter_coalesced), and
  the optimizer state offloaded to pinned host memory.
* c4 (Llama-3-8B set, 8.03B parameters, ranks 0 and 7) and c5 (ragged 7.46B
  set, N = 64, ranks 63 and 0, fp16, misaligned), in bench.py's launch configuration
  (three gradient streams, fused norm): each call fed fresh synthetic
  inputs, its outputs checked on a sample of whole parameters (the oracle
  recomputes those parameters only) or, for the norm, over the whole flat
  gradient the reduce-scatter produced.
* One whole step of c4 rank 0 and of c5 rank 63 in bench.py's default launch
  configuration: every element of the flat gradient, master, momentum,
  variance and shard against the oracle.
"""

import gc

import numpy as np
import pytest

import oracle
from synth import get_config
from synth.gen import KIND_GRAD, KIND_STATE, KIND_WEIGHT, device_normal16, weights_host

from gpu_util import assert_f32_close, note, ordinal16, require_gpu, sync

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _step(cfg, rank, fuse_norm=False, reduce_path="contiguous", offload=False):
    from zero_sharded_state_amd.shard_step import AdamConfig, ShardStep
    return ShardStep(world_size=cfg.world_size, rank=rank, threshold=cfg.threshold, ds_ids=cfg.ds_ids,
                     numels=cfg.numels, dtype=cfg.dtype, prefetch_bucket_size=cfg.prefetch_bucket_size,
                     reduce_bucket_size=cfg.reduce_bucket_size, sub_group_size=cfg.sub_group_size,
                     adam=AdamConfig(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay),
                     max_norm=cfg.max_norm, rs_streams=3, fuse_norm=fuse_norm, reduce_path=reduce_path,
                     offload=bool(offload), offload_chunk=3_000_001 if offload == "staged" else 0)


def h16(t):
    return t.cpu().numpy().view(np.uint16)


def _hp(cfg, t):
    return oracle.AdamHParams(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, t)


def _recv_grads(step, L, host_recv):
    """Oracle-side gradients: virtual rank v's full gradient of every
    parameter, zero except the slice this rank receives (the oracle reads
    only that slice)."""
    N = step.N
    grads = []
    for v in range(N):
        g = {}
        for p in L.params:
            lo, hi = L.own_range(p, step.rank)
            a = np.zeros(p.numel, np.uint16)
            o = step.recv_index(v, p.ds_id)
            a[lo:hi] = host_recv[o:o + (hi - lo)]
            g[p.ds_id] = a
        grads.append(g)
    return grads


# --------------------------------------------------------------------------
# c2 / c3: the whole step, chained, 10 steps
# --------------------------------------------------------------------------

def _oracle_reduce(step, L, cfg, rank, host_recv, host_own=None, host_x=None):
    """The oracle's flat gradient of one step.  Contiguous path: from the
    received slices.  Non-contiguous path: partitioned parameters from the
    N chunks addressed to this rank (its own packed by the oracle, the
    peers' as the GPU held them), persistent ones from the slices."""
    gf = np.zeros(L.shard_numel, np.uint16)
    grads = _recv_grads(step, L, host_recv)
    for bi, b in enumerate(oracle.reduce_buckets(L, cfg.reduce_bucket_size)):
        if step.reduce_path == "contiguous":
            oracle.reduce_scatter(L, rank, cfg.dtype, b, grads, gf)
            continue
        ids_part, ids_pers, C, _, chunks = step.coalesced[bi]
        assert sorted(ids_part + ids_pers) == sorted(b)
        if ids_part:
            own = {d: host_own[step.grad_off[d]:step.grad_off[d] + L.slot(d).numel] for d in ids_part}
            recv = [oracle.scatter_pack(L, ids_part, own)[rank] if v == rank else
                    host_x[chunks[v]:chunks[v] + C] for v in range(step.N)]
            oracle.scatter_reduce(L, rank, cfg.dtype, ids_part, recv, gf)
        if ids_pers:
            oracle.reduce_scatter(L, rank, cfg.dtype, ids_pers, grads, gf)
    return gf


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rank,fuse_norm,reduce_path,offload", [
    ("c2", 0, False, "contiguous", False), ("c2", 7, False, "contiguous", False),
    ("c3", 0, False, "contiguous", False), ("c3", 7, False, "contiguous", False),
    ("c2", 3, True, "contiguous", False), ("c2", 7, True, "coalesced", False),
    ("c3", 0, True, "coalesced", False), ("c2", 5, True, "contiguous", "staged"),
    ("c3", 7, True, "contiguous", "direct")])
def test_chained_steps_match_oracle(name, rank, fuse_norm, reduce_path, offload):
    import torch
    cfg = get_config(name)
    N, dt = cfg.world_size, cfg.dtype
    note(f"chain {name} rank={rank} fuse_norm={fuse_norm} {reduce_path} offload={offload}: set-up")
    step = _step(cfg, rank, fuse_norm, reduce_path, offload)
    L = oracle.make_layout(N, cfg.threshold, cfg.ds_ids, cfg.numels)
    try:
        full = {d: weights_host(cfg, d) for d in cfg.ds_ids}
        for d in cfg.ds_ids:
            p = step.by_id[d]
            if p["persistent"]:
                o = step.pers_off[d]
                step.pers_full[o:o + p["numel"]].copy_(torch.from_numpy(full[d].view(np.int16)))
            else:
                o = step.full_off[d]
                step.full[o:o + p["numel"]].copy_(torch.from_numpy(full[d].view(np.int16)))
        step.init_from_full()
        # oracle: every rank's shard and every bucket's chunks, this rank's fp32 state
        shards = [oracle.partition(L, v, full) for v in range(N)]
        chunks = {tuple(b): [oracle.pack(L, v, b, shards[v]) for v in range(N)] for b in step.gather_buckets}
        shard = shards[rank].copy()
        w, m, v_ = oracle.init_state(shard, dt)
        peers = np.random.default_rng(cfg.config_id).uniform(0.5, 2.0, N) * 1e-3   # what the all-reduce delivers
        for t in range(1, cfg.steps + 1):
            note(f"chain {name} rank={rank}: step {t}")
            device_normal16(step.recv.numel(), cfg.grad_std, dt, step.device, (cfg.seed, cfg.config_id, KIND_GRAD, t),
                            outlier_prob=cfg.outlier_prob, outlier_mult=cfg.outlier_mult, out=step.recv)
            host_recv = h16(step.recv)
            host_own = host_x = None
            if reduce_path == "coalesced":
                device_normal16(step.own_grads.numel(), cfg.grad_std, dt, step.device,
                                (cfg.seed, cfg.config_id, KIND_GRAD, 100 + t), outlier_prob=cfg.outlier_prob,
                                outlier_mult=cfg.outlier_mult, out=step.own_grads)
                device_normal16(step.xbuf.numel(), cfg.grad_std, dt, step.device,
                                (cfg.seed, cfg.config_id, KIND_GRAD, 200 + t), outlier_prob=cfg.outlier_prob,
                                outlier_mult=cfg.outlier_mult, out=step.xbuf)
                host_own, host_x = h16(step.own_grads), h16(step.xbuf)
            # GPU: the step as bench.py runs it, with the peers' partial sums supplied
            step.t = t - 1
            step.gather_pass()
            step.gather_pass()
            step.reduce_scatter()
            step.sumsq.copy_(torch.from_numpy(np.append(peers, 0.0)))
            step.grad_norm()
            step.adam_step(t)
            step.t = t
            # oracle chain
            gf = _oracle_reduce(step, L, cfg, rank, host_recv, host_own, host_x)
            a, q = oracle.grad_norm_partial(L, rank, dt, gf)
            parts = list(peers)
            parts[rank] = a
            norm, coef, scale, bad = oracle.grad_norm_finalize(parts, q, cfg.max_norm)
            shard_before = shard.copy()
            for b, e in oracle.sub_groups(L, cfg.sub_group_size):
                oracle.adam_step(L, rank, dt, b, e, w, m, v_, gf, shard, scale, bad, _hp(cfg, t))
            sync()
            assert np.array_equal(h16(step.grad), gf), f"reduce-scatter differs at step {t}"
            o = step.outs.cpu().numpy()
            assert abs(float(o[0]) - norm) <= 1e-5 * norm
            assert int(o[1:2].view(np.int32)[1]) == int(bad)
        # gathered parameters of the last step = the oracle's gather of the shard it started from
        got_full = h16(step.full)
        for bi, b in enumerate(step.gather_buckets):
            ch = list(chunks[tuple(b)])
            ch[rank] = oracle.pack(L, rank, b, shard_before)
            ref, offs = oracle.unpack(L, b, ch)
            fo, fn, _, _ = step.bucket_meta[bi]
            assert np.array_equal(got_full[fo:fo + fn], ref), f"bucket {bi} gathered parameters differ"
        for nm, got, ref in (("master", step.master, w), ("exp_avg", step.exp_avg, m),
                             ("exp_avg_sq", step.exp_avg_sq, v_)):
            assert_f32_close(got.cpu().numpy(), ref, 2e-6, nm)
        d = np.abs(ordinal16(h16(step.shard)) - ordinal16(shard))
        assert d.max() <= 1
    finally:
        step.destroy()
        del step


# --------------------------------------------------------------------------
# c4 / c5: every call at full size, sampled parameters
# --------------------------------------------------------------------------

def _sample_params(L, cfg, k=6):
    """A deterministic sample: the largest partitioned parameter, the last
    one, a persistent one, and a few spread over the ds_id range."""
    part = [p for p in L.params if not p.persistent]
    pers = [p for p in L.params if p.persistent]
    pick = {max(part, key=lambda p: p.numel).ds_id, part[-1].ds_id}
    if pers:
        pick.add(pers[len(pers) // 2].ds_id)
    idx = np.linspace(0, len(L.params) - 1, k).astype(int)
    pick |= {L.params[i].ds_id for i in idx}
    return sorted(pick)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rank", [("c4", 0), ("c4", 7), ("c5", 63), ("c5", 0)])
def test_fullsize_calls_on_sampled_parameters(name, rank):
    """In bench.py's launch configuration: gradient buckets over three
    streams, the norm fused into the reduce-scatter; the first and the last
    rank of each workload (c5's last rank holds every padded tail)."""
    import torch
    cfg = get_config(name)
    N, dt = cfg.world_size, cfg.dtype
    note(f"fullsize {name} rank={rank}: set-up")
    step = _step(cfg, rank, fuse_norm=True)
    L = oracle.make_layout(N, cfg.threshold, cfg.ds_ids, cfg.numels)
    sample = _sample_params(L, cfg)
    dev = step.device
    try:
        # ---- partition: synthetic full parameters -> shard
        device_normal16(step.full.numel(), cfg.weight_std, dt, dev, (cfg.seed, cfg.config_id, KIND_WEIGHT, 0),
                        out=step.full)
        device_normal16(step.P, cfg.weight_std, dt, dev, (cfg.seed, cfg.config_id, KIND_WEIGHT, 1), out=step.pers_full)
        note(f"fullsize {name}: partition")
        step.repartition()
        sync()
        got = h16(step.shard)
        for d in sample:
            p = L.slot(d)
            if p.persistent:
                o = step.pers_off[d]
                src = h16(step.pers_full[o:o + p.numel])
            else:
                o = step.full_off[d]
                src = h16(step.full[o:o + p.numel])
            sub = oracle.make_layout(N, cfg.threshold, [d], [p.numel])
            ref = oracle.partition(sub, rank, {d: src})
            assert np.array_equal(got[p.shard_offset:p.shard_offset + p.partition_size], ref), f"partition {d}"

        # ---- gather: synthetic shard and wire -> own chunks and full parameters
        device_normal16(step.S, cfg.weight_std, dt, dev, (cfg.seed, cfg.config_id, KIND_WEIGHT, 2), out=step.shard)
        device_normal16(step.W, cfg.weight_std, dt, dev, (cfg.seed, cfg.config_id, KIND_WEIGHT, 3), out=step.wire)
        sb = {bi for bi, b in enumerate(step.gather_buckets) if set(b) & set(sample)}
        wire_before = {bi: h16(step.wire[step.bucket_meta[bi][2]:step.bucket_meta[bi][2] +
                                         N * step.bucket_meta[bi][3]]) for bi in sb}
        note(f"fullsize {name}: gather pass")
        step.gather_pass()
        sync()
        shard_h = h16(step.shard)
        full_h = h16(step.full)
        for bi in sorted(sb):
            b = step.gather_buckets[bi]
            fo, fn, wo, cn = step.bucket_meta[bi]
            ch = [wire_before[bi][v * cn:(v + 1) * cn] for v in range(N)]
            ch[rank] = oracle.pack(L, rank, b, shard_h)
            ref, _ = oracle.unpack(L, b, ch)
            assert np.array_equal(full_h[fo:fo + fn], ref), f"gathered bucket {bi}"
            own = h16(step.wire[wo + rank * cn:wo + (rank + 1) * cn])
            assert np.array_equal(own, ch[rank]), f"packed chunk of bucket {bi}"

        # ---- reduce-scatter: synthetic received slices -> flat gradient
        device_normal16(step.recv.numel(), cfg.grad_std, dt, dev, (cfg.seed, cfg.config_id, KIND_GRAD, 1),
                        outlier_prob=cfg.outlier_prob, outlier_mult=cfg.outlier_mult, out=step.recv)
        note(f"fullsize {name}: reduce-scatter")
        step.grad.fill_(0x3C3C)
        step.reduce_scatter()
        sync()
        gh = h16(step.grad)
        for d in sample:
            p = L.slot(d)
            lo, hi = L.own_range(p, rank)
            grads = []
            for v in range(N):
                a = np.zeros(p.numel, np.uint16)
                o = step.recv_index(v, p.ds_id)
                a[lo:hi] = h16(step.recv[o:o + (hi - lo)])
                grads.append({d: a})
            sub = oracle.make_layout(N, cfg.threshold, [d], [p.numel])
            ref = np.zeros(sub.shard_numel, np.uint16)
            oracle.reduce_scatter(sub, rank, dt, [d], grads, ref)
            assert np.array_equal(gh[p.shard_offset:p.shard_offset + p.partition_size], ref), f"reduce-scatter {d}"

        # ---- norm: the partial sums the reduce-scatter just wrote, over the
        # whole flat gradient it produced -> norm and scale
        peers = np.random.default_rng(5).uniform(0.5, 2.0, N)
        step.sumsq.copy_(torch.from_numpy(np.append(peers, 0.0)))
        note(f"fullsize {name}: grad norm")
        step.grad_norm()
        sync()
        gflat = gh
        a, q = oracle.grad_norm_partial(L, rank, dt, gflat)
        parts = list(peers)
        parts[rank] = a
        norm, coef, scale, bad = oracle.grad_norm_finalize(parts, q, cfg.max_norm)
        s = step.sumsq.cpu().numpy()
        assert s[rank] == pytest.approx(a, rel=1e-10) and s[N] == pytest.approx(q, rel=1e-10, abs=1e-300)
        o = step.outs.cpu().numpy()
        assert abs(float(o[0]) - norm) <= 1e-5 * norm
        gscale = float(o[1:2].view(np.float32)[0])
        assert abs(gscale - float(scale)) <= np.spacing(np.float32(scale))

        # ---- Adam: synthetic master, 10 steps of synthetic gradients, the GPU's scale
        device_normal16(step.S, 1.0, "bf16", dev, (cfg.seed, cfg.config_id, KIND_STATE, 0), out=step.grad)
        step.master.copy_(step.grad.view(torch.bfloat16).to(torch.float32) * 0.02)
        step.exp_avg.zero_()
        step.exp_avg_sq.zero_()
        w0 = {d: step.master[L.slot(d).shard_offset:L.slot(d).shard_offset + L.slot(d).partition_size].cpu().numpy()
              for d in sample}
        gs = {d: [] for d in sample}
        for t in range(1, 11):
            device_normal16(step.S, 1e-3, dt, dev, (cfg.seed, cfg.config_id, KIND_GRAD, 10 + t), out=step.grad)
            for d in sample:
                p = L.slot(d)
                gs[d].append(h16(step.grad[p.shard_offset:p.shard_offset + p.partition_size]))
            note(f"fullsize {name}: adam step {t}")
            step.adam_step(t)
        sync()
        sc = np.float32(gscale)
        for d in sample:
            p = L.slot(d)
            sub = oracle.make_layout(N, cfg.threshold, [d], [p.numel])
            w = w0[d].copy()
            m = np.zeros_like(w)
            v = np.zeros_like(w)
            sh = np.zeros(p.partition_size, np.uint16)
            for t in range(1, 11):
                oracle.adam_step(sub, rank, dt, 0, sub.shard_numel, w, m, v, gs[d][t - 1], sh, sc, False, _hp(cfg, t))
            o0, o1 = p.shard_offset, p.shard_offset + p.partition_size
            real = ~oracle.padding_mask(sub, rank)
            for nm, got, ref in (("master", step.master[o0:o1], w), ("exp_avg", step.exp_avg[o0:o1], m),
                                 ("exp_avg_sq", step.exp_avg_sq[o0:o1], v)):
                gg = got.cpu().numpy()
                assert_f32_close(gg[real], ref[real], 2e-6, f"{nm} of {d}")
            dd = np.abs(ordinal16(h16(step.shard[o0:o1])[real]) - ordinal16(sh[real]))
            assert dd.max() <= 1, f"shard of {d}"
    finally:
        step.destroy()
        del step


# --------------------------------------------------------------------------
# c4 rank 0: every element of one whole step
# --------------------------------------------------------------------------

@pytest.mark.timeout(900)
def test_c4_rank0_whole_step_every_element():
    """One whole c4 step of rank 0 in bench.py's default launch configuration
    (gather buckets over two streams, gradient buckets over three, received
    slices per bucket, fused norm), then every element of the rank's flat
    gradient, fp32 master, momentum, variance and 16-bit shard compared with
    the oracle, parameter by parameter (rank 0's own range of every parameter
    starts at element 0, so a one-parameter layout and the received slices
    are all the oracle needs; host memory stays bounded by the largest
    parameter).  Bit-exact, with Adam run on the scale the GPU used; that
    scale within 1 ulp of the oracle's and the norm within 1e-5."""
    import torch

    import bench
    cfg = get_config("c4")
    N, dt, rank = cfg.world_size, cfg.dtype, 0
    note("c4 rank 0 whole step: set-up")
    step = bench.make_step(cfg, rank, rs_streams=3, gather_streams=2, fuse_norm=True, recv_layout="bucket")
    try:
        bench.fill_inputs(step, cfg)
        sync()
        shard0 = h16(step.shard).copy()                       # the shard before the step (2 GB)
        note("c4 rank 0 whole step: one step")
        step.step()
        sync()
        o = step.outs.cpu().numpy()
        gpu_norm = float(o[0])
        gpu_scale = np.float32(o[1:2].view(np.float32)[0])
        assert int(o[1:2].view(np.int32)[1]) == 0
        sumsq = step.sumsq.cpu().numpy()
        # pass 1: the flat gradient, and the oracle's partial sums
        part = pers = 0.0
        for p in step.params:
            d, n, ps, off = p["ds_id"], p["numel"], p["partition_size"], p["shard_offset"]
            lo, hi = p["own"]
            assert lo == 0
            L1 = oracle.make_layout(N, cfg.threshold, [d], [n])
            grads = [{d: h16(step.recv[step.recv_index(v, d):step.recv_index(v, d) + hi])} for v in range(N)]
            ref = np.zeros(ps, np.uint16)
            oracle.reduce_scatter(L1, rank, dt, [d], grads, ref)
            got = h16(step.grad[off:off + ps])
            assert np.array_equal(got, ref), f"flat gradient of ds_id {d}"
            a, q = oracle.grad_norm_partial(L1, rank, dt, ref)
            part += a
            pers += q
        peers = [float(sumsq[v]) if v != rank else part for v in range(N)]
        norm, coef, scale, bad = oracle.grad_norm_finalize(peers, pers, cfg.max_norm)
        assert not bad
        assert abs(gpu_norm - norm) <= 1e-5 * norm
        assert abs(float(gpu_scale) - float(scale)) <= float(np.spacing(np.float32(scale)))
        assert float(sumsq[rank]) == pytest.approx(part, rel=1e-12)
        # pass 2: Adam (t = 1) on every parameter's range, with the GPU's scale
        hp = _hp(cfg, 1)
        for p in step.params:
            d, n, ps, off = p["ds_id"], p["numel"], p["partition_size"], p["shard_offset"]
            L1 = oracle.make_layout(N, cfg.threshold, [d], [n])
            g = h16(step.grad[off:off + ps])
            sh = shard0[off:off + ps].copy()
            w, m, v_ = oracle.init_state(sh, dt)
            oracle.adam_step(L1, rank, dt, 0, ps, w, m, v_, g, sh, gpu_scale, False, hp)
            for name, t, ref in (("master", step.master, w), ("exp_avg", step.exp_avg, m),
                                 ("exp_avg_sq", step.exp_avg_sq, v_)):
                got = t[off:off + ps].cpu().numpy()
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{name} of ds_id {d}"
            assert np.array_equal(h16(step.shard[off:off + ps]), sh), f"16-bit shard of ds_id {d}"
        note(f"c4 rank 0 whole step: every element equal (norm {gpu_norm:.6g})")
    finally:
        step.destroy()


# --------------------------------------------------------------------------
# c5 rank 63: every element of one whole step (N = 64, fp16, ragged)
# --------------------------------------------------------------------------

@pytest.mark.timeout(900)
def test_c5_rank63_whole_step_every_element():
    """One whole c5 step of the last rank (N = 64, fp16, every partitioned
    tensor padded; the wide reduce-scatter) in bench.py's default launch
    configuration, then every element of the rank's flat gradient, fp32
    master, momentum, variance and 16-bit shard compared with the oracle,
    parameter by parameter.  The last rank's own range starts at 63 x
    partition_size, so the oracle's owner-side reduce takes the 64 received
    slices themselves (its reading of the arithmetic is the reduce-scatter's,
    R23); persistent parameters, whole on every rank, go through the oracle's
    reduce-scatter.  Host memory stays bounded by 64 slices of the largest
    parameter.  Bit-exact, with Adam run on the scale the GPU used; that
    scale within 1 ulp of the oracle's and the norm within 1e-5."""
    import bench
    cfg = get_config("c5")
    N, dt = cfg.world_size, cfg.dtype
    rank = N - 1
    note(f"c5 rank {rank} whole step: set-up")
    step = bench.make_step(cfg, rank, rs_streams=3, gather_streams=2, fuse_norm=True, recv_layout="bucket")
    try:
        bench.fill_inputs(step, cfg)
        sync()
        shard0 = h16(step.shard).copy()
        note(f"c5 rank {rank} whole step: one step")
        step.step()
        sync()
        o = step.outs.cpu().numpy()
        gpu_norm = float(o[0])
        gpu_scale = np.float32(o[1:2].view(np.float32)[0])
        assert int(o[1:2].view(np.int32)[1]) == 0
        sumsq = step.sumsq.cpu().numpy()
        part = pers = 0.0
        n_padded = 0
        for p in step.params:
            d, n, ps, off = p["ds_id"], p["numel"], p["partition_size"], p["shard_offset"]
            lo, hi = p["own"]
            real = hi - lo
            L1 = oracle.make_layout(N, cfg.threshold, [d], [n])
            ref = np.full(ps, 0xFFFF, np.uint16)
            slices = [h16(step.recv[step.recv_index(v, d):step.recv_index(v, d) + real]) for v in range(N)]
            if p["persistent"]:
                assert lo == 0 and real == n
                oracle.reduce_scatter(L1, rank, dt, [d], [{d: s} for s in slices], ref)
            else:
                n_padded += int(real < ps)
                received = [np.concatenate([s, np.zeros(ps - real, np.uint16)]) for s in slices]
                oracle.scatter_reduce(L1, rank, dt, [d], received, ref)
            got = h16(step.grad[off:off + ps])
            assert np.array_equal(got, ref), f"flat gradient of ds_id {d}"
            a, q = oracle.grad_norm_partial(L1, rank, dt, ref)
            part += a
            pers += q
        assert n_padded > 100, "the last rank must hold padding in most partitioned tensors"
        peers = [float(sumsq[v]) if v != rank else part for v in range(N)]
        norm, coef, scale, bad = oracle.grad_norm_finalize(peers, pers, cfg.max_norm)
        assert not bad
        assert abs(gpu_norm - norm) <= 1e-5 * norm
        assert abs(float(gpu_scale) - float(scale)) <= float(np.spacing(np.float32(scale)))
        assert float(sumsq[rank]) == pytest.approx(part, rel=1e-12)
        hp = _hp(cfg, 1)
        for p in step.params:
            d, n, ps, off = p["ds_id"], p["numel"], p["partition_size"], p["shard_offset"]
            L1 = oracle.make_layout(N, cfg.threshold, [d], [n])
            g = h16(step.grad[off:off + ps])
            sh = shard0[off:off + ps].copy()
            w, m, v_ = oracle.init_state(sh, dt)
            oracle.adam_step(L1, rank, dt, 0, ps, w, m, v_, g, sh, gpu_scale, False, hp)
            for name, t, want in (("master", step.master, w), ("exp_avg", step.exp_avg, m),
                                  ("exp_avg_sq", step.exp_avg_sq, v_)):
                got = t[off:off + ps].cpu().numpy()
                assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{name} of ds_id {d}"
            assert np.array_equal(h16(step.shard[off:off + ps]), sh), f"16-bit shard of ds_id {d}"
        note(f"c5 rank {rank} whole step: every element equal (norm {gpu_norm:.6g})")
    finally:
        step.destroy()
