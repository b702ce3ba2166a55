"""Whole shard steps through ShardStep, and norm calls on several streams.

* The 16-bit shard is the round-to-nearest-even of the fp32 master after
  every step ([codex] 6.3: the optimizer writes the updated partition back
  into the shard; nothing else writes the shard during a step, because the
  pre-step pass that puts parameters back in partitioned form only drops
  the gathered views).  Checked on the GPT-2-shaped workload (98 persistent
  parameters) with the static gather buckets and with the gathers the
  fetch/release coordinator returns: two steps, then a step whose gradient
  holds an inf, which sets the non-finite flag and must leave master,
  momentum, variance and shard exactly as they were.
* The norm's scratch is per stream: two norm calls of one layout on two
  streams, launched back to back with no wait between them, give the same
  bits as the same calls one after the other (separate norm and the norm
  from the fused partial sums).
"""

import gc

import numpy as np
import pytest

import oracle
import zero_sharded_state_amd as zs
from synth import get_config
from synth.gen import random_bits16

from gpu_util import Buf16, note, require_gpu, sync

pytestmark = pytest.mark.gpu

INF16 = {"fp16": 0x7C00, "bf16": 0x7F80}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _h16(t):
    return t.cpu().numpy().view(np.uint16).copy()


def _assert_shard_is_rounded_master(step, what):
    master = step.master.cpu().numpy()
    want = oracle.from_f32(master, step.dtype)
    got = _h16(step.shard)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{what}: shard != round16(master) at {bad[:5]}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("schedule", ["static", "trace"])
def test_shard_is_rounded_master_and_inf_step_changes_nothing(schedule):
    import torch

    import bench
    from synth.modules import module_table, step_order
    from zero_sharded_state_amd.trace_schedule import TraceGatherPass

    cfg = get_config("c2")
    rank = 3
    note(f"shard step c2 rank={rank} schedule={schedule}: set-up")
    step = bench.make_step(cfg, rank, rs_streams=3, fuse_norm=True)
    trace = None
    try:
        bench.fill_inputs(step, cfg)
        assert step.P > 0, "the workload must have persistent parameters"
        if schedule == "trace":
            _, mods = module_table(cfg)
            trace = TraceGatherPass(step, mods, step_order(cfg),
                                    {"prefetch_bucket_size": cfg.prefetch_bucket_size,
                                     "max_live_parameters": int(1e9), "max_reuse_distance": int(1e9)})
            trace.plan()
            trace.fill_peer_chunks()
        sync()
        _assert_shard_is_rounded_master(step, "after set-up")
        for t in (1, 2):
            note(f"shard step c2 {schedule}: step {t}")
            step.step(trace_pass=trace)
            sync()
            assert int(step.outs.cpu().numpy()[1:2].view(np.int32)[1]) == 0
            _assert_shard_is_rounded_master(step, f"after step {t}")
        before = {k: getattr(step, k).cpu().numpy().view(np.uint32).copy() for k in ("master", "exp_avg", "exp_avg_sq")}
        shard_before = _h16(step.shard)
        # an inf in one received gradient slice: the averaged gradient, the
        # norm and the flag follow, and Adam must write nothing
        step.recv[5] = INF16[cfg.dtype] - (65536 if INF16[cfg.dtype] >= 32768 else 0)
        note(f"shard step c2 {schedule}: step 3 with an inf gradient")
        step.step(trace_pass=trace)
        sync()
        o = step.outs.cpu().numpy()
        assert int(o[1:2].view(np.int32)[1]) == 1, "non-finite flag not set"
        assert not np.isfinite(float(o[0]))
        for k, v in before.items():
            assert np.array_equal(getattr(step, k).cpu().numpy().view(np.uint32), v), f"{k} changed on a skipped step"
        assert np.array_equal(_h16(step.shard), shard_before), "shard changed on a skipped step"
        _assert_shard_is_rounded_master(step, "after the skipped step")
    finally:
        if trace is not None:
            trace.destroy()
        step.destroy()


@pytest.mark.timeout(300)
def test_norm_calls_on_two_streams_do_not_share_scratch():
    import torch
    N, T = 8, 100
    rng = np.random.default_rng(5)
    numels = [int(x) for x in rng.integers(50, 3_000_000, 12)] + [64, 90]
    ids = list(range(len(numels)))
    h = zs.zs3_layout_create(N, T, ids, numels)
    L = oracle.make_layout(N, T, ids, numels)
    try:
        S = L.shard_numel
        r = 2
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        # two flat gradients and their fused partial sums (from the library's reduce-scatter)
        grads, partials = [], []
        for k in range(2):
            gsrc = [Buf16(S, fill=random_bits16(100 * k + v, S, "bf16", 1e-3, 3)) for v in range(N)]
            gflat = Buf16(S)
            pt = torch.full((n_slots,), float("nan"), dtype=torch.float64, device="cuda")
            src = []
            for p in L.params:
                src += [b.ptr() + 2 * p.shard_offset for b in gsrc]
            zs.zs3_reduce_scatter_local(h, r, "bf16", ids, src, gflat.ptr(), pt)
            sync()
            del gsrc
            grads.append(gflat)
            partials.append(pt)
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        sumsq = [torch.full((N + 1,), 1e-3, dtype=torch.float64, device="cuda") for _ in range(2)]
        outs = [torch.zeros(2, dtype=torch.float64, device="cuda") for _ in range(2)]

        def call(kind, k):
            o = outs[k]
            if kind == "norm":
                zs.zs3_grad_norm(h, r, "bf16", grads[k].ptr(), sumsq[k], True, 1.0, 1.0, o.data_ptr(),
                                 o.data_ptr() + 8, o.data_ptr() + 12, stream=streams[k])
            else:
                zs.zs3_grad_norm_partials(h, r, partials[k], sumsq[k], True, 1.0, 1.0, o.data_ptr(),
                                          o.data_ptr() + 8, o.data_ptr() + 12, stream=streams[k])

        def snap():
            return [np.concatenate([s.cpu().numpy().view(np.uint64), x.cpu().numpy().view(np.uint64)])
                    for s, x in zip(sumsq, outs)]

        for kind in ("norm", "partials"):
            note(f"two-stream norm: {kind}, one after the other")
            for k in range(2):
                call(kind, k)
                sync()
            ref = snap()
            assert not np.array_equal(ref[0], ref[1]), "the two gradients must give different norms"
            for rep in range(20):
                for x in outs:
                    x.zero_()
                sync()
                call(kind, 0)
                call(kind, 1)
                sync()
                got = snap()
                for k in range(2):
                    assert np.array_equal(got[k], ref[k]), f"{kind}: stream {k} differs on repetition {rep}"
    finally:
        zs.zs3_layout_destroy(h)
