"""Run-to-run bit identity and checkpoint/resume, in bench.py's launch
configuration (gradient buckets over three streams, the norm fused into the
reduce-scatter), on the one-Llama-layer workload (bf16, N = 8, rank 7).

* Two runs of six whole steps from the same inputs give bit-identical
  master, momentum, variance, 16-bit shard, flat gradient and norm: nothing
  in the path depends on stream timing or the order in which concurrent
  workgroups finish.
* Resume: three steps, then the flat state (fp32 master/m/v, the 16-bit
  shard and the step counter) copied to the host, the step object and all
  its device buffers destroyed, a new one built (fresh allocations), the
  state restored, three more steps: bit-identical to the six uninterrupted
  steps.
"""

import gc

import numpy as np
import pytest

from synth import get_config
from synth.gen import KIND_GRAD, device_normal16, weights_host

from gpu_util import note, require_gpu, sync

pytestmark = pytest.mark.gpu

NAME, RANK, STEPS, SPLIT = "c3", 7, 6, 3


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _new_step(cfg):
    import torch
    from zero_sharded_state_amd.shard_step import AdamConfig, ShardStep
    step = ShardStep(world_size=cfg.world_size, rank=RANK, threshold=cfg.threshold, ds_ids=cfg.ds_ids,
                     numels=cfg.numels, dtype=cfg.dtype, prefetch_bucket_size=cfg.prefetch_bucket_size,
                     reduce_bucket_size=cfg.reduce_bucket_size, sub_group_size=cfg.sub_group_size,
                     adam=AdamConfig(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay),
                     max_norm=cfg.max_norm, rs_streams=3, fuse_norm=True)
    for d in cfg.ds_ids:
        w = torch.from_numpy(weights_host(cfg, d).view(np.int16))
        p = step.by_id[d]
        if p["persistent"]:
            o = step.pers_off[d]
            step.pers_full[o:o + p["numel"]].copy_(w)
        else:
            o = step.full_off[d]
            step.full[o:o + p["numel"]].copy_(w)
    step.init_from_full()
    return step


def _run(step, cfg, t_from, t_to, norms):
    import torch
    peers = np.random.default_rng(cfg.config_id).uniform(0.5, 2.0, cfg.world_size) * 1e-3
    for t in range(t_from, t_to + 1):
        device_normal16(step.recv.numel(), cfg.grad_std, cfg.dtype, step.device,
                        (cfg.seed, cfg.config_id, KIND_GRAD, t), outlier_prob=cfg.outlier_prob,
                        outlier_mult=cfg.outlier_mult, out=step.recv)
        step.gather_pass()
        step.gather_pass()
        step.reduce_scatter()
        step.sumsq.copy_(torch.from_numpy(np.append(peers, 0.0)))
        step.grad_norm()
        step.adam_step(t)
        step.t = t
        sync()
        norms.append(step.outs.cpu().numpy().view(np.uint64).copy())


def _state(step):
    return {"master": step.master.cpu().numpy().view(np.uint32).copy(),
            "exp_avg": step.exp_avg.cpu().numpy().view(np.uint32).copy(),
            "exp_avg_sq": step.exp_avg_sq.cpu().numpy().view(np.uint32).copy(),
            "shard": step.shard.cpu().numpy().view(np.uint16).copy(),
            "grad": step.grad.cpu().numpy().view(np.uint16).copy(),
            "t": step.t}


def _six_steps(cfg, label):
    note(f"determinism {NAME} rank={RANK}: {label}")
    step = _new_step(cfg)
    norms = []
    try:
        _run(step, cfg, 1, STEPS, norms)
        return _state(step), norms
    finally:
        step.destroy()


def _assert_same(a, b, what):
    for k in ("master", "exp_avg", "exp_avg_sq", "shard", "grad"):
        assert np.array_equal(a[k], b[k]), f"{what}: {k} differs at {np.nonzero(a[k] != b[k])[0][:5]}"
    assert a["t"] == b["t"]


@pytest.mark.timeout(600)
def test_two_runs_are_bit_identical():
    cfg = get_config(NAME)
    s1, n1 = _six_steps(cfg, "run 1")
    gc.collect()
    s2, n2 = _six_steps(cfg, "run 2")
    _assert_same(s1, s2, "second run")
    assert all(np.array_equal(x, y) for x, y in zip(n1, n2)), "norm or scale differs"


@pytest.mark.timeout(600)
def test_resume_from_flat_state_is_bit_identical():
    import torch
    cfg = get_config(NAME)
    ref, ref_norms = _six_steps(cfg, "uninterrupted")
    gc.collect()
    note(f"determinism {NAME} rank={RANK}: {SPLIT} steps, then checkpoint")
    step = _new_step(cfg)
    norms = []
    try:
        _run(step, cfg, 1, SPLIT, norms)
        ckpt = {"master": step.master.cpu().clone(), "exp_avg": step.exp_avg.cpu().clone(),
                "exp_avg_sq": step.exp_avg_sq.cpu().clone(), "shard": step.shard.cpu().clone(), "t": step.t}
    finally:
        step.destroy()
        del step
    gc.collect()
    torch.cuda.empty_cache()
    note(f"determinism {NAME} rank={RANK}: resume from the checkpoint")
    step = _new_step(cfg)
    try:
        for k in ("master", "exp_avg", "exp_avg_sq", "shard"):
            getattr(step, k).copy_(ckpt[k])
        step.t = ckpt["t"]
        _run(step, cfg, SPLIT + 1, STEPS, norms)
        _assert_same(_state(step), ref, "resumed run")
    finally:
        step.destroy()
    assert all(np.array_equal(x, y) for x, y in zip(norms, ref_norms)), "norm or scale differs"
