"""The allocation-free slot norm (zs3_grad_norm_partials_noalloc) against
zs3_grad_norm_partials, through the C ABI: the same partial sums, norm,
clip scale and non-finite flag, bit for bit, on calls in a row whose slot
arrays shrink (the static scratch keeps the previous call's contents, so
each call must not read what it did not write), with and without the
finalize step, and with an inf among the slots."""

import numpy as np
import pytest

import zero_sharded_state_amd as zs
from synth import get_config

from gpu_util import note, require_gpu, sync

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _layout(name):
    cfg = get_config(name)
    return cfg, zs.zs3_layout_create(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)


def _run(fn, h, rank, N, partials, finalize, max_norm):
    import torch
    sumsq = torch.tensor(np.linspace(0.5, 2.0, N + 1), dtype=torch.float64, device="cuda")
    outs = torch.full((2,), -1.0, dtype=torch.float64, device="cuda")
    fn(h, rank, partials, sumsq, finalize, max_norm, 1.0, outs.data_ptr(), outs.data_ptr() + 8,
       outs.data_ptr() + 12)
    sync()
    return sumsq.cpu().numpy().view(np.uint64).copy(), outs.cpu().numpy().view(np.uint64).copy()


@pytest.mark.parametrize("order", [("c4", "c3", "c1"), ("c5", "c2", "c0")])
def test_noalloc_norm_matches_the_cached_entry_point(order):
    import torch
    for i, name in enumerate(order):
        cfg, h = _layout(name)
        try:
            N = cfg.world_size
            n_slots, n_part = zs.zs3_layout_norm_slots(h)
            rng = np.random.default_rng(100 + i)
            vals = rng.random(n_slots) * rng.choice([1e-9, 1.0, 1e6], n_slots)
            partials = torch.from_numpy(vals).cuda()
            rank = N - 1
            for finalize, max_norm in ((True, 1.0), (False, 1.0), (True, 1e9)):
                note(f"no-alloc norm: call {i} on {name} ({n_slots} slots), finalize={finalize} max_norm={max_norm}")
                ref = _run(zs.zs3_grad_norm_partials, h, rank, N, partials, finalize, max_norm)
                got = _run(zs.zs3_grad_norm_partials_noalloc, h, rank, N, partials, finalize, max_norm)
                assert np.array_equal(got[0], ref[0]), f"{name}: partial sums differ"
                assert np.array_equal(got[1], ref[1]), f"{name}: norm, scale or flag differ"
            # a non-finite slot: both set the flag the same way
            partials[n_slots // 2] = float("inf")
            note(f"no-alloc norm: call {i} on {name} with an inf slot")
            ref = _run(zs.zs3_grad_norm_partials, h, rank, N, partials, True, 1.0)
            got = _run(zs.zs3_grad_norm_partials_noalloc, h, rank, N, partials, True, 1.0)
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
            assert int(got[1][1:2].view(np.int32)[1]) == 1
        finally:
            zs.zs3_layout_destroy(h)
