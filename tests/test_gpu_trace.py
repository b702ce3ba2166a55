"""GPU parity of the gathers the fetch/release coordinator drives: after a
coordinator-driven forward+backward pass, every gather's buffer holds the
bucket's full parameters exactly as the oracle's pack + unpack gives them
(through the C ABI, on the workloads' module orders), with the gathers on
one stream or dealt over two."""

import numpy as np
import pytest

import oracle
from synth import get_config
from synth.gen import weights_host
from synth.modules import module_table, step_order

from gpu_util import note, require_gpu, sync

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _step(cfg, rank, gather_streams=1):
    from zero_sharded_state_amd.shard_step import AdamConfig, ShardStep
    return ShardStep(world_size=cfg.world_size, rank=rank, threshold=cfg.threshold, ds_ids=cfg.ds_ids,
                     numels=cfg.numels, dtype=cfg.dtype, prefetch_bucket_size=cfg.prefetch_bucket_size,
                     reduce_bucket_size=cfg.reduce_bucket_size, sub_group_size=cfg.sub_group_size,
                     adam=AdamConfig(), max_norm=cfg.max_norm, gather_streams=gather_streams)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rank,cc,streams", [
    ("c1", 1, (64, 10**9, 0), 1),
    ("c2", 0, (int(5e7), int(1e9), int(1e9)), 1),
    ("c2", 0, (int(5e7), int(1e9), int(1e9)), 2),
    ("c2", 5, (int(1e6), int(2e7), 0), 2),
    ("c3", 7, (int(5e7), int(1e9), int(1e9)), 1),
    ("c3", 7, (int(5e7), int(1e9), int(1e9)), 2),
    ("c3", 0, (int(2e7), int(6e7), int(3e7)), 1),
])
def test_coordinator_driven_gathers_match_oracle(name, rank, cc, streams):
    import torch
    from zero_sharded_state_amd.trace_schedule import TraceGatherPass
    cfg = get_config(name)
    N = cfg.world_size
    step = _step(cfg, rank, streams)
    L = oracle.make_layout(N, cfg.threshold, cfg.ds_ids, cfg.numels)
    tp = None
    try:
        full = {d: weights_host(cfg, d) for d in cfg.ds_ids}
        for d in cfg.ds_ids:
            p = step.by_id[d]
            buf, o = (step.pers_full, step.pers_off[d]) if p["persistent"] else (step.full, step.full_off[d])
            buf[o:o + p["numel"]].copy_(torch.from_numpy(full[d].view(np.int16)))
        step.init_from_full()
        _, mods = module_table(cfg)
        tp = TraceGatherPass(step, mods, step_order(cfg), {"prefetch_bucket_size": cc[0],
                                                          "max_live_parameters": cc[1], "max_reuse_distance": cc[2]})
        tp.plan()
        note(f"trace gathers {name} rank={rank} cfg={cc} streams={streams}: {len(tp.ops)} gathers")
        tp.fill_peer_chunks()
        tp.full.fill_(0x5A5A)
        for _ in range(2):
            assert tp.run() == len(tp.ops)
        sync()
        got = tp.full.cpu().numpy().view(np.uint16)
        shards = [oracle.partition(L, v, full) for v in range(N)]
        for g, (fo, n, _, _) in zip(tp.ops, tp.meta):
            ref, offs = oracle.unpack(L, g, [oracle.pack(L, v, g, shards[v]) for v in range(N)])
            assert np.array_equal(got[fo:fo + n], ref), f"gather {g}"
            for d in g:
                assert np.array_equal(got[fo + offs[d]:fo + offs[d] + full[d].size], full[d])
        # every partitioned parameter is gathered at least once per step, none is persistent
        seen = {d for g in tp.ops for d in g}
        assert seen == {p.ds_id for p in L.params if not p.persistent}
    finally:
        if tp is not None:
            tp.destroy()
        step.destroy()
