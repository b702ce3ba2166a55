"""The coordinator of the C ABI (zs3_coord_*) against the oracle, event by
event: every gather (kind and ds_ids), every release list, the mode, the
live count and the trace signature, over the workloads' module orders and
random structures, several steps, changed orders and every limit (CPU
only: the coordinator is host code)."""

import random

import pytest
from hypothesis import given, settings, strategies as st

import zero_sharded_state_amd as zs
from oracle import coordinator as co
from synth import get_config
from synth.modules import module_table, step_order


def _pair(numels, thresh, mods, cfg, N=4):
    ids = list(range(len(numels)))
    h = zs.zs3_layout_create(N, thresh, ids, numels)
    c = zs.zs3_coord_create(h, mods, cfg.__dict__)
    o = co.Coordinator({d: n for d, n in zip(ids, numels)}, {d: n < thresh for d, n in zip(ids, numels)},
                       [list(m) for m in mods], cfg)
    return h, c, o


def _same_step(c, o, order, release=True):
    for m in order:
        assert zs.zs3_coord_fetch(c, m) == [(k, g) for k, g in o.fetch(m)], f"fetch {m}"
        if release:
            assert zs.zs3_coord_release(c, m) == o.release(m), f"release {m}"
        info = zs.zs3_coord_info(c)
        assert (info["mode"], info["live_numel"], info["invalidations"]) == (o.mode, o.live, o.invalidations)


def _run(c, o, orders):
    for order in orders:
        _same_step(c, o, order)
        assert zs.zs3_coord_release_all(c) == o.release_all()
        assert zs.zs3_coord_reset_step(c) == o.reset_step()
        assert zs.zs3_coord_trace_signature(c) == o.signature()


CFGS = [co.CoordConfig(), co.CoordConfig(int(5e7), int(2e8), 0), co.CoordConfig(int(1e6), int(1e9), int(5e8)),
        co.CoordConfig(0, int(1e12), 0), co.CoordConfig(int(2e8), int(3e8), int(2e9))]


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("ci", range(len(CFGS)))
def test_workload_orders_match_oracle(name, ci):
    cfg = get_config(name)
    _, mods = module_table(cfg)
    order = step_order(cfg)
    h, c, o = _pair(cfg.numels, cfg.threshold, mods, CFGS[ci], cfg.world_size)
    try:
        changed = order[:3] + order[4:3:-1] + order[3:4] + order[5:] if len(order) > 5 else order[::-1]
        _run(c, o, [order, order, order, order, changed, changed, changed, order])
        for d in range(len(cfg.numels)):
            if any(d in m for m in mods):
                assert zs.zs3_coord_param_status(c, d) == o.status[d]
    finally:
        zs.zs3_coord_destroy(c)
        zs.zs3_layout_destroy(h)


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 10**7))
def test_random_structures_match_oracle(seed):
    rng = random.Random(seed)
    n_p = rng.randint(1, 14)
    numels = [rng.randint(1, 60) for _ in range(n_p)]
    thresh = rng.choice([0, 5, 20])
    mods = [rng.sample(range(n_p), rng.randint(1, min(4, n_p))) for _ in range(rng.randint(1, 7))]
    order = [rng.randrange(len(mods)) for _ in range(rng.randint(1, 14))]
    other = [rng.randrange(len(mods)) for _ in range(rng.randint(1, 14))]
    cfg = co.CoordConfig(rng.choice([0, 1, 30, 100]), rng.choice([0, 40, 200, 10**9]), rng.choice([0, 25, 10**9]))
    h, c, o = _pair(numels, thresh, mods, cfg, rng.randint(1, 8))
    try:
        steps = [order] * 3 + [other if rng.random() < 0.3 else order for _ in range(4)]
        for s in steps:
            # releases in a shuffled subset: modules may stay fetched until release_all
            for m in s:
                assert zs.zs3_coord_fetch(c, m) == o.fetch(m)
                if rng.random() < 0.8:
                    assert zs.zs3_coord_release(c, m) == o.release(m)
            assert zs.zs3_coord_info(c)["live_numel"] == o.live
            assert zs.zs3_coord_release_all(c) == o.release_all()
            assert zs.zs3_coord_reset_step(c) == o.reset_step()
            assert zs.zs3_coord_trace_signature(c) == o.signature()
    finally:
        zs.zs3_coord_destroy(c)
        zs.zs3_layout_destroy(h)


def test_signatures_tell_orders_apart():
    cfg = co.CoordConfig()
    h = zs.zs3_layout_create(2, 0, [0, 1, 2], [10, 20, 30])
    a = zs.zs3_coord_create(h, [[0], [1, 2], [2]], cfg.__dict__)
    b = zs.zs3_coord_create(h, [[0], [1, 2], [2]], cfg.__dict__)
    try:
        for c, order in ((a, [0, 1, 2]), (b, [0, 2, 1])):
            for _ in range(2):
                for m in order:
                    zs.zs3_coord_fetch(c, m)
                zs.zs3_coord_release_all(c)
                zs.zs3_coord_reset_step(c)
        sa, sb = zs.zs3_coord_trace_signature(a), zs.zs3_coord_trace_signature(b)
        assert sa[2] == sb[2] == 3
        assert sa[0] != sb[0] and sa[1] != sb[1]
        assert sa[0] == co.fnv1a64([0, 1, 2]) and sa[1] == co.fnv1a64([0, 1, 2, 2])
    finally:
        zs.zs3_coord_destroy(a)
        zs.zs3_coord_destroy(b)
        zs.zs3_layout_destroy(h)


def test_coordinator_validation():
    h = zs.zs3_layout_create(2, 0, [0, 1], [10, 20])
    cfg = {"prefetch_bucket_size": 10, "max_live_parameters": 100, "max_reuse_distance": 0}
    try:
        with pytest.raises(zs.Zs3Error) as e:
            zs.zs3_coord_create(h, [[0, 0]], cfg)
        assert e.value.status == zs.ZS3_EDUPID
        with pytest.raises(zs.Zs3Error) as e:
            zs.zs3_coord_create(h, [[5]], cfg)
        assert e.value.status == zs.ZS3_ENOTFOUND
        with pytest.raises(zs.Zs3Error) as e:
            zs.zs3_coord_create(h, [[0]], dict(cfg, max_reuse_distance=-1))
        assert e.value.status == zs.ZS3_EINVAL
        c = zs.zs3_coord_create(h, [[0], [1]], cfg)
        try:
            with pytest.raises(zs.Zs3Error) as e:
                zs.zs3_coord_fetch(c, 2)
            assert e.value.status == zs.ZS3_EINVAL
            with pytest.raises(zs.Zs3Error) as e:
                zs.zs3_coord_release(c, 1)                 # not fetched
            assert e.value.status == zs.ZS3_EINVAL
            zs.zs3_coord_fetch(c, 1)
            assert zs.zs3_coord_release(c, 1) == [1]
            with pytest.raises(zs.Zs3Error):
                zs.zs3_coord_release(c, 1)                 # released already
            with pytest.raises(zs.Zs3Error) as e:
                zs.zs3_coord_param_status(c, 7)
            assert e.value.status == zs.ZS3_ENOTFOUND
        finally:
            zs.zs3_coord_destroy(c)
    finally:
        zs.zs3_layout_destroy(h)
