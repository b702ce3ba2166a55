"""Pins of the oracle's layout, partition and bucket plans (CPU only)."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import brute
from synth import get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layout(cfg):
    return oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)


def test_c1_partition_sizes_and_16psi_over_n():
    cfg = get_config("c1")
    L = _layout(cfg)
    assert [p.partition_size for p in L.params] == [512, 8, 128, 4]
    assert [p.shard_offset for p in L.params] == [0, 512, 520, 648]
    assert L.shard_numel == 652
    psi = cfg.total_params
    assert psi == 2608
    # 16 Psi / N bytes per rank when every numel divides by N
    assert L.bytes_per_rank == 16 * psi // cfg.world_size == 10432


def test_accounting_120gb_for_7p5b():
    g = json.load(open(os.path.join(GOLDEN, "accounting.json")))
    b = g["bytes_per_param"]
    assert b["param"] + b["grad"] + b["optimizer"] == b["total"] == 16
    assert b["optimizer"] // b["param"] == g["optimizer_over_param"]
    m = g["model_7p5b"]
    n = m["params"]
    # N = 1 holds everything: one persistent-free layout of the 7.5B elements
    L = oracle.make_layout(1, 0, [0, 1, 2], [n // 3, n // 3, n - 2 * (n // 3)])
    assert L.shard_numel == n
    assert L.bytes_per_rank == m["total_gb"] * 10**9
    assert 2 * n == m["param_gb"] * 10**9 == m["grad_gb"] * 10**9
    assert 12 * n == m["optimizer_gb"] * 10**9
    # and 1/N of it per rank when sharded over N ranks with divisible sizes
    for N in (2, 4, 8, 64):
        L = oracle.make_layout(N, 0, [0], [n])
        assert L.bytes_per_rank * N == 16 * n


@pytest.mark.parametrize("name,total,S,P,npers,npad", [
    ("c2", 124_439_808, 15_539_808, 121_344, 98, 0),
    ("c3", 218_112_000, 27_262_976, 8_192, 2, 0),
    ("c4", 8_030_261_248, 1_003_749_376, 266_240, 65, 0),
    ("c5", 7_461_217_053, 116_551_583, 1_924_758, 290, 145),
])
def test_config_shapes(name, total, S, P, npers, npad):
    cfg = get_config(name)
    assert cfg.total_params == total
    L = _layout(cfg)
    pers = [p for p in L.params if p.persistent]
    part = [p for p in L.params if not p.persistent]
    assert sum(p.partition_size for p in part) == S
    assert sum(p.numel for p in pers) == P
    assert L.shard_numel == S + P
    assert len(pers) == npers
    assert sum(1 for p in part if p.numel % cfg.world_size) == npad


def test_c5_rank63_real_elements():
    cfg = get_config("c5")
    L = _layout(cfg)
    real = sum(L.own_range(p, 63)[1] - L.own_range(p, 63)[0] for p in L.params if not p.persistent)
    assert real == 116_542_566
    assert sum(p.partition_size * 64 - p.numel for p in L.params if not p.persistent) == 9_017


@pytest.mark.parametrize("name,ng,nr,subs", [
    ("c1", 1, 1, None),
    ("c2", 3, 20, None),
    ("c3", 4, 8, None),
    ("c4", 130, 258, [(0, 938_348_544), (938_348_544, 938_348_544 + 65_667_072)]),
    ("c5", 146, 218, None),
])
def test_bucket_and_subgroup_plans(name, ng, nr, subs):
    cfg = get_config(name)
    L = _layout(cfg)
    gb = oracle.gather_buckets(L, cfg.prefetch_bucket_size)
    rb = oracle.reduce_buckets(L, cfg.reduce_bucket_size)
    assert len(gb) == ng
    assert len(rb) == nr
    # every non-persistent param in exactly one gather bucket, every param in one reduce bucket
    assert sorted(d for b in gb for d in b) == [p.ds_id for p in L.params if not p.persistent]
    assert sorted(d for b in rb for d in b) == [p.ds_id for p in L.params]
    for b in gb:
        assert len(b) == 1 or sum(L.slot(d).numel for d in b) <= cfg.prefetch_bucket_size
    sg = oracle.sub_groups(L, cfg.sub_group_size)
    assert sg[0][0] == 0 and sg[-1][1] == L.shard_numel
    assert all(a[1] == b[0] for a, b in zip(sg, sg[1:]))
    if subs is not None:
        assert sg == subs


def test_c3_gather_buckets_are_qkvo_gate_up_down():
    cfg = get_config("c3")
    L = _layout(cfg)
    assert oracle.gather_buckets(L, cfg.prefetch_bucket_size) == [[0, 1, 2, 3], [4], [5], [6]]


def test_layout_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.make_layout(0, 0, [0], [1])
    with pytest.raises(ValueError):
        oracle.make_layout(2, 0, [0, 0], [1, 1])
    with pytest.raises(ValueError):
        oracle.make_layout(2, 0, [0], [0])


small_layouts = st.integers(1, 6).flatmap(lambda n: st.tuples(
    st.sampled_from([1, 2, 3, 4, 8]),
    st.sampled_from([0, 5, 20]),
    st.permutations(list(range(0, 3 * n, 3)))  # ds_ids, shuffled, with gaps
    , st.lists(st.integers(1, 40), min_size=n, max_size=n)))


@settings(max_examples=150, deadline=None)
@given(small_layouts, st.data())
def test_partition_matches_brute_force_and_concatenates_to_padded_flat(lay, data):
    N, T, ds_ids, numels = lay
    L = oracle.make_layout(N, T, ds_ids, numels)
    full = {d: np.arange(1, n + 1, dtype=np.uint16) * 7 + d for d, n in zip(ds_ids, numels)}
    shards = [oracle.partition(L, r, full) for r in range(N)]
    for r in range(N):
        bf = brute.partition(N, T, ds_ids, numels, {d: list(map(int, full[d])) for d in full}, r)
        assert list(map(int, shards[r])) == bf
    for p in L.params:
        cat = np.concatenate([s[p.shard_offset:p.shard_offset + p.partition_size] for s in shards])
        if p.persistent:
            for s in shards:
                assert np.array_equal(s[p.shard_offset:p.shard_offset + p.numel], full[p.ds_id])
        else:
            padded = np.zeros(N * p.partition_size, np.uint16)
            padded[:p.numel] = full[p.ds_id]
            assert np.array_equal(cat, padded)
