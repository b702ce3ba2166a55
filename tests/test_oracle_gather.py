"""Pins of the oracle's coalesced gather (pack, wire, unpack), CPU only."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import brute
from synth import get_config
from synth.gen import weights_host


def _random_problem(seed, N, T, n_params, max_numel=40):
    rng = np.random.default_rng(seed)
    ds_ids = list(rng.permutation(np.arange(n_params) * 5 + 3))
    numels = list(rng.integers(1, max_numel + 1, n_params))
    full = {int(d): rng.integers(0, 1 << 16, int(n), dtype=np.uint16) for d, n in zip(ds_ids, numels)}
    return oracle.make_layout(N, T, ds_ids, numels), full


def _gather_all(L, full, buckets):
    N = L.world_size
    shards = [oracle.partition(L, r, full) for r in range(N)]
    out = {}
    for b in buckets:
        chunks = [oracle.pack(L, r, b, shards[r]) for r in range(N)]
        flat, offs = oracle.unpack(L, b, chunks)
        for d, o in offs.items():
            out[d] = flat[o:o + L.slot(d).numel]
    return out, shards


@settings(max_examples=120, deadline=None)
@given(st.integers(0, 10**6), st.sampled_from([1, 2, 3, 4, 8]), st.sampled_from([0, 5, 20]),
       st.integers(1, 7), st.sampled_from([1, 10, 60, 10**9]))
def test_partition_then_gather_is_identity(seed, N, T, n_params, limit):
    L, full = _random_problem(seed, N, T, n_params)
    buckets = oracle.gather_buckets(L, limit)
    got, _ = _gather_all(L, full, buckets)
    for p in L.params:
        if not p.persistent:
            assert np.array_equal(got[p.ds_id], full[p.ds_id])


@settings(max_examples=80, deadline=None)
@given(st.integers(0, 10**6), st.sampled_from([1, 2, 3, 4, 8]), st.integers(1, 6))
def test_unpack_matches_element_by_element_brute_force(seed, N, n_params):
    L, full = _random_problem(seed, N, 0, n_params)
    ds_ids = [p.ds_id for p in L.params]
    numels = [p.numel for p in L.params]
    shards = [oracle.partition(L, r, full) for r in range(N)]
    bucket = ds_ids[::-1]
    chunks = [oracle.pack(L, r, bucket, shards[r]) for r in range(N)]
    flat, offs = oracle.unpack(L, bucket, chunks)
    bf_flat, bf_offs = brute.gather_full(N, 0, ds_ids, numels,
                                         [list(map(int, s)) for s in shards], bucket)
    assert list(map(int, flat)) == bf_flat
    assert offs == bf_offs


def test_request_order_does_not_matter():
    L, full = _random_problem(7, 4, 0, 6)
    shards = [oracle.partition(L, r, full) for r in range(4)]
    ids = [p.ds_id for p in L.params]
    rng = np.random.default_rng(1)
    ref_chunks = [oracle.pack(L, r, ids, shards[r]) for r in range(4)]
    ref_flat, ref_offs = oracle.unpack(L, ids, ref_chunks)
    for _ in range(5):
        perm = list(rng.permutation(ids))
        chunks = [oracle.pack(L, r, perm, shards[r]) for r in range(4)]
        for a, b in zip(chunks, ref_chunks):
            assert np.array_equal(a, b)
        flat, offs = oracle.unpack(L, perm, chunks)
        assert np.array_equal(flat, ref_flat) and offs == ref_offs


def test_wire_is_rank_major_and_views_are_ds_id_ordered():
    cfg = get_config("c1")
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    full = {d: weights_host(cfg, d) for d in cfg.ds_ids}
    shards = [oracle.partition(L, r, full) for r in range(4)]
    chunks = [oracle.pack(L, r, cfg.ds_ids, shards[r]) for r in range(4)]
    w = oracle.wire(chunks)
    assert w.size == 4 * 652
    for r in range(4):
        assert np.array_equal(w[r * 652:(r + 1) * 652], chunks[r])
    flat, offs = oracle.unpack(L, cfg.ds_ids, chunks)
    assert offs == {0: 0, 1: 2048, 2: 2080, 3: 2592}
    assert flat.size == 2608
    assert oracle.bucket_sizes(L, cfg.ds_ids) == (652, 2608)


def test_gather_rejects_persistent_and_duplicates():
    L = oracle.make_layout(2, 10, [0, 1], [4, 40])
    with pytest.raises(ValueError):
        oracle.pack(L, 0, [0], np.zeros(L.shard_numel, np.uint16))
    with pytest.raises(ValueError):
        oracle.pack(L, 0, [1, 1], np.zeros(L.shard_numel, np.uint16))
    with pytest.raises(KeyError):
        oracle.pack(L, 0, [5], np.zeros(L.shard_numel, np.uint16))


def test_bucket_size_does_not_change_full_params():
    L, full = _random_problem(11, 3, 5, 9, max_numel=60)
    results = []
    for limit in (1, 30, 100, 10**9):
        got, _ = _gather_all(L, full, oracle.gather_buckets(L, limit))
        results.append(got)
    for r in results[1:]:
        assert r.keys() == results[0].keys()
        for d in r:
            assert np.array_equal(r[d], results[0][d])
