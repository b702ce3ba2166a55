"""Pins of the oracle's non-contiguous gradient path: the send-side pack of
reduce_scatter_coalesced and the owner-side reduce (CPU only).

[codex] 6.2 lists two gradient paths that both end with the rank's own
averaged slice in the flat gradient buffer; the non-contiguous one scatters
straight to the owners.  Pins: the [csdn] worked example, an element-by-
element derivation of the wire through the owner map, the round trip
through the all-gather's unpack (the wire of one is the wire of the other),
and bit-for-bit agreement with the contiguous path and with the per-element
brute force.
"""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import brute
from synth import get_config
from synth.gen import grad_host, to16_host

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _exchange(L, dtype, ds_ids, grads):
    """Every virtual rank packs; rank r receives chunk r of every rank's wire."""
    N = L.world_size
    sends = [oracle.scatter_pack(L, ds_ids, grads[v]) for v in range(N)]
    outs = []
    for r in range(N):
        gf = np.full(L.shard_numel, 0xFFFF, np.uint16)
        oracle.scatter_reduce(L, r, dtype, ds_ids, [sends[v][r] for v in range(N)], gf)
        outs.append(gf)
    return sends, outs


def test_worked_example():
    """[csdn] worked example: 4 GPUs, the 4 units as one 4-element parameter,
    every GPU with the same gradients; GPU r keeps the average of unit r."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    N = ex["world_size"]
    L = oracle.make_layout(N, 0, [0], [4])
    g16 = to16_host(np.array(ex["grads_every_rank"], np.float32), "fp16")
    _, outs = _exchange(L, "fp16", [0], [{0: g16} for _ in range(N)])
    for r in range(N):
        assert oracle.to_f32(outs[r], "fp16").tolist() == [ex["averaged"][ex["unit_owned_by_rank"][r]]]
    assert float(oracle.to_f32(outs[0], "fp16")[0]) == ex["gpu0_keeps"]


def _random_case(seed, N, T, n_params, dtype, lo=1, hi=40):
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(lo, hi, n_params)]
    ids = [int(x) for x in rng.permutation(n_params) * 5 + 2]
    L = oracle.make_layout(N, T, ids, numels)
    grads = [{d: to16_host(rng.standard_normal(n).astype(np.float32) * np.float32(1e-2), dtype)
              for d, n in zip(ids, numels)} for _ in range(N)]
    bucket = [p.ds_id for p in L.params if not p.persistent]
    return L, grads, bucket


@settings(max_examples=80, deadline=None)
@given(st.integers(0, 10**6), st.sampled_from([1, 2, 3, 4, 5, 8]), st.integers(1, 6))
def test_wire_through_the_owner_map(seed, N, n_params):
    """Element e of parameter d travels in chunk e // ps at c_d + e % ps
    (brute.owner); every other chunk position is padding and holds 0."""
    L, grads, bucket = _random_case(seed, N, 0, n_params, "bf16")
    chunks = oracle.scatter_pack(L, bucket, grads[0])
    rows, _ = brute.layout_table(N, 0, [p.ds_id for p in L.params], [p.numel for p in L.params])
    expect = [[0] * sum(r[3] for r in rows) for _ in range(N)]
    c = 0
    for d, n, pers, ps, off in rows:
        assert not pers
        for e in range(n):
            r, k = brute.owner(e, ps)
            expect[r][c + k] = int(grads[0][d][e])
        c += ps
    assert [ch.tolist() for ch in chunks] == expect


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10**6), st.sampled_from([1, 2, 3, 4, 8, 64]), st.integers(1, 6))
def test_wire_is_the_all_gather_wire(seed, N, n_params):
    """Unpacking the scatter wire with the all-gather's unpack gives back the
    full gradients: both collectives use the same ds_id-ordered layout."""
    L, grads, bucket = _random_case(seed, N, 0, n_params, "fp16")
    chunks = oracle.scatter_pack(L, bucket, grads[1 % N])
    full, offs = oracle.unpack(L, bucket, chunks)
    for d in bucket:
        n = L.slot(d).numel
        assert np.array_equal(full[offs[d]:offs[d] + n], grads[1 % N][d])


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10**6), st.sampled_from([1, 2, 3, 4, 5, 8]), st.sampled_from(["fp16", "bf16"]),
       st.integers(1, 5))
def test_owner_slices_match_brute_force_and_the_contiguous_path(seed, N, dtype, n_params):
    L, grads, bucket = _random_case(seed, N, 0, n_params, dtype, hi=30)
    _, outs = _exchange(L, dtype, bucket, grads)
    for r in range(N):
        ref = np.full(L.shard_numel, 0xFFFF, np.uint16)
        oracle.reduce_scatter(L, r, dtype, bucket, grads, ref)
        assert np.array_equal(outs[r], ref)
        for p in L.params:
            lo, hi = L.own_range(p, r)
            for k in range(p.partition_size):
                got = int(outs[r][p.shard_offset + k])
                if lo + k >= hi:
                    assert got == 0
                else:
                    vals = [int(grads[v][p.ds_id][lo + k]) for v in range(N)]
                    assert got == brute.reduce_scatter_elem(vals, dtype)


def test_real_config_matches_contiguous_path():
    cfg = get_config("c1")
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    grads = [{d: grad_host(cfg, 0, v, d) for d in cfg.ds_ids} for v in range(cfg.world_size)]
    bucket = [p.ds_id for p in L.params if not p.persistent]
    _, outs = _exchange(L, cfg.dtype, bucket, grads)
    for r in range(cfg.world_size):
        ref = np.full(L.shard_numel, 0xFFFF, np.uint16)
        oracle.reduce_scatter(L, r, cfg.dtype, bucket, grads, ref)
        assert np.array_equal(outs[r], ref)


def test_padding_of_received_chunks_is_ignored():
    """The owner writes 0 at padding positions whatever arrives there."""
    L = oracle.make_layout(4, 0, [0, 1], [10, 7])     # ps 3 and 2; rank 3 owns 1 and 1 real elements
    rng = np.random.default_rng(5)
    grads = [{0: rng.integers(0, 0x3c00, 10).astype(np.uint16), 1: rng.integers(0, 0x3c00, 7).astype(np.uint16)}
             for _ in range(4)]
    sends = [oracle.scatter_pack(L, [0, 1], g) for g in grads]
    recv = [s[3].copy() for s in sends]
    for ch in recv:
        ch[1:3] = 0x7BFF      # padding of parameter 0 in chunk 3
        ch[4] = 0x7BFF        # padding of parameter 1 in chunk 3
    gf = np.full(L.shard_numel, 0xFFFF, np.uint16)
    oracle.scatter_reduce(L, 3, "fp16", [0, 1], recv, gf)
    ref = np.full(L.shard_numel, 0xFFFF, np.uint16)
    oracle.reduce_scatter(L, 3, "fp16", [0, 1], grads, ref)
    assert np.array_equal(gf, ref)
    assert gf[1] == 0 and gf[2] == 0 and gf[4] == 0


def test_persistent_parameters_take_the_all_reduce_path():
    L = oracle.make_layout(2, 10, [0, 1], [4, 50])
    with pytest.raises(ValueError):
        oracle.scatter_pack(L, [0, 1], {0: np.zeros(4, np.uint16), 1: np.zeros(50, np.uint16)})
    with pytest.raises(ValueError):
        oracle.scatter_reduce(L, 0, "fp16", [0], [np.zeros(4, np.uint16)] * 2, np.zeros(L.shard_numel, np.uint16))
