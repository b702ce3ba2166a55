"""The C ABI without a GPU: the library loads, exports every declared
symbol, its host-side planner agrees with the oracle exactly, and invalid
arguments are rejected before any device work (CPU only)."""

import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import zero_sharded_state_amd as zs
from synth import CONFIGS, get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "zs3.h")).read()
    return sorted(set(re.findall(r"ZS3_API\s+[\w\s\*]*?\b(zs3_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return zs.lib()


def test_library_exports_every_declared_symbol(L):
    syms = _declared_symbols()
    assert len(syms) == 35
    assert sorted(zs.EXPORTS) == syms
    for s in syms:
        assert hasattr(L, s), s
    assert zs.zs3_abi_version() == 3
    assert zs.zs3_status_str(-5).startswith("persistent")


def _both(cfg_or_args):
    if isinstance(cfg_or_args, str):
        cfg = get_config(cfg_or_args)
        args = (cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    else:
        args = cfg_or_args
    h = zs.zs3_layout_create(*args)
    return h, oracle.make_layout(*args)


def _assert_same_layout(h, ol):
    info = zs.zs3_layout_info(h)
    assert info["world_size"] == ol.world_size
    assert info["n_params"] == len(ol.params)
    assert info["shard_numel"] == ol.shard_numel
    assert info["bytes_per_rank"] == ol.bytes_per_rank
    assert zs.zs3_layout_totals(h) == (ol.shard_numel, ol.bytes_per_rank)
    for i, p in enumerate(ol.params):
        q = zs.zs3_layout_param_at(h, i)
        assert (q["ds_id"], q["numel"], q["partition_size"], q["persistent"], q["shard_offset"]) == \
               (p.ds_id, p.numel, p.partition_size, p.persistent, p.shard_offset)
        assert zs.zs3_layout_param(h, p.ds_id) == q
        for r in sorted({0, ol.world_size - 1, ol.world_size // 2}):
            assert zs.zs3_layout_own_range(h, p.ds_id, r) == ol.own_range(p, r)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_layout_and_plans_match_oracle(name):
    cfg = get_config(name)
    h, ol = _both(name)
    try:
        _assert_same_layout(h, ol)
        assert zs.zs3_plan_buckets(h, zs.ZS3_GATHER_BUCKETS, cfg.prefetch_bucket_size) == \
            oracle.gather_buckets(ol, cfg.prefetch_bucket_size)
        assert zs.zs3_plan_buckets(h, zs.ZS3_REDUCE_BUCKETS, cfg.reduce_bucket_size) == \
            oracle.reduce_buckets(ol, cfg.reduce_bucket_size)
        assert zs.zs3_sub_groups(h, cfg.sub_group_size) == oracle.sub_groups(ol, cfg.sub_group_size)
        for b in oracle.gather_buckets(ol, cfg.prefetch_bucket_size)[:5]:
            assert zs.zs3_bucket_sizes(h, b[::-1]) == oracle.bucket_sizes(ol, b)
    finally:
        zs.zs3_layout_destroy(h)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 70), st.integers(0, 60), st.lists(st.integers(1, 500), min_size=0, max_size=12),
       st.integers(0, 10**6), st.integers(1, 3000))
def test_random_layouts_match_oracle(N, T, numels, seed, limit):
    ids = list(np.random.default_rng(seed).permutation(len(numels)) * 3 + 1)
    h, ol = _both((N, T, ids, numels))
    try:
        _assert_same_layout(h, ol)
        assert zs.zs3_plan_buckets(h, zs.ZS3_GATHER_BUCKETS, limit) == oracle.gather_buckets(ol, limit)
        assert zs.zs3_plan_buckets(h, zs.ZS3_REDUCE_BUCKETS, limit) == oracle.reduce_buckets(ol, limit)
        assert zs.zs3_sub_groups(h, limit) == oracle.sub_groups(ol, limit)
    finally:
        zs.zs3_layout_destroy(h)


def test_layout_create_errors():
    with pytest.raises(zs.Zs3Error) as e:
        zs.zs3_layout_create(0, 0, [0], [1])
    assert e.value.status == zs.ZS3_EINVAL
    with pytest.raises(zs.Zs3Error) as e:
        zs.zs3_layout_create(2, 0, [3, 3], [1, 2])
    assert e.value.status == zs.ZS3_EDUPID
    with pytest.raises(zs.Zs3Error) as e:
        zs.zs3_layout_create(2, 0, [3], [0])
    assert e.value.status == zs.ZS3_EINVAL and "numel" in e.value.message
    with pytest.raises(zs.Zs3Error) as e:
        zs.zs3_layout_create(2, 0, [-1], [4])
    assert e.value.status == zs.ZS3_EINVAL


def test_call_validation_enqueues_nothing():
    """Each of these fails during validation, before any HIP call."""
    h = zs.zs3_layout_create(4, 10, [0, 1, 2], [100, 5, 33])   # ds_id 1 persistent
    S = zs.zs3_layout_info(h)["shard_numel"]
    base = 1 << 40     # fake, never dereferenced: every call below is rejected first
    try:
        cases = [
            (zs.ZS3_EDTYPE, lambda: zs.zs3_partition(h, 0, 7, [0], [base], base + 4096, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_partition(h, 4, "fp16", [0], [base], base + 4096, stream=0)),
            (zs.ZS3_ENOTFOUND, lambda: zs.zs3_partition(h, 0, "fp16", [9], [base], base + 4096, stream=0)),
            (zs.ZS3_EDUPID, lambda: zs.zs3_partition(h, 0, "fp16", [0, 0], [base, base], base + 4096, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_partition(h, 0, "fp16", [0], [base], base + 10, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_partition(h, 0, "fp16", [0], [base + 1], base + 4096, stream=0)),
            (zs.ZS3_EPERSIST, lambda: zs.zs3_gather_coalesced(h, 0, "bf16", zs.ZS3_PACK, [1], base, base + 4096,
                                                              stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_gather_coalesced(h, 0, "bf16", 4, [0], base, base + 4096, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_gather_coalesced(h, 0, "bf16", zs.ZS3_PACK, [0, 2], base, base + 2 * S - 2,
                                                            stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_gather_coalesced(h, 0, "bf16", zs.ZS3_UNPACK, [0], None, None,
                                                            [base + 4096 * v for v in range(4)], base + 8192,
                                                            stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_gather_coalesced(h, 0, "bf16", zs.ZS3_UNPACK, [0], None, None,
                                                            [base] * 3 + [0], base + 1 << 20, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_reduce_scatter_local(h, 0, "bf16", [0], [base + 2 * k for k in range(4)],
                                                                base, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_grad_norm(h, 0, "bf16", base, base + 4096 + 4, True, 1.0, 1.0,
                                                     base + 8192, base + 8200, base + 8204, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_grad_norm(h, 0, "bf16", base, base + 4096, True, 0.0, 1.0,
                                                     base + 8192, base + 8200, base + 8204, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_adam_step(h, 0, "bf16", 0, S + 1, base, base + 1 << 20, base + 2 << 20,
                                                     base + 3 << 20, base + 4 << 20, base + 5 << 20, None,
                                                     {"lr": 1e-3, "beta1": .9, "beta2": .999, "eps": 1e-8, "step": 1},
                                                     stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_adam_step(h, 0, "bf16", 0, S, base, base + 1 << 20, base + 2 << 20,
                                                     base + 3 << 20, base + 4 << 20, base + 5 << 20, None,
                                                     {"lr": 1e-3, "beta1": .9, "beta2": .999, "eps": 1e-8, "step": 0},
                                                     stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_adam_step(h, 0, "bf16", 0, S, base, base + 8, base + (2 << 20),
                                                     base + (3 << 20), base + (4 << 20), base + (5 << 20), None,
                                                     {"lr": 1e-3, "beta1": .9, "beta2": .999, "eps": 1e-8, "step": 1},
                                                     stream=0)),
            (zs.ZS3_EPERSIST, lambda: zs.zs3_reduce_scatter_coalesced(h, 0, "bf16", zs.ZS3_PACK, [0, 1],
                                                                      grads=[base, base + 4096], send=base + 8192,
                                                                      stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_reduce_scatter_coalesced(h, 0, "bf16", zs.ZS3_UNPACK, [0],
                                                                    grads=[base], send=base + 8192, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_reduce_scatter_coalesced(h, 0, "bf16", zs.ZS3_PACK, [0],
                                                                    grads=None, send=base + 8192, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_reduce_scatter_coalesced(h, 0, "bf16", zs.ZS3_PACK, [0],
                                                                    grads=[base], send=base + 100, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_reduce_scatter_coalesced(h, 0, "bf16", zs.ZS3_REDUCE, [0, 2],
                                                                    recv_chunks=[base + 4096 * k for k in range(4)],
                                                                    grad_flat=base + 4096 * 3 - 2, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_reduce_scatter_coalesced(h, 0, "bf16", zs.ZS3_REDUCE, [0],
                                                                    recv_chunks=[base + 4096 * k for k in range(4)],
                                                                    grad_flat=base + 65536, partials=base + 65536 * 2 + 4,
                                                                    stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_reduce_scatter_local(h, 0, "bf16", [0], [base + 4096 * k for k in range(4)],
                                                                base + 65536, partials=base + 65536 + 8, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_grad_norm_partials(h, 0, base + 4, base + 8192, False, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_grad_norm_partials(h, 0, base, base + 1 << 20, True, 0.0, 1.0,
                                                              base + 8192, base + 8200, base + 8204, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_grad_norm_partials(h, 0, base, base + 8, False, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_grad_norm_partials_noalloc(h, 0, base + 4, base + 8192, False, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_grad_norm_partials_noalloc(h, 0, base, base + 8, False, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_grad_norm_partials_noalloc(h, 7, base, base + 8192, False, stream=0)),
            # several gather buckets in one launch
            (zs.ZS3_EINVAL, lambda: zs.zs3_gather_coalesced_buckets(h, 0, "bf16", [[0], []], base,
                                                                    [base + 4096, base + 8192],
                                                                    [[base + 4096] * 4, [base + 8192] * 4],
                                                                    [base + 65536, base + 131072], stream=0)),
            (zs.ZS3_EDUPID, lambda: zs.zs3_gather_coalesced_buckets(h, 0, "bf16", [[0], [2, 0]], base,
                                                                    [base + 4096, base + 8192],
                                                                    [[base + 4096] + [base + 16384] * 3,
                                                                     [base + 8192] + [base + 24576] * 3],
                                                                    [base + 65536, base + 131072], stream=0)),
            (zs.ZS3_EPERSIST, lambda: zs.zs3_gather_coalesced_buckets(h, 0, "bf16", [[1]], base, [base + 4096],
                                                                      [[base + 4096] * 4], [base + 65536],
                                                                      stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_gather_coalesced_buckets(h, 0, "bf16", [[0]], base, [base + 4096],
                                                                    [[base + 8192] * 4], [base + 65536], stream=0)),
            # bucket 1's gathered buffer overlaps bucket 0's own chunk
            (zs.ZS3_EALIAS, lambda: zs.zs3_gather_coalesced_buckets(h, 0, "bf16", [[0], [2]], base,
                                                                    [base + 4096, base + 8192],
                                                                    [[base + 4096] + [base + 16384] * 3,
                                                                     [base + 8192] + [base + 24576] * 3],
                                                                    [base + 65536, base + 4100], stream=0)),
            # a peer's chunk of bucket 1 overlaps bucket 0's gathered buffer
            (zs.ZS3_EALIAS, lambda: zs.zs3_gather_coalesced_buckets(h, 0, "bf16", [[0], [2]], base,
                                                                    [base + 4096, base + 8192],
                                                                    [[base + 4096] + [base + 16384] * 3,
                                                                     [base + 8192] + [base + 65600] * 3],
                                                                    [base + 65536, base + 131072], stream=0)),
            # the fp32 master partition
            (zs.ZS3_EINVAL, lambda: zs.zs3_init_master(h, 0, "bf16", 0, S + 1, base, base + (1 << 20), stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_init_master(h, 0, "bf16", 5, 4, base, base + (1 << 20), stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_init_master(h, 0, "bf16", 0, S, base, base + (1 << 20) + 2, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_init_master(h, 0, "bf16", 0, S, base, None, stream=0)),
            (zs.ZS3_EDTYPE, lambda: zs.zs3_init_master(h, 0, 3, 0, S, base, base + (1 << 20), stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_init_master(h, 4, "bf16", 0, S, base, base + (1 << 20), stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_init_master(h, 0, "bf16", 0, S, base, base + 8, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_init_master(h, 0, "bf16", 0, S, base, base + (1 << 20),
                                                       base + (1 << 20) + 4 * S - 4, stream=0)),
            # offloaded Adam: every check below runs before any HIP call
            (zs.ZS3_EINVAL, lambda: zs.zs3_adam_step_offload(h, 0, "bf16", 0, S, base, base + (1 << 20),
                                                             base + (2 << 20), base + (3 << 20), 95,
                                                             base + (4 << 20), base + (5 << 20), base + (6 << 20),
                                                             None, {"lr": 1e-3, "beta1": .9, "beta2": .999,
                                                                    "eps": 1e-8, "step": 1}, stream=0)),
            (zs.ZS3_EINVAL, lambda: zs.zs3_adam_step_offload(h, 0, "bf16", 0, S, 0, base + (1 << 20),
                                                             base + (2 << 20), base + (3 << 20), 1 << 12,
                                                             base + (4 << 20), base + (5 << 20), base + (6 << 20),
                                                             None, {"lr": 1e-3, "beta1": .9, "beta2": .999,
                                                                    "eps": 1e-8, "step": 1}, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_adam_step_offload(h, 0, "bf16", 0, S, base, base + 4,
                                                             base + (2 << 20), base + (3 << 20), 1 << 12,
                                                             base + (4 << 20), base + (5 << 20), base + (6 << 20),
                                                             None, {"lr": 1e-3, "beta1": .9, "beta2": .999,
                                                                    "eps": 1e-8, "step": 1}, stream=0)),
            (zs.ZS3_EALIAS, lambda: zs.zs3_adam_step_offload(h, 0, "bf16", 0, S, base, base + (1 << 20),
                                                             base + (2 << 20), base + (3 << 20), 1 << 12,
                                                             base + (3 << 20) + 64, base + (5 << 20),
                                                             base + (6 << 20), None,
                                                             {"lr": 1e-3, "beta1": .9, "beta2": .999,
                                                              "eps": 1e-8, "step": 1}, stream=0)),
        ]
        for want, call in cases:
            with pytest.raises(zs.Zs3Error) as e:
                call()
            assert e.value.status == want, (want, e.value)
            assert zs.zs3_last_error() != ""
        # an empty request is a no-op, not an error
        zs.zs3_partition(h, 0, "fp16", [], [], base, stream=0)
        assert zs.zs3_gather_coalesced(h, 0, "fp16", zs.ZS3_PACK, [], base, base + 4096, stream=0) == []
        zs.zs3_reduce_scatter_coalesced(h, 0, "fp16", zs.ZS3_PACK | zs.ZS3_REDUCE, [], grads=[], send=base,
                                        recv_chunks=[base] * 4, grad_flat=base + 65536, stream=0)
        zs.zs3_init_master(h, 0, "fp16", 3, 3, base, base + (1 << 20), stream=0)
        zs.zs3_gather_coalesced_buckets(h, 0, "fp16", [], base, [], [], [], stream=0)
    finally:
        zs.zs3_layout_destroy(h)


def _slot_count(ps_list, piece=256 * 2 * 8 * 8, per_piece=8 * 4):
    return sum(per_piece * (1 if ps <= piece else -(-ps // piece)) for ps in ps_list)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_norm_slots_cover_every_parameter(name):
    """One group of slots (one per wave of the piece's workgroups) per
    reduce-scatter piece of each parameter's partition, partitioned
    parameters first."""
    cfg = get_config(name)
    h, ol = _both(name)
    try:
        n_slots, n_part = zs.zs3_layout_norm_slots(h)
        assert n_part == _slot_count([p.partition_size for p in ol.params if not p.persistent])
        assert n_slots == n_part + _slot_count([p.partition_size for p in ol.params if p.persistent])
    finally:
        zs.zs3_layout_destroy(h)


def test_noalloc_norm_rejects_layouts_past_its_scratch():
    """The allocation-free norm's limit is checked before any device work: a
    layout whose slot array is larger than 1024 * 65536 slots is refused
    with a message (the layout itself is host-only, never allocated)."""
    h = zs.zs3_layout_create(1, 0, [0], [1 << 37])
    try:
        n_slots, _ = zs.zs3_layout_norm_slots(h)
        assert n_slots > 1024 * 65536
        base = 1 << 40     # fake, never dereferenced
        with pytest.raises(zs.Zs3Error) as e:
            zs.zs3_grad_norm_partials_noalloc(h, 0, base, base + 8 * n_slots + 4096, True, 1.0, 1.0,
                                              base + 8 * n_slots + 8192, base + 8 * n_slots + 8200,
                                              base + 8 * n_slots + 8204, stream=0)
        assert e.value.status == zs.ZS3_EINVAL and "at most" in e.value.message
    finally:
        zs.zs3_layout_destroy(h)
