"""Pins of the oracle's local reduce-scatter (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import brute
from synth import get_config
from synth.gen import grad_host, to16_host

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ex():
    return json.load(open(os.path.join(GOLDEN, "worked_example.json")))


def _rs_all(L, dtype, grads, buckets=None):
    out = []
    buckets = buckets or [[p.ds_id for p in L.params]]
    for r in range(L.world_size):
        gf = np.full(L.shard_numel, 0xFFFF, np.uint16)  # poison: every slot must be written
        for b in buckets:
            oracle.reduce_scatter(L, r, dtype, b, grads, gf)
        out.append(gf)
    return out


def test_worked_example_one_param_per_gpu():
    """Encoding A: the 4 units as one 4-element parameter, so GPU r owns unit r."""
    ex = _ex()
    N = ex["world_size"]
    L = oracle.make_layout(N, 0, [0], [4])
    g16 = to16_host(np.array(ex["grads_every_rank"], np.float32), "fp16")
    grads = [{0: g16} for _ in range(N)]
    outs = _rs_all(L, "fp16", grads)
    for r in range(N):
        assert oracle.to_f32(outs[r], "fp16").tolist() == [ex["averaged"][ex["unit_owned_by_rank"][r]]]
    assert float(oracle.to_f32(outs[0], "fp16")[0]) == ex["gpu0_keeps"]


def test_worked_example_four_scalar_params():
    """Encoding B: 4 scalar parameters; per-parameter ranges give rank 0 all
    four averages and ranks 1-3 only zero padding."""
    ex = _ex()
    N = ex["world_size"]
    L = oracle.make_layout(N, 0, [0, 1, 2, 3], [1, 1, 1, 1])
    grads = [{d: to16_host(np.array([ex["grads_every_rank"][d]], np.float32), "fp16")
              for d in range(4)} for _ in range(N)]
    outs = _rs_all(L, "fp16", grads)
    assert oracle.to_f32(outs[0], "fp16").tolist() == ex["averaged"]
    assert float(oracle.to_f32(outs[0], "fp16")[0]) == ex["gpu0_keeps"]
    for r in range(1, N):
        assert outs[r].tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("N", [1, 2, 4, 8, 64])
def test_identical_grads_average_to_themselves(dtype, N):
    """With every rank holding the same g, sum = N*g exactly in fp32 and /N
    is exact for N = 2^k, so the averaged slice is g bit for bit."""
    g = np.random.default_rng(N).standard_normal(300).astype(np.float32) * np.float32(1e-3)
    g16 = to16_host(g, dtype)
    L = oracle.make_layout(N, 0, [0], [300])
    grads = [{0: g16} for _ in range(N)]
    outs = _rs_all(L, dtype, grads)
    cat = np.concatenate([o[:L.params[0].partition_size] for o in outs])[:300]
    assert np.array_equal(cat, g16)


def _ordinal(bits, dtype):
    b = np.asarray(bits, np.int64)
    sign = (b & 0x8000) != 0
    mag = b & 0x7FFF
    return np.where(sign, -mag, mag)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 10**6), st.sampled_from([1, 2, 3, 4, 5, 8]), st.sampled_from(["fp16", "bf16"]),
       st.integers(1, 5))
def test_matches_brute_force_and_exact_mean(seed, N, dtype, n_params):
    rng = np.random.default_rng(seed)
    numels = list(rng.integers(1, 30, n_params))
    ids = list(range(n_params))
    L = oracle.make_layout(N, 7, ids, numels)
    grads = [{d: to16_host(rng.standard_normal(int(n)).astype(np.float32) * np.float32(1e-2), dtype)
              for d, n in zip(ids, numels)} for _ in range(N)]
    outs = _rs_all(L, dtype, grads)
    for r in range(N):
        for p in L.params:
            lo, hi = L.own_range(p, r)
            for k in range(p.partition_size):
                got = int(outs[r][p.shard_offset + k])
                j = lo + k
                if j >= hi:
                    assert got == 0
                    continue
                vals = [int(grads[v][p.ds_id][j]) for v in range(N)]
                assert got == brute.reduce_scatter_elem(vals, dtype)
                # within one unit in the last place of the exactly rounded mean
                exact = sum(Fraction(brute.value16(b, dtype)) for b in vals) / N
                ref = brute.bits16(float(exact), dtype)
                assert abs(int(_ordinal([got], dtype)[0]) - int(_ordinal([ref], dtype)[0])) <= 1


def test_bucketing_does_not_change_the_slices():
    cfg = get_config("c1")
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    grads = [{d: grad_host(cfg, 0, v, d) for d in cfg.ds_ids} for v in range(cfg.world_size)]
    a = _rs_all(L, cfg.dtype, grads)
    b = _rs_all(L, cfg.dtype, grads, buckets=oracle.reduce_buckets(L, 100))
    c = _rs_all(L, cfg.dtype, grads, buckets=[[3], [1, 0], [2]])
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_concatenated_slices_equal_dense_average():
    """No rank holds the full averaged gradient, but the union of the ranks'
    slices is it: check against an independent float64 mean rounded once."""
    cfg = get_config("c1")
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    grads = [{d: grad_host(cfg, 0, v, d) for d in cfg.ds_ids} for v in range(cfg.world_size)]
    outs = _rs_all(L, cfg.dtype, grads)
    for p in L.params:
        cat = np.concatenate([o[p.shard_offset:p.shard_offset + p.partition_size] for o in outs])[:p.numel]
        mean64 = np.mean([oracle.to_f32(grads[v][p.ds_id], cfg.dtype).astype(np.float64)
                          for v in range(cfg.world_size)], axis=0)
        ref = to16_host(mean64.astype(np.float32), cfg.dtype)
        d = np.abs(_ordinal(cat, cfg.dtype) - _ordinal(ref, cfg.dtype))
        assert d.max() <= 1
        assert (d == 0).mean() > 0.99


# Values whose fp32 sum depends on the order of the adds: in rank order the
# middle value is lost to a tie rounded to even, so the sum is exactly 0;
# in reverse order it survives.  bf16: 2^24, 1, -2^24 (2^24 + 1 needs 25
# significant bits).  fp16: 2^15, 2^-9, -2^15 (2^-9 is half an fp32 ulp of
# 2^15).
ORDER_TRIPLES = {
    "bf16": ([0x4B80, 0x3F80, 0xCB80], 1.0),
    "fp16": ([0x7800, 0x1800, 0xF800], 2.0 ** -9),
}


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_rank_order_of_the_sum_is_observable(dtype):
    """Reading of [csdn] step 3 / [codex] 6.2 (the pages give only "sum, then
    average"): the fp32 sum runs over the ranks in rank order.  With the
    triple above every rank's averaged element is exactly +0; the reverse
    order would give the small value divided by 3."""
    bits, small = ORDER_TRIPLES[dtype]
    N = 3
    L = oracle.make_layout(N, 0, [0], [N])          # one element per rank
    grads = [{0: np.full(N, bits[v], np.uint16)} for v in range(N)]
    outs = _rs_all(L, dtype, grads)
    assert [int(o[0]) for o in outs] == [0x0000] * N
    assert brute.reduce_scatter_elem(bits, dtype) == 0x0000
    rev = brute.reduce_scatter_elem(bits[::-1], dtype)
    assert brute.value16(rev, dtype) == pytest.approx(small / 3, rel=2 ** -7)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_sum_starts_at_positive_zero(dtype):
    """The fp32 sum starts at +0: when every rank's gradient is -0 the
    average is +0 (a sum seeded with the first rank's value would give -0)."""
    N = 4
    L = oracle.make_layout(N, 0, [0], [2 * N])
    grads = [{0: np.full(2 * N, 0x8000, np.uint16)} for _ in range(N)]
    for o in _rs_all(L, dtype, grads):
        assert o.tolist() == [0x0000, 0x0000]
    assert brute.reduce_scatter_elem([0x8000] * N, dtype) == 0x0000
