"""Pins of the oracle's shard-aware gradient norm and clip coefficient (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute
from synth import get_config
from synth.gen import grad_host, to16_host

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _norm_all_ranks(L, dtype, grad_flats, max_norm):
    parts, pers = [], None
    for r, gf in enumerate(grad_flats):
        a, q = oracle.grad_norm_partial(L, r, dtype, gf)
        parts.append(a)
        if pers is None:
            pers = q
        assert q == pers            # the persistent sum is the same on every rank
    return oracle.grad_norm_finalize(parts, pers, max_norm)


def _rs(L, dtype, grads):
    outs = []
    for r in range(L.world_size):
        gf = np.zeros(L.shard_numel, np.uint16)
        oracle.reduce_scatter(L, r, dtype, [p.ds_id for p in L.params], grads, gf)
        outs.append(gf)
    return outs


def test_worked_example_norm_and_coefficient():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    for ids, numels in (([0], [4]), ([0, 1, 2, 3], [1, 1, 1, 1])):
        L = oracle.make_layout(4, 0, ids, numels)
        if len(ids) == 1:
            grads = [{0: to16_host(np.array(ex["grads_every_rank"], np.float32), "fp16")}] * 4
        else:
            grads = [{d: to16_host(np.array([ex["grads_every_rank"][d]], np.float32), "fp16")
                      for d in ids}] * 4
        norm, coef, scale, bad = _norm_all_ranks(L, "fp16", _rs(L, "fp16", grads), 1.0)
        # averaged grads 0.5, 1, 1.5, 2: sum of squares 7.5
        assert norm == math.sqrt(7.5) == 2.7386127875258306
        assert coef == pytest.approx(1.0 / (math.sqrt(7.5) + 1e-6), rel=0, abs=0)
        assert float(scale) == 0.36514824628829956
        assert not bad


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_constant_gradient_closed_form(dtype):
    c = 0.375  # exact in both 16-bit types
    L = oracle.make_layout(8, 50, [0, 1, 2], [1000, 37, 333])
    grads = [{p.ds_id: to16_host(np.full(p.numel, c, np.float32), dtype) for p in L.params}] * 8
    norm, coef, scale, bad = _norm_all_ranks(L, dtype, _rs(L, dtype, grads), 1e9)
    assert norm == pytest.approx(c * math.sqrt(1000 + 37 + 333), rel=1e-15)
    assert coef == 1.0 and float(scale) == 1.0 and not bad


def test_equals_l2_norm_of_dense_averaged_gradient():
    cfg = get_config("c1")
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    grads = [{d: grad_host(cfg, 0, v, d) for d in cfg.ds_ids} for v in range(cfg.world_size)]
    outs = _rs(L, cfg.dtype, grads)
    norm, _, _, _ = _norm_all_ranks(L, cfg.dtype, outs, cfg.max_norm)
    dense = []
    bits = []
    for p in L.params:
        cat = np.concatenate([o[p.shard_offset:p.shard_offset + p.partition_size] for o in outs])[:p.numel]
        dense.append(oracle.to_f32(cat, cfg.dtype).astype(np.float64))
        bits += list(map(int, cat))
    ref = float(np.linalg.norm(np.concatenate(dense)))
    assert norm == pytest.approx(ref, rel=1e-12)
    assert norm == pytest.approx(math.sqrt(brute.sumsq(bits, cfg.dtype)), rel=1e-13)
    assert 0.015 < norm < 0.04       # N(0, 1e-3) grads averaged over 4 ranks: no clipping


@pytest.mark.parametrize("dtype,max_norm,outliers", [("bf16", 1.0, True), ("fp16", 0.01, False),
                                                      ("bf16", 1.0, False)])
def test_coefficient_matches_torch_clip_grad_norm(dtype, max_norm, outliers):
    """[llmnex] pitfall 1 names torch's clip_grad_norm_ as the routine that
    must see the global norm.  Handed the dense averaged gradient (every
    element once, persistent parameters once) as fp64 gradients, it finds
    the same total norm and multiplies every gradient by the same
    coefficient -- its epsilon and its clamp at 1 included -- as the
    oracle's shard-aware norm computes from the ranks' slices.  Two cases
    clip (outliers; a small max_norm), one does not."""
    import torch

    rng = np.random.default_rng(7)
    ids, numels = [3, 0, 5, 1], [1000, 37, 333, 4099]
    L = oracle.make_layout(8, 50, ids, numels)               # ds_id 0 (37 elements) is persistent
    grads = []
    for v in range(8):
        g = {}
        for d, n in zip(ids, numels):
            x = rng.normal(0.0, 1e-2, n).astype(np.float32)
            if outliers:
                x[rng.random(n) < 0.01] *= 100
            g[d] = to16_host(x, dtype)
        grads.append(g)
    outs = _rs(L, dtype, grads)
    norm, coef, scale, bad = _norm_all_ranks(L, dtype, outs, max_norm)
    assert not bad
    params = []
    for p in L.params:
        cat = np.concatenate([o[p.shard_offset:p.shard_offset + p.partition_size] for o in outs])[:p.numel]
        t = torch.nn.Parameter(torch.zeros(p.numel, dtype=torch.float64))
        t.grad = torch.from_numpy(oracle.to_f32(cat, dtype).astype(np.float64))
        params.append(t)
    before = [t.grad.clone() for t in params]
    total = torch.nn.utils.clip_grad_norm_(params, max_norm, norm_type=2.0)
    assert float(total) == pytest.approx(norm, rel=1e-13)
    applied = torch.cat([(t.grad / b)[b != 0] for t, b in zip(params, before)])
    assert float(applied.min()) == pytest.approx(coef, rel=1e-13)
    assert float(applied.max()) == pytest.approx(coef, rel=1e-13)
    assert (coef < 1.0) == (max_norm < norm)
    assert scale == np.float32(coef)


def test_persistent_counted_once():
    L = oracle.make_layout(4, 10, [0, 1], [3, 40])        # param 0 persistent
    g = {0: to16_host(np.array([1.0, 2.0, 2.0], np.float32), "bf16"),
         1: to16_host(np.zeros(40, np.float32), "bf16")}
    norm, _, _, _ = _norm_all_ranks(L, "bf16", _rs(L, "bf16", [g] * 4), 100.0)
    assert norm == 3.0


def test_per_rank_local_norms_disagree():
    """The pitfall of the llmnex page: clipping each shard by its own local
    norm gives every rank a different coefficient."""
    cfg = get_config("c1")
    L = oracle.make_layout(cfg.world_size, cfg.threshold, cfg.ds_ids, cfg.numels)
    grads = [{d: grad_host(cfg, 0, v, d) for d in cfg.ds_ids} for v in range(cfg.world_size)]
    outs = _rs(L, cfg.dtype, grads)
    max_norm = 0.005
    _, coef, _, _ = _norm_all_ranks(L, cfg.dtype, outs, max_norm)
    local = []
    for r in range(cfg.world_size):
        a, q = oracle.grad_norm_partial(L, r, cfg.dtype, outs[r])
        local.append(oracle.grad_norm_finalize([a], q, max_norm)[1])
    assert len(set(local)) == cfg.world_size
    assert all(c != coef for c in local)


def test_nonfinite_sets_flag():
    L = oracle.make_layout(2, 0, [0], [8])
    g = to16_host(np.array([1, 2, np.inf, 0, 0, 0, 0, 0], np.float32), "fp16")
    outs = _rs(L, "fp16", [{0: g}, {0: g}])
    norm, coef, scale, bad = _norm_all_ranks(L, "fp16", outs, 1.0)
    assert bad
