"""Pins of the oracle's fused Adam + 16-bit cast (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from synth import get_config
from synth.gen import grad_host, to16_host, weights_host


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_first_step_closed_form(dtype):
    """At t = 1 with zero state and wd = 0, bias correction cancels the
    moment decay: w1 = w0 - lr * g / (|g| + eps)."""
    rng = np.random.default_rng(5)
    n = 20000
    w16 = to16_host(rng.standard_normal(n).astype(np.float32) * np.float32(0.02), dtype)
    g16 = to16_host(rng.standard_normal(n).astype(np.float32) * np.float32(1e-3), dtype)
    L = oracle.make_layout(1, 0, [0], [n])
    master, m, v = oracle.init_state(w16, dtype)
    w0 = master.copy()
    shard = w16.copy()
    hp = oracle.AdamHParams(lr=1e-3, step=1)
    scale = np.float32(0.75)
    oracle.adam_step(L, 0, dtype, 0, n, master, m, v, g16, shard, scale, False, hp)
    g = oracle.to_f32(g16, dtype).astype(np.float64) * 0.75
    closed = 1e-3 * g / (np.abs(g) + 1e-8)
    upd = w0.astype(np.float64) - master.astype(np.float64)
    bound = 8 * 2.0**-24 * np.abs(closed) + _ulp32(w0) + _ulp32(master)
    assert np.all(np.abs(upd - closed) <= bound)
    assert np.array_equal(shard, oracle.from_f32(master, dtype))
    np.testing.assert_array_equal(m, np.float32(0.1) * (oracle.to_f32(g16, dtype) * scale))


def test_worked_example_after_one_step():
    """Weights 1, 2, 3, 4, averaged grads 0.5, 1, 1.5, 2 (norm sqrt 7.5 > 1,
    so clipped): every weight moves by lr = 1e-3 to 0.999 .. 3.999 and the
    fp16 shard rounds that to the nearest fp16 (the four units held as one
    unsharded state, N = 1)."""
    L = oracle.make_layout(1, 0, [0], [4])
    w16 = to16_host(np.array([1, 2, 3, 4], np.float32), "fp16")
    g16 = to16_host(np.array([0.5, 1, 1.5, 2], np.float32), "fp16")
    master, m, v = oracle.init_state(w16, "fp16")
    shard = w16.copy()
    scale = np.float32(0.36514824628829956)
    oracle.adam_step(L, 0, "fp16", 0, 4, master, m, v, g16, shard, scale, False, oracle.AdamHParams())
    np.testing.assert_allclose(master, [0.999, 1.999, 2.999, 3.999], rtol=0, atol=3e-7)
    assert oracle.to_f32(shard, "fp16").tolist() == [0.9990234375, 1.9990234375, 2.998046875, 3.998046875]


@pytest.mark.parametrize("wd", [0.0, 0.01])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_matches_pure_python_fp32_emulation(dtype, wd):
    rng = np.random.default_rng(9)
    n = 64
    w16 = to16_host(rng.standard_normal(n).astype(np.float32) * np.float32(0.02), dtype)
    L = oracle.make_layout(1, 0, [0], [n])
    master, m, v = oracle.init_state(w16, dtype)
    shard = w16.copy()
    bw = [float(x) for x in master]
    bm = [0.0] * n
    bv = [0.0] * n
    for t in range(1, 4):
        g16 = to16_host(rng.standard_normal(n).astype(np.float32) * np.float32(1e-3), dtype)
        scale = np.float32(0.8125)
        hp = oracle.AdamHParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, step=t)
        oracle.adam_step(L, 0, dtype, 0, n, master, m, v, g16, shard, scale, False, hp)
        for i in range(n):
            bw[i], bm[i], bv[i], sb = brute.adam_elem(bw[i], bm[i], bv[i], int(g16[i]), dtype,
                                                      float(scale), 1e-3, 0.9, 0.999, 1e-8, t, wd)
            assert int(shard[i]) == sb
        assert master.tolist() == bw and m.tolist() == bm and v.tolist() == bv


def test_agrees_with_torch_adam():
    """torch.optim.Adam orders its fp32 operations differently (it divides
    sqrt(v) by sqrt(bias_correction2) and folds 1/bias_correction1 into the
    step), so agreement is to rounding, not bit for bit."""
    rng = np.random.default_rng(3)
    n = 50000
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    L = oracle.make_layout(1, 0, [0], [n])
    master = w0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    shard = oracle.from_f32(w0, "bf16")
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                           foreach=False, fused=False)
    for t in range(1, 11):
        g16 = to16_host((rng.standard_normal(n) * 1e-3).astype(np.float32), "bf16")
        g = oracle.to_f32(g16, "bf16")
        oracle.adam_step(L, 0, "bf16", 0, n, master, m, v, g16, shard, np.float32(1.0), False,
                         oracle.AdamHParams(step=t))
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    tw = p.detach().numpy()
    st = opt.state[p]
    # torch updates m by lerp (m + (1 - b1) (g - m)): a cancellation near m = 0,
    # so the tolerance is relative to the moment's scale, not elementwise
    tm, tv = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()
    np.testing.assert_allclose(m, tm, rtol=0, atol=2e-6 * np.abs(tm).max())
    np.testing.assert_allclose(v, tv, rtol=2e-6, atol=2e-6 * np.abs(tv).max())
    # weights: the 10 updates of size <= lr agree to a few fp32 roundings each
    assert np.max(np.abs(master.astype(np.float64) - tw)) <= 10 * (2e-6 * 1e-3) + 4 * np.max(_ulp32(w0))
    moved = np.abs(master.astype(np.float64) - w0)
    assert moved.min() > 0 and moved.max() <= 10 * 1e-3 * 1.0001


@pytest.mark.parametrize("wd", [0.01, 0.1])
def test_weight_decay_with_zero_gradient_closed_form(wd):
    """Decoupled weight decay (Loshchilov & Hutter): with a zero gradient the
    moments stay 0, the Adam term is lr * (0 / eps) = 0, and one step only
    shrinks the weight: w1 = w0 * (1 - lr * wd), to within one fp32 rounding
    of each of the two operations.  (L2 decay folded into the gradient would
    move every weight by about lr instead.)"""
    rng = np.random.default_rng(21)
    n = 4096
    w0 = (rng.standard_normal(n) * 0.5).astype(np.float32)
    L = oracle.make_layout(1, 0, [0], [n])
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    shard = oracle.from_f32(w0, "bf16")
    lr = 1e-3
    oracle.adam_step(L, 0, "bf16", 0, n, w, m, v, np.zeros(n, np.uint16), shard, np.float32(1.0), False,
                     oracle.AdamHParams(lr=lr, weight_decay=wd, step=1))
    exact = w0.astype(np.float64) * (1.0 - lr * wd)
    assert np.all(np.abs(w - exact) <= 1.5 * _ulp32(w0))
    assert np.all(m == 0) and np.all(v == 0)
    assert np.array_equal(shard, oracle.from_f32(w, "bf16"))
    assert np.all(np.abs(w) < np.abs(w0)) or np.all(w0 == 0)


def test_agrees_with_torch_adamw():
    """torch.optim.AdamW shrinks the weight by lr * weight_decay before the
    Adam update, as the oracle does; agreement to rounding over 10 steps."""
    rng = np.random.default_rng(4)
    n = 50000
    wd = 0.1
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    L = oracle.make_layout(1, 0, [0], [n])
    master = w0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    shard = oracle.from_f32(w0, "bf16")
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.AdamW([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd, foreach=False,
                            fused=False)
    for t in range(1, 11):
        g16 = to16_host((rng.standard_normal(n) * 1e-3).astype(np.float32), "bf16")
        g = oracle.to_f32(g16, "bf16")
        oracle.adam_step(L, 0, "bf16", 0, n, master, m, v, g16, shard, np.float32(1.0), False,
                         oracle.AdamHParams(weight_decay=wd, step=t))
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    tw = p.detach().numpy()
    assert np.max(np.abs(master.astype(np.float64) - tw)) <= 10 * (2e-6 * 1e-3) + 6 * np.max(_ulp32(w0))
    # the decay is visible: it moved the weights by about 10 * lr * wd * |w0|
    plain = w0.copy()
    m2, v2 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    rng = np.random.default_rng(4)
    rng.standard_normal(n)
    for t in range(1, 11):
        g16 = to16_host((rng.standard_normal(n) * 1e-3).astype(np.float32), "bf16")
        oracle.adam_step(L, 0, "bf16", 0, n, plain, m2, v2, g16, shard.copy(), np.float32(1.0), False,
                         oracle.AdamHParams(step=t))
    shrink = np.abs(plain.astype(np.float64) - master)
    big = np.abs(w0) > 0.01
    assert np.all(shrink[big] >= 0.5 * 10 * 1e-3 * wd * np.abs(w0[big]))


def test_nonfinite_skips_step_and_padding_stays_zero():
    L = oracle.make_layout(3, 0, [0, 1], [7, 5])   # ps 3 and 2: rank 2 has padding
    r = 2
    w = oracle.partition(L, r, {0: to16_host(np.arange(1, 8, dtype=np.float32), "bf16"),
                                1: to16_host(np.arange(1, 6, dtype=np.float32), "bf16")})
    master, m, v = oracle.init_state(w, "bf16")
    g = to16_host(np.array([1, 1, 1, 1, 1], np.float32), "bf16")
    shard = w.copy()
    before = (master.copy(), m.copy(), v.copy(), shard.copy())
    oracle.adam_step(L, r, "bf16", 0, L.shard_numel, master, m, v, g, shard, np.float32(1), True,
                     oracle.AdamHParams())
    for a, b in zip((master, m, v, shard), before):
        assert np.array_equal(a, b)
    oracle.adam_step(L, r, "bf16", 0, L.shard_numel, master, m, v, g, shard, np.float32(1), False,
                     oracle.AdamHParams())
    pad = oracle.padding_mask(L, r)
    assert pad.tolist() == [False, True, True, False, True]
    assert np.all(master[pad] == 0) and np.all(shard[pad] == 0) and np.all(m[pad] == 0)
    assert np.all(master[~pad] != before[0][~pad])


def test_sharded_steps_equal_dense_data_parallel_steps():
    """Three steps of c1 on all four ranks, concatenated, equal three steps
    of unsharded data-parallel Adam bit for bit, and the sub-group split
    does not matter."""
    cfg = get_config("c1")
    N, dt = cfg.world_size, cfg.dtype
    L = oracle.make_layout(N, cfg.threshold, cfg.ds_ids, cfg.numels)
    full = {d: weights_host(cfg, d) for d in cfg.ds_ids}
    shards = [oracle.partition(L, r, full) for r in range(N)]
    states = [oracle.init_state(s, dt) for s in shards]
    dense_params, dense_state = dict(full), None
    for step in range(1, cfg.steps + 1):
        grads = [{d: grad_host(cfg, step, v, d) for d in cfg.ds_ids} for v in range(N)]
        gfs = []
        for r in range(N):
            gf = np.zeros(L.shard_numel, np.uint16)
            for b in oracle.reduce_buckets(L, cfg.reduce_bucket_size):
                oracle.reduce_scatter(L, r, dt, b, grads, gf)
            gfs.append(gf)
        parts = [oracle.grad_norm_partial(L, r, dt, gfs[r]) for r in range(N)]
        norm, coef, scale, bad = oracle.grad_norm_finalize([a for a, _ in parts], parts[0][1], cfg.max_norm)
        hp = oracle.AdamHParams(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, step)
        for r in range(N):
            master, m, v = states[r]
            groups = oracle.sub_groups(L, 600 if r % 2 else cfg.sub_group_size)
            for b, e in groups:
                oracle.adam_step(L, r, dt, b, e, master, m, v, gfs[r], shards[r], scale, bad, hp)
        dense_params, dense_state, dnorm, dscale = oracle.dense_reference_step(
            dt, dense_params, grads, dense_state, cfg.max_norm, hp)
        assert dnorm == pytest.approx(norm, rel=1e-13)
        assert dscale == scale
        for p in L.params:
            cat = np.concatenate([s[p.shard_offset:p.shard_offset + p.partition_size] for s in shards])
            assert np.array_equal(cat[:p.numel], dense_params[p.ds_id])
            for k, arr in enumerate(zip(*states)):
                cat = np.concatenate([a[p.shard_offset:p.shard_offset + p.partition_size] for a in arr])
                assert np.array_equal(cat[:p.numel], dense_state[p.ds_id][k])
