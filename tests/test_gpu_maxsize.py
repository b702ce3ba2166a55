"""GPU parity at the largest single-segment sizes: one ragged parameter of
2^32 + 2^20 + 7 elements split over N = 2 ranks, so that every call moves a
contiguous run of more than 2^31 elements (more than 4 GiB of 16-bit data)
in one launch and every index above 2^31 must be 64-bit.  Rank 1 holds the
padding (its real part is one element short of the partition size).

Outputs are checked against the oracle on sampled positions: the run's
first and last elements, both sides of 2^31 and 2^32, the last real element
and the padding, and a few hundred seeded random positions.
"""

import gc

import numpy as np
import pytest

import oracle
from synth.gen import device_normal16

from gpu_util import assert_f32_close, note, ordinal16, require_gpu, sync

pytestmark = pytest.mark.gpu

N, RANK, DT = 2, 1, "bf16"
NUMEL = (1 << 32) + (1 << 20) + 7
PS = (NUMEL + N - 1) // N
REAL = NUMEL - RANK * PS          # rank 1's real elements: PS - 1


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    import torch
    gc.collect()
    torch.cuda.empty_cache()


def _positions(length, rng, extra=()):
    fixed = [0, 1, 7, 8, 9, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, (1 << 32) - 1, 1 << 32, (1 << 32) + 1,
             length - 2, length - 1, *extra]
    pos = {p for p in fixed if 0 <= p < length}
    pos |= set(rng.integers(0, length, 300).tolist())
    return np.array(sorted(pos), np.int64)


def _take16(t, idx):
    import torch
    return t[torch.from_numpy(idx).to(t.device)].cpu().numpy().view(np.uint16)


def _take32(t, idx):
    import torch
    return t[torch.from_numpy(idx).to(t.device)].cpu().numpy()


@pytest.mark.timeout(900)
def test_more_than_2_pow_31_elements_per_launch():
    import torch
    import zero_sharded_state_amd as zs

    assert PS > (1 << 31) and REAL == PS - 1
    dev = torch.device("cuda")
    rng = np.random.default_rng(11)
    L = oracle.make_layout(N, 0, [0], [NUMEL])
    h = zs.zs3_layout_create(N, 0, [0], [NUMEL])
    try:
        # ---- partition: rank 1's range of the full parameter -> its shard
        full = device_normal16(NUMEL, 0.02, DT, dev, (11, 0, 0))
        shard = torch.full((PS,), 0x1234, dtype=torch.int16, device=dev)
        note(f"maxsize: partition numel={NUMEL} ps={PS}")
        zs.zs3_partition(h, RANK, DT, [0], [full], shard)
        sync()
        k = _positions(PS, rng)
        got = _take16(shard, k)
        j = RANK * PS + k
        real = j < NUMEL
        ref = np.zeros(len(k), np.uint16)
        ref[real] = _take16(full, j[real])
        assert np.array_equal(got, ref), "partition"
        assert got[k == PS - 1][0] == 0, "padding element"

        # ---- fused pack + unpack: rank 0's chunk from the wire, rank 1's from its shard
        wire0 = device_normal16(PS, 0.02, DT, dev, (11, 0, 1))
        own = torch.full((PS,), 0x1234, dtype=torch.int16, device=dev)
        note("maxsize: gather (pack + unpack)")
        offs = zs.zs3_gather_coalesced(h, RANK, DT, zs.ZS3_PACK | zs.ZS3_UNPACK, [0], shard, own, [wire0, own], full)
        sync()
        assert offs == [0]
        f = _positions(NUMEL, rng, extra=(PS - 1, PS, PS + 1, NUMEL - 1))
        got = _take16(full, f)
        ref = np.where(f < PS, _take16(wire0, np.minimum(f, PS - 1)), _take16(shard, np.maximum(f - PS, 0)))
        assert np.array_equal(got, ref), "gathered parameter"
        k = _positions(PS, rng)
        assert np.array_equal(_take16(own, k), _take16(shard, k)), "packed chunk"
        del wire0, own, full
        gc.collect()
        torch.cuda.empty_cache()

        # ---- reduce-scatter: two received slices -> rank 1's flat gradient
        recv = [device_normal16(PS, 1e-3, DT, dev, (11, 1, v)) for v in range(N)]
        grad = torch.full((PS,), 0x1234, dtype=torch.int16, device=dev)
        note("maxsize: reduce-scatter")
        zs.zs3_reduce_scatter_local(h, RANK, DT, [0], recv, grad)
        sync()
        k = _positions(PS, rng)
        kr = k[k < REAL]
        m = len(kr)
        sub = oracle.make_layout(N, 0, [0], [2 * m])           # rank 1 owns [m, 2m): every sample is real
        grads = [{0: np.concatenate([np.zeros(m, np.uint16), _take16(recv[v], kr)])} for v in range(N)]
        ref = np.zeros(m, np.uint16)
        oracle.reduce_scatter(sub, RANK, DT, [0], grads, ref)
        got = _take16(grad, k)
        assert np.array_equal(got[k < REAL], ref), "reduce-scatter"
        assert np.all(got[k >= REAL] == 0), "reduce-scatter padding"
        del recv
        gc.collect()
        torch.cuda.empty_cache()

        # ---- norm over the whole flat gradient
        sumsq = torch.tensor([0.75, 0.0, 0.0], dtype=torch.float64, device=dev)
        outs = torch.zeros(2, dtype=torch.float64, device=dev)
        scale = torch.zeros(1, dtype=torch.float32, device=dev)
        flag = torch.zeros(1, dtype=torch.int32, device=dev)
        note("maxsize: grad norm")
        zs.zs3_grad_norm(h, RANK, DT, grad, sumsq, True, 1.0, 1.0, outs, scale, flag)
        sync()
        gh = grad.cpu().numpy().view(np.uint16)
        a, q = oracle.grad_norm_partial(L, RANK, DT, gh)
        del gh
        s = sumsq.cpu().numpy()
        assert s[RANK] == pytest.approx(a, rel=1e-10) and s[N] == 0.0
        norm, coef, sc, bad = oracle.grad_norm_finalize([0.75, a], q, 1.0)
        assert abs(float(outs[0].item()) - norm) <= 1e-5 * norm and not bad and int(flag.item()) == 0
        assert abs(float(scale.item()) - float(sc)) <= np.spacing(np.float32(sc))

        # ---- Adam over the whole partition, one step (t = 3) with the GPU's scale
        master = torch.randn(PS, device=dev).mul_(0.02)
        exp_avg = torch.randn(PS, device=dev).mul_(1e-4)
        exp_avg_sq = torch.rand(PS, device=dev).mul_(1e-8)
        k = _positions(PS, rng)
        w0, m0, v0 = _take32(master, k), _take32(exp_avg, k), _take32(exp_avg_sq, k)
        g0, s0 = _take16(grad, k), _take16(shard, k)
        hp = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.0, "step": 3}
        note("maxsize: adam")
        zs.zs3_adam_step(h, RANK, DT, 0, PS, master, exp_avg, exp_avg_sq, grad, shard, scale, flag, hp)
        sync()
        r = k < REAL
        m = int(r.sum())
        sub = oracle.make_layout(N, 0, [0], [2 * m])
        w, mm, vv = w0[r].copy(), m0[r].copy(), v0[r].copy()
        sh = np.zeros(m, np.uint16)
        oracle.adam_step(sub, RANK, DT, 0, m, w, mm, vv, g0[r], sh, np.float32(scale.item()), False,
                         oracle.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.0, 3))
        gw, gm, gv, gs = _take32(master, k), _take32(exp_avg, k), _take32(exp_avg_sq, k), _take16(shard, k)
        assert_f32_close(gw[r], w, what="master")
        assert_f32_close(gm[r], mm, what="exp_avg")
        assert_f32_close(gv[r], vv, what="exp_avg_sq")
        assert np.max(np.abs(ordinal16(gs[r]) - ordinal16(sh))) <= 1, "shard"
        # padding is skipped: state and shard untouched
        assert np.array_equal(gw[~r], w0[~r]) and np.array_equal(gm[~r], m0[~r]) and np.array_equal(gv[~r], v0[~r])
        assert np.array_equal(gs[~r], s0[~r]), "padding of the shard"
    finally:
        zs.zs3_layout_destroy(h)
