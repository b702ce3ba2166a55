"""GPU parity of Adam on optimizer state held in pinned host memory
(zs3_adam_step_offload): the same update as zs3_adam_step bit for bit, and
the oracle's, with the state read and written directly through its device
mapping, or streamed through a small staging buffer in many ragged chunks,
from misaligned sub-group starts."""

import numpy as np
import pytest

import oracle
import zero_sharded_state_amd as zs
from synth.gen import random_bits16

from gpu_util import Buf16, Buf32, note, require_gpu, sync
from test_gpu_parity import _layout, _problem

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _hp(t):
    return {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.0, "step": t}


@pytest.mark.parametrize("seed,N,T,n,mx", [(11, 8, 100, 9, 40000), (12, 3, 0, 12, 9000), (13, 64, 500, 6, 60000)])
@pytest.mark.parametrize("chunk", [None, 8, 1000, 1 << 16])
def test_offload_matches_device_adam_and_oracle(seed, N, T, n, mx, chunk):
    import torch
    ids, numels, _ = _problem(seed, N, T, n, mx, "bf16")
    h, L = _layout(ids, numels, N, T)
    try:
        r = N - 1
        S = L.shard_numel
        rng = np.random.default_rng(seed)
        shard0 = random_bits16(seed, S, "bf16", 0.02, 3)
        shard0[oracle.padding_mask(L, r)] = 0
        wbuf, sbuf = Buf32(S), Buf16(S, fill=shard0)
        zs.zs3_init_master(h, r, "bf16", 0, S, sbuf.ptr(), wbuf.ptr())     # the master from the library
        sync()
        w0 = wbuf.host()
        assert np.array_equal(w0.view(np.uint32), oracle.init_state(shard0, "bf16")[0].view(np.uint32))
        m0 = (rng.standard_normal(S) * 1e-4).astype(np.float32)
        v0 = (rng.random(S) * 1e-7).astype(np.float32)
        # device reference: zs3_adam_step on device copies
        dw, dm, dv = (torch.from_numpy(x.copy()).cuda() for x in (w0, m0, v0))
        ds = Buf16(S, fill=shard0)
        # offloaded: pinned host state
        hw, hm, hv = (torch.from_numpy(x.copy()).pin_memory() for x in (w0, m0, v0))
        hs = Buf16(S, fill=shard0)
        stage = torch.full((6 * (chunk + 8),), float("nan"), dtype=torch.float32, device="cuda") if chunk else None
        scale = torch.tensor([0.75], dtype=torch.float32, device="cuda")
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        cin, cout = torch.cuda.Stream(), torch.cuda.Stream()
        groups = oracle.sub_groups(L, max(1, S // 3))
        ow, om, ov, osh = w0.copy(), m0.copy(), v0.copy(), shard0.copy()
        for t in range(1, 4):
            g = random_bits16(seed + t, S, "bf16", 1e-3, 5)
            g[oracle.padding_mask(L, r)] = 0
            gb = Buf16(S, fill=g)
            note(f"offload seed={seed} N={N} chunk={chunk} step={t}")
            for b, e in groups:
                zs.zs3_adam_step(h, r, "bf16", b, e, dw, dm, dv, gb.ptr(), ds.ptr(), scale, flag, _hp(t))
                zs.zs3_adam_step_offload(h, r, "bf16", b, e, hw, hm, hv, stage, stage.numel() if chunk else 0,
                                         gb.ptr(), hs.ptr(), scale, flag, _hp(t), copy_in_stream=cin,
                                         copy_out_stream=cout)
                oracle.adam_step(L, r, "bf16", b, e, ow, om, ov, g, osh, np.float32(0.75), False,
                                 oracle.AdamHParams(step=t))
            sync()
            for got, dev, ref in ((hw, dw, ow), (hm, dm, om), (hv, dv, ov)):
                assert np.array_equal(got.numpy().view(np.uint32), dev.cpu().numpy().view(np.uint32))
                assert np.array_equal(got.numpy().view(np.uint32), ref.view(np.uint32))
            assert np.array_equal(hs.host(), ds.host()) and np.array_equal(hs.host(), osh)
            hs.check_guards()
    finally:
        zs.zs3_layout_destroy(h)


@pytest.mark.parametrize("staged", [False, True])
def test_offload_nonfinite_flag_leaves_everything(staged):
    import torch
    h = zs.zs3_layout_create(2, 0, [0, 1], [3000, 1000])
    try:
        S = zs.zs3_layout_info(h)["shard_numel"]
        w = torch.randn(S).pin_memory()
        m = torch.randn(S).pin_memory()
        v = torch.rand(S).pin_memory()
        keep = [x.clone() for x in (w, m, v)]
        sh = Buf16(S, fill=random_bits16(1, S, "fp16", 0.02, 1))
        before = sh.host()
        g = Buf16(S, fill=random_bits16(2, S, "fp16", 1e-3, 1))
        stage = torch.empty(6 * 264, dtype=torch.float32, device="cuda")
        scale = torch.tensor([1.0], device="cuda")
        flag = torch.ones(1, dtype=torch.int32, device="cuda")
        zs.zs3_adam_step_offload(h, 0, "fp16", 0, S, w, m, v, stage if staged else None,
                                 stage.numel() if staged else 0, g.ptr(), sh.ptr(), scale, flag, _hp(1))
        sync()
        for a, b in zip((w, m, v), keep):
            assert torch.equal(a, b)
        assert np.array_equal(sh.host(), before)
    finally:
        zs.zs3_layout_destroy(h)


def test_offload_rejects_pageable_host_memory():
    import torch
    h = zs.zs3_layout_create(1, 0, [0], [100])
    try:
        w = torch.zeros(100)              # pageable
        stage = torch.empty(6 * 64, dtype=torch.float32, device="cuda")
        g = Buf16(100)
        sh = Buf16(100)
        scale = torch.tensor([1.0], device="cuda")
        with pytest.raises(zs.Zs3Error) as e:
            zs.zs3_adam_step_offload(h, 0, "fp16", 0, 100, w, w.clone(), w.clone(), stage, stage.numel(), g.ptr(),
                                     sh.ptr(), scale, None, _hp(1))
        assert e.value.status == zs.ZS3_EINVAL and "pinned" in e.value.message
    finally:
        zs.zs3_layout_destroy(h)
