"""The layout's cache of work lists when it fills up: a layout holds at most
16,384 cached call shapes; the next new shape waits for the device, frees
them all and starts again.  More than that many distinct calls (a partition
into a destination that moves by one element each time) must all give the
right result, including a shape built before the eviction and called again
after it, and calls enqueued right before the eviction.  The calls use
device work lists (more segments than fit in the kernel arguments), so the
eviction frees tables that earlier launches read."""

import numpy as np
import pytest
import torch

import oracle
import zero_sharded_state_amd as zs
from synth.gen import random_bits16

from gpu_util import note, require_gpu, sync

pytestmark = pytest.mark.gpu

CACHE = 16384


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.timeout(600)
def test_more_distinct_calls_than_the_cache_holds():
    N, T = 2, 0
    # 45 parameters: more segments than a plan in the kernel arguments holds,
    # so every call's work list is a device table that the eviction frees
    rng = np.random.default_rng(5)
    ids = [int(x) for x in rng.permutation(45) * 3 + 1]
    numels = [int(x) for x in rng.integers(1, 400, 45)]
    full = {d: random_bits16(77, n, "bf16", 0.02, 1, d) for d, n in zip(ids, numels)}
    L = oracle.make_layout(N, T, ids, numels)
    ref = oracle.partition(L, 1, full)
    S = L.shard_numel
    h = zs.zs3_layout_create(N, T, ids, numels)
    try:
        src = [torch.from_numpy(full[d].view(np.int16)).cuda() for d in ids]
        calls = CACHE + 300
        out = torch.zeros(calls + S, dtype=torch.int16, device="cuda")
        first = torch.zeros(S, dtype=torch.int16, device="cuda")
        zs.zs3_partition(h, 1, "bf16", ids, src, first)            # one shape, cached first
        note(f"plan cache: {calls} distinct partition calls")
        for i in range(calls):
            # destination start i: every call is a new shape; each later call
            # overwrites all but the first element of the previous one
            zs.zs3_partition(h, 1, "bf16", ids, src, out.data_ptr() + 2 * i)
            if i == CACHE // 2:
                first.zero_()
                zs.zs3_partition(h, 1, "bf16", ids, src, first)    # cached shape, before the eviction
                sync()
                assert np.array_equal(first.cpu().numpy().view(np.uint16), ref)
        first.zero_()
        zs.zs3_partition(h, 1, "bf16", ids, src, first)            # rebuilt after the eviction
        sync()
        got = out.cpu().numpy().view(np.uint16)
        # position i holds the first element written by call i (later calls start after it)
        assert np.all(got[:calls] == ref[0]), "an earlier call's first element"
        assert np.array_equal(got[calls - 1:calls - 1 + S], ref), "the last call"
        assert np.array_equal(first.cpu().numpy().view(np.uint16), ref), "a shape rebuilt after the eviction"
    finally:
        zs.zs3_layout_destroy(h)
