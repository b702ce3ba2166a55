"""Pins of the oracle's 16-bit conversions against library routines and an
exact-rational derivation (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def _interesting_f32(seed=0, n=200000):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # exact ties and near-ties of bf16 rounding, subnormals, powers of two
    ties = (rng.integers(0, 1 << 16, 5000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    near = ties + rng.integers(-2, 3, 5000).astype(np.int64).astype(np.uint32)
    extra = np.concatenate([ties, near]).view(np.float32)
    extra = extra[np.isfinite(extra)]
    small = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17e-38, 6e-8, 6.1e-5, 65504.0, 65520.0, 65519.99,
                      3.3895314e38, 3.4e38], np.float32)
    return np.concatenate([x, extra, small, rng.standard_normal(10000).astype(np.float32) * 1e-3])


def test_bf16_round_matches_torch():
    x = _interesting_f32()
    ours = oracle.from_f32(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_fp16_round_matches_torch():
    x = _interesting_f32(1)
    ours = oracle.from_f32(x, "fp16")
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_matches_exact_rational_rounding(dtype):
    x = _interesting_f32(2, 3000)
    if dtype == "bf16":
        x = x[np.abs(x) < 3.38e38]
    ours = oracle.from_f32(x, dtype)
    for xi, oi in zip(x.tolist(), ours.tolist()):
        assert oi == brute.bits16(xi, dtype), xi


@pytest.mark.parametrize("dtype,tdt", [("fp16", torch.float16), ("bf16", torch.bfloat16)])
def test_widen_matches_torch(dtype, tdt):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.to_f32(bits, dtype)
    ref = torch.from_numpy(bits.view(np.int16)).view(tdt).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
