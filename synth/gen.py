"""Seeded synthetic inputs: weights ~ N(0, weight_std), per-rank gradients
~ N(0, grad_std) with optional x100 outliers, rounded to the 16-bit dtype.

Host generation (numpy PCG64) serves the sizes a CPU check can hold;
device generation (torch's generator on the GPU) serves the full-size
workloads.  Values are returned as 16-bit bit patterns (``np.uint16`` on the
host, ``torch.int16`` views on the device): the consumers reinterpret them
in the configuration's dtype.

The 16-bit rounding of the synthetic fp32 draws uses numpy (fp16) or
torch (bf16) conversions: it is part of producing an input, not of the
method being checked.
"""

from __future__ import annotations

import hashlib
from typing import Optional, Sequence

import numpy as np

from .configs import Config

KIND_WEIGHT = 1
KIND_GRAD = 2
KIND_OUTLIER = 3
KIND_STATE = 4


def _seed_words(*words: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(w) & 0xFFFFFFFF for w in words])


def rng(cfg_or_seed, *words: int) -> np.random.Generator:
    if isinstance(cfg_or_seed, Config):
        base = (cfg_or_seed.seed, cfg_or_seed.config_id)
    else:
        base = (int(cfg_or_seed), 0)
    return np.random.Generator(np.random.PCG64(_seed_words(*base, *words)))


def to16_host(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws -> 16-bit bit patterns (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
        return t.numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def weights_host(cfg: Config, ds_id: int) -> np.ndarray:
    """Full flattened weight of parameter ``ds_id``."""
    if cfg.name in ("c0", "c0b"):
        vals = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
        return to16_host(vals if cfg.name == "c0b" else vals[ds_id:ds_id + 1], cfg.dtype)
    n = cfg.params[ds_id].numel
    x = rng(cfg, KIND_WEIGHT, ds_id).standard_normal(n, dtype=np.float32) * np.float32(cfg.weight_std)
    return to16_host(x, cfg.dtype)


def grad_host(cfg: Config, step: int, vrank: int, ds_id: int,
              lo: int = 0, hi: Optional[int] = None) -> np.ndarray:
    """Virtual rank ``vrank``'s gradient of parameter ``ds_id`` at ``step``,
    elements [lo, hi) of the flattened gradient (whole gradient by default).

    A slice is drawn from its own stream (seeded by ``lo``), so a slice is
    not a window of the whole-gradient draw; consumers always share the same
    array.
    """
    n = cfg.params[ds_id].numel
    hi = n if hi is None else hi
    if cfg.name in ("c0", "c0b"):
        vals = np.array([0.5, 1.0, 1.5, 2.0], np.float32)
        full = vals if cfg.name == "c0b" else vals[ds_id:ds_id + 1]
        return to16_host(full[lo:hi], cfg.dtype)
    m = hi - lo
    r = rng(cfg, KIND_GRAD, step, vrank, ds_id, lo)
    x = r.standard_normal(m, dtype=np.float32) * np.float32(cfg.grad_std)
    if cfg.outlier_prob > 0:
        mask = r.random(m) < cfg.outlier_prob
        x[mask] *= np.float32(cfg.outlier_mult)
    return to16_host(x, cfg.dtype)


def random_bits16(seed: int, n: int, dtype: str, std: float = 1.0, *words: int) -> np.ndarray:
    """Generic N(0, std) 16-bit values for property tests."""
    x = rng(seed, *words).standard_normal(n, dtype=np.float32) * np.float32(std)
    return to16_host(x, dtype)


# --------------------------------------------------------------------------
# Device-side generation (full-size workloads)
# --------------------------------------------------------------------------

def _torch_seed(*words: int) -> int:
    h = hashlib.sha256(",".join(str(int(w)) for w in words).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def device_normal16(n: int, std: float, dtype: str, device, words: Sequence[int],
                    outlier_prob: float = 0.0, outlier_mult: float = 100.0, out=None):
    """N(0, std) draws rounded to the 16-bit dtype, generated on ``device``
    in chunks; returns (or fills) a flat ``torch.int16`` tensor of bit
    patterns."""
    import torch
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    if out is None:
        out = torch.empty(n, dtype=torch.int16, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(*words))
    chunk = 1 << 26
    view = out.view(tdt)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        x.mul_(std)
        if outlier_prob > 0:
            mask = torch.rand(e - s, generator=g, device=device) < outlier_prob
            x[mask] *= outlier_mult
        view[s:e].copy_(x)
        del x
    return out
