"""Helpers for the GPU parity tests: device buffers with canary guards,
16-bit host<->device transfers, and a per-test layout handle."""

from __future__ import annotations

import sys

import numpy as np
import pytest

GUARD = 64                 # canary elements on each side of every output buffer
CANARY16 = 0x5A5A
CANARY32 = -1.2345e-33


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import zero_sharded_state_amd as zs
    zs.lib()                # raises if the HIP library is not built


def note(msg: str) -> None:
    """Name the case before a GPU step (visible even if the step hangs)."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


class Buf16:
    """A device buffer of n 16-bit elements that starts `shift` elements into
    an allocation surrounded by canaries."""

    def __init__(self, n: int, shift: int = 0, fill=None):
        import torch
        self.n, self.shift = int(n), int(shift)
        self.base = torch.full((self.n + 2 * GUARD + shift,), CANARY16 - 65536 if CANARY16 >= 32768 else CANARY16,
                               dtype=torch.int16, device="cuda")
        self.view = self.base[GUARD + shift:GUARD + shift + self.n]
        if fill is not None:
            self.view.copy_(torch.from_numpy(np.ascontiguousarray(fill, np.uint16).view(np.int16)).cuda())

    def ptr(self) -> int:
        return self.view.data_ptr()

    def host(self) -> np.ndarray:
        return self.view.cpu().numpy().view(np.uint16).copy()

    def check_guards(self) -> None:
        b = self.base.cpu().numpy().view(np.uint16)
        lo = b[:GUARD + self.shift]
        hi = b[GUARD + self.shift + self.n:]
        assert np.all(lo == CANARY16) and np.all(hi == CANARY16), "write outside the output buffer"


class Buf32:
    def __init__(self, n: int, shift: int = 0, fill=None):
        import torch
        self.n, self.shift = int(n), int(shift)
        self.base = torch.full((self.n + 2 * GUARD + shift,), CANARY32, dtype=torch.float32, device="cuda")
        self.view = self.base[GUARD + shift:GUARD + shift + self.n]
        if fill is not None:
            self.view.copy_(torch.from_numpy(np.ascontiguousarray(fill, np.float32)).cuda())

    def ptr(self) -> int:
        return self.view.data_ptr()

    def host(self) -> np.ndarray:
        return self.view.cpu().numpy().copy()

    def check_guards(self) -> None:
        b = self.base.cpu().numpy()
        assert np.all(b[:GUARD + self.shift] == np.float32(CANARY32))
        assert np.all(b[GUARD + self.shift + self.n:] == np.float32(CANARY32))


def sync():
    import torch
    torch.cuda.synchronize()


def ordinal16(bits):
    b = np.asarray(bits, np.int64)
    return np.where((b & 0x8000) != 0, -(b & 0x7FFF), b & 0x7FFF)


def assert_f32_close(got, ref, rtol=2e-6, what=""):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    den = np.maximum(np.abs(ref).astype(np.float64), 2.0 ** -126)
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64)) / den
    assert np.all(np.isfinite(got)), what
    assert err.max() <= rtol, f"{what}: max rel err {err.max():.3e} at {int(err.argmax())}"
    return float(err.max()), int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
