"""Pure-Python, per-element brute force for tiny inputs (TEST INFRASTRUCTURE ONLY).

A second derivation of the oracle's results, structured differently on
purpose so that an indexing or arithmetic slip in ``oracle.zero3`` shows up:

* layouts are walked element by element through the *inverse* map (which
  rank and which local position owns element e of a parameter);
* fp32 arithmetic is emulated on Python floats: each +, -, *, /, sqrt is
  done in binary64 and rounded to binary32 with ``struct``.  Because 53 >=
  2 * 24 + 2, rounding the binary64 result of one such operation to binary32
  gives the correctly rounded binary32 result (double rounding is innocuous
  for these five operations; Figueroa's theorem), for normal results;
* 16-bit conversions use ``struct``'s binary16 packing (fp16) and an exact
  rational rounding written from the definition of round-to-nearest-even
  (bf16);
* sums of squares use ``math.fsum`` (exactly rounded).

Page tags are defined in ``oracle/__init__.py``; each function cites the
passage it restates.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction
from typing import Dict, List, Sequence, Tuple


def f32(x: float) -> float:
    """Round a binary64 value to the nearest binary32 (ties to even)."""
    try:
        return struct.unpack("<f", struct.pack("<f", x))[0]
    except OverflowError:
        return math.copysign(math.inf, x)


def fp16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def fp16_bits(x: float) -> int:
    try:
        return struct.unpack("<H", struct.pack("<e", x))[0]
    except OverflowError:
        return 0xFC00 if x < 0 else 0x7C00


def bf16_bits(x: float) -> int:
    """Nearest bf16 (8 significant bits, fp32 exponent range), ties to even,
    derived with exact rationals."""
    if math.isnan(x):
        raise ValueError("nan")
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    a = Fraction(abs(x))
    # exponent e with 2^e <= a < 2^(e+1)
    e = math.floor(math.log2(abs(x)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                    # below 2^-126 the spacing stays 2^-133
    q = Fraction(2) ** (e - 7)          # spacing of 8-bit significands at this exponent
    n = a / q
    k = math.floor(n)
    r = n - k
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and k % 2 == 1):
        k += 1
    value = k * q
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    # encode
    bits = struct.unpack("<I", struct.pack("<f", float(value)))[0] >> 16
    return sign | bits


def value16(bits: int, dtype: str) -> float:
    return fp16_value(bits) if dtype == "fp16" else bf16_value(bits)


def bits16(x: float, dtype: str) -> int:
    return fp16_bits(x) if dtype == "fp16" else bf16_bits(x)


# --------------------------------------------------------------------------
# Layout through the inverse map
# --------------------------------------------------------------------------

def layout_table(N: int, T: int, ds_ids: Sequence[int], numels: Sequence[int]):
    """List of (ds_id, numel, persistent, ps, offset) in ds_id order
    ([codex] 3.1 element ranges, 5.3 persistence)."""
    rows = sorted(zip(ds_ids, numels))
    out = []
    off = 0
    for d, n in rows:
        pers = n < T
        ps = n if pers else (n + N - 1) // N
        out.append((d, n, pers, ps, off))
        off += ps
    return out, off


def owner(e: int, ps: int) -> Tuple[int, int]:
    """Rank and local position holding element e of a partitioned parameter."""
    return e // ps, e % ps


def partition(N: int, T: int, ds_ids, numels, full: Dict[int, List[int]], rank: int) -> List[int]:
    rows, total = layout_table(N, T, ds_ids, numels)
    out = [0] * total
    for d, n, pers, ps, off in rows:
        for e in range(n):
            if pers:
                out[off + e] = full[d][e]
            else:
                r, k = owner(e, ps)
                if r == rank:
                    out[off + k] = full[d][e]
    return out


def gather_full(N: int, T: int, ds_ids, numels, shards: List[List[int]], bucket: Sequence[int]):
    """Full params of a bucket, element by element, from every rank's flat
    shard ([codex] 5.2): element e of parameter d lives on rank e // ps at
    local position e % ps.  Returns the param-major flat buffer (ds_id
    order) and {ds_id: offset}."""
    rows, _ = layout_table(N, T, ds_ids, numels)
    by_id = {r[0]: r for r in rows}
    out: List[int] = []
    offs = {}
    for d in sorted(bucket):
        _, n, pers, ps, off = by_id[d]
        assert not pers
        offs[d] = len(out)
        for e in range(n):
            r, k = owner(e, ps)
            out.append(shards[r][off + k])
    return out, offs


# --------------------------------------------------------------------------
# Arithmetic of the step
# --------------------------------------------------------------------------

def reduce_scatter_elem(vals: Sequence[int], dtype: str) -> int:
    """One averaged element: fp32 sum from +0 over the ranks in order, fp32
    division by N, round to the 16-bit type ([codex] 6.2, [csdn] step 3)."""
    acc = 0.0
    for b in vals:
        acc = f32(acc + value16(b, dtype))
    avg = f32(acc / len(vals))
    return bits16(avg, dtype)


def sumsq(bits: Sequence[int], dtype: str) -> float:
    return math.fsum(value16(b, dtype) ** 2 for b in bits)


def adam_elem(w: float, m: float, v: float, gbits: int, dtype: str, scale: float,
              lr: float, b1: float, b2: float, eps: float, t: int, wd: float = 0.0):
    """One element of one Adam step, every operation rounded to fp32.  A
    non-zero ``wd`` first shrinks the weight by lr * wd, decoupled from the
    gradient (Loshchilov & Hutter's AdamW)."""
    c_lr, c_b1, c_b2, c_eps = f32(lr), f32(b1), f32(b2), f32(eps)
    omb1, omb2 = f32(1.0 - b1), f32(1.0 - b2)
    bc1, bc2 = f32(1.0 - b1 ** t), f32(1.0 - b2 ** t)
    g = f32(value16(gbits, dtype) * scale)
    if wd != 0.0:
        w = f32(w - f32(f32(lr * wd) * w))
    m = f32(f32(c_b1 * m) + f32(omb1 * g))
    v = f32(f32(c_b2 * v) + f32(omb2 * f32(g * g)))
    mh = f32(m / bc1)
    vh = f32(v / bc2)
    den = f32(f32(math.sqrt(vh)) + c_eps)
    w = f32(w - f32(c_lr * f32(mh / den)))
    return w, m, v, bits16(w, dtype)
