"""Double quantization of the NF4 block scales (absmax) — oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

The pages keep the base weight resident in 4-bit form to save memory ("Reading
the Unsloth changelog", section 1.1 and the memory list of section 1) but say
nothing about the per-block scales, which cost 32 bits per 64 weights at
float32. Double quantization (Dettmers et al., QLoRA, 2023, section 3)
quantizes those scales once more: 8-bit floats in blocks of 256 scales, centred
before quantization. The readings taken (all fixed here, none by the pages):

* 8-bit format: OCP FP8 E4M3 ("E4M3FN": 1 sign, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals, largest finite 448, no infinities). Encoding
  rounds to the nearest representable value, ties to the even code, and
  saturates magnitudes beyond 448 to 448; the sign of the code is the sign bit
  of the input.
* Blocks: 256 consecutive entries of the row-major absmax array (the last
  block may be shorter). Per block, with lo and hi its minimum and maximum:
      offset = f32(lo / 2 + hi / 2)                  (one rounding)
      d      = max(f32(hi - offset), f32(offset - lo))
      scale  = f32(d / 448)                          (correctly rounded divide)
      code   = e4m3(f32(f32(a - offset) / scale))     (scale > 0; else code 0)
  The centring uses the block's mid-range rather than a global mean, so the
  result does not depend on a summation order.
* Dequantization: a' = f32(f32(e4m3value(code) * scale) + offset), two
  roundings, no fused multiply-add. The NF4 dequantization then uses a' in
  place of absmax.

Every step is stated as float32 operations, so the float32 arithmetic here
(numpy float32, IEEE-754 round-to-nearest-even) is the definition itself.
"""
from __future__ import annotations

import numpy as np

DQ_BLOCK = 256
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 E4M3FN codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        mant = c & 7
        if e == 0xF and mant == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sign * mant * 2.0 ** -9
        else:
            out[c] = sign * (1.0 + mant / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of each finite float32 value, ties to the even code,
    saturating at +-448. Brute force over the 127 non-negative finite codes."""
    x = np.asarray(x, dtype=np.float32).ravel()
    vals = e4m3_values()[:0x7F]  # codes 0x00 .. 0x7E, ascending values
    out = np.empty(x.size, dtype=np.uint8)
    signs = np.signbit(x)
    for i, xi in enumerate(np.abs(x.astype(np.float64))):
        if xi >= E4M3_MAX:
            c = 0x7E
        else:
            dist = np.abs(vals - xi)
            best = dist.min()
            cands = np.nonzero(dist == best)[0]
            c = int(cands[0]) if cands.size == 1 else int(cands[cands % 2 == 0][0])
        out[i] = c | (0x80 if signs[i] else 0)
    return out


def quantize_absmax(absmax: np.ndarray):
    """float32 absmax [n] (any shape, row-major) -> (codes uint8 [n], scale float32
    [ceil(n/256)], offset float32 [ceil(n/256)]), per the module docstring."""
    a = np.ascontiguousarray(absmax, dtype=np.float32).ravel()
    n = a.size
    nb = (n + DQ_BLOCK - 1) // DQ_BLOCK
    codes = np.zeros(n, dtype=np.uint8)
    scale = np.zeros(nb, dtype=np.float32)
    offset = np.zeros(nb, dtype=np.float32)
    half = np.float32(0.5)
    for b in range(nb):
        blk = a[b * DQ_BLOCK:(b + 1) * DQ_BLOCK]
        lo, hi = blk.min(), blk.max()
        off = np.float32(lo * half + hi * half)  # products exact; one rounded add
        d = max(np.float32(hi - off), np.float32(off - lo))
        sc = np.float32(d / np.float32(E4M3_MAX))
        offset[b], scale[b] = off, sc
        if sc > 0:
            t = (blk - off).astype(np.float32) / sc
            codes[b * DQ_BLOCK:b * DQ_BLOCK + blk.size] = e4m3_encode(t.astype(np.float32))
    return codes, scale, offset


def dequantize_absmax(codes: np.ndarray, scale: np.ndarray, offset: np.ndarray) -> np.ndarray:
    """float32 [n]: a' = f32(f32(value(code) * scale) + offset), block b = i // 256."""
    c = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    blk = np.arange(c.size) // DQ_BLOCK
    v = e4m3_values()[c].astype(np.float32)  # every finite code is exact in float32
    prod = (v * scale[blk]).astype(np.float32)
    return (prod + offset[blk]).astype(np.float32)
