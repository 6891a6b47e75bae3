"""NF4 (4-bit NormalFloat) codebook, quantization and dequantization — oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What the pages fix: the frozen base weight of the LoRA linear is held in 4-bit
NF4 form ("Unsloth acceleration principles: CUDA kernel fusion and memory
optimization", kernel-fusion section: ``load_in_4bit=True``; "Reading the
Unsloth changelog", section 1.1: weights resident in NF4 format). The pages name
NF4 but never define it. The readings taken here (each listed in the design doc):

* Codebook: the NormalFloat construction of the QLoRA paper (Dettmers et al.,
  2023, section 3): 16 quantiles of the standard normal with an exact zero,
  8 positive and 7 negative levels, normalized so the outer levels are +-1, each
  rounded to float32.
* Blocks: 64 consecutive elements along a row of the row-major [rows, cols]
  matrix (cols % 64 == 0); one float32 absmax per block.
* Code of w in a block with absmax a > 0: the level nearest to the real number
  w / a, ties to the higher code. All-zero block: absmax +0.0, every code 7.
* Packing: two codes per byte, the even element in the low nibble.
* Dequantization to float32: the exact product q[c] * a rounded once to
  float32 (nearest-even); to bf16: that float32 rounded to nearest-even bf16.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

BLOCK = 64
ZERO_CODE = 7

# Outer probability of the construction: the mean of 1 - 1/(2*15) and
# 1 - 1/(2*16), the half-bin probabilities of 15 and 16 equal-mass bins.
DELTA = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


def norm_cdf(z: float) -> float:
    """Standard normal CDF, Phi(z) = erfc(-z / sqrt 2) / 2, from libm's erfc."""
    return 0.5 * math.erfc(-z / math.sqrt(2.0))


def norm_ppf(p: float) -> float:
    """Standard normal quantile for 0 < p < 1 by bisection on ``norm_cdf``.

    Phi is strictly increasing, so bisection on [-40, 40] converges to the
    float64 point where Phi crosses p; 200 halvings exhaust float64 resolution.
    """
    if not 0.0 < p < 1.0:
        raise ValueError("p must lie in (0, 1)")
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if norm_cdf(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _evenly_spaced(start: float, stop: float, count: int) -> list:
    """``count`` points from start to stop inclusive, evenly spaced."""
    step = (stop - start) / (count - 1)
    return [start + i * step for i in range(count)]


def codebook_f64() -> np.ndarray:
    """The 16 NF4 levels in float64, ascending, before rounding to float32.

    Positive side: quantiles at the first 8 of 9 evenly spaced probabilities from
    DELTA down to 1/2 (1/2 itself, the zero, excluded). Negative side: minus the
    quantiles at the first 7 of 8 evenly spaced probabilities from DELTA to 1/2.
    An exact 0 completes the 16; all are divided by the largest, Phi^-1(DELTA).
    """
    pos = [norm_ppf(p) for p in _evenly_spaced(DELTA, 0.5, 9)[:-1]]
    neg = [-norm_ppf(p) for p in _evenly_spaced(DELTA, 0.5, 8)[:-1]]
    levels = sorted(pos + [0.0] + neg)
    top = max(abs(v) for v in levels)
    return np.array([v / top for v in levels], dtype=np.float64)


def codebook_f32() -> np.ndarray:
    """The NF4 table as stored: each level rounded to the nearest float32."""
    return codebook_f64().astype(np.float32)


def midpoints() -> np.ndarray:
    """Decision thresholds m_i = (q_i + q_{i+1}) / 2 of the float32 table, in float64.

    Each q_i has a 24-bit significand and neighbouring levels differ in exponent
    by at most one, so every sum and half is exact in float64.
    """
    q = codebook_f32().astype(np.float64)
    return (q[:-1] + q[1:]) / 2.0


def quantize(w: np.ndarray):
    """Blockwise NF4 quantization of a row-major [rows, cols] float32 matrix.

    Returns (codes, absmax): codes uint8 [rows, cols // 2] with the even element
    of each pair in the low nibble, absmax float32 [rows, cols // 64].

    code(w) = #{i : w >= m_i * a} — the number of decision thresholds the value
    reaches, i.e. the nearest level to w / a with ties going up. m_i * a has at
    most 27 + 24 significant bits, so the products and comparisons are exact in
    float64.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % BLOCK != 0:
        raise ValueError("expected a 2-D matrix whose row length is a multiple of 64")
    rows, cols = w.shape
    blocks = w.astype(np.float64).reshape(rows, cols // BLOCK, BLOCK)
    a = np.max(np.abs(blocks), axis=2)
    m = midpoints()
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    for mi in m:
        codes += (blocks >= (mi * a)[..., None]).astype(np.uint8)
    codes[a == 0.0] = ZERO_CODE
    flat = codes.reshape(rows, cols)
    packed = (flat[:, 0::2] | (flat[:, 1::2] << 4)).astype(np.uint8)
    absmax = a.astype(np.float32)  # a is a float32 magnitude: exact
    return packed, absmax


def unpack(codes: np.ndarray) -> np.ndarray:
    """uint8 [rows, cols/2] -> codes uint8 [rows, cols] (low nibble = even element)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def dequantize_exact(codes: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """float64 [rows, cols]: the exact products q[c] * a (24 x 24 bits, exact in float64)."""
    c = unpack(codes)
    rows, cols = c.shape
    q = codebook_f32().astype(np.float64)
    a = np.asarray(absmax, dtype=np.float32).astype(np.float64)
    return (q[c].reshape(rows, cols // BLOCK, BLOCK) * a[..., None]).reshape(rows, cols)


def dequantize_f32(codes: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """float32 [rows, cols]: each exact product rounded once to nearest-even float32."""
    return dequantize_exact(codes, absmax).astype(np.float32)


def f32_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 of finite float32 values, as uint16 bit patterns.

    Adding 0x7FFF plus the lowest kept bit to the float32 bit pattern and
    truncating the low 16 bits rounds to nearest with ties to the even pattern.
    """
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    return ((u + 0x7FFF + keep_lsb) >> 16).astype(np.uint16)


def dequantize_bf16(codes: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """bf16 bit patterns [rows, cols]: nearest-even bf16 of ``dequantize_f32``."""
    return f32_to_bf16_rne(dequantize_f32(codes, absmax))


def nearest_code_exact(w: float, a: float) -> int:
    """Brute-force reference for one element: argmin over the 16 levels of
    |w/a - q_c| in exact rational arithmetic, ties to the higher code."""
    if a == 0.0:
        return ZERO_CODE
    t = Fraction(float(w)) / Fraction(float(a))
    q = [Fraction(float(v)) for v in codebook_f32()]
    best, best_d = 0, abs(t - q[0])
    for c in range(1, 16):
        d = abs(t - q[c])
        if d <= best_d:  # '<=' so a tie moves to the higher code
            best, best_d = c, d
    return best
