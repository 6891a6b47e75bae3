"""Pins for the oracle's NF4 codebook, quantizer and dequantizer (CPU only).

Each check compares the oracle with something other than itself: an independent
quantile routine (SciPy, 50-digit mpmath), exact rational brute force, closed
forms and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4

Q32 = nf4.codebook_f32()


def _construct(ppf):
    """The NormalFloat construction, spelt out again with a different quantile routine."""
    delta = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)
    pos = [ppf(delta + i * (0.5 - delta) / 8) for i in range(8)]
    neg = [-ppf(delta + i * (0.5 - delta) / 7) for i in range(7)]
    v = sorted(pos + neg + [0.0])
    return np.array(v) / ppf(delta)


def test_codebook_structure():
    assert Q32.dtype == np.float32 and Q32.shape == (16,)
    assert Q32[0] == -1.0 and Q32[7] == 0.0 and Q32[15] == 1.0
    assert np.all(np.diff(Q32.astype(np.float64)) > 0)
    assert np.sum(Q32 > 0) == 8 and np.sum(Q32 < 0) == 7


def test_codebook_matches_scipy_quantile():
    from scipy.special import ndtri
    ref = _construct(lambda p: float(ndtri(p))).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), Q32.view(np.uint32))


def test_codebook_matches_mpmath_50_digits():
    import mpmath
    mpmath.mp.dps = 50

    def ppf(p):
        return float(mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1))

    ref = _construct(ppf).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), Q32.view(np.uint32))


def test_norm_ppf_against_scipy():
    from scipy.special import ndtri
    for p in np.linspace(0.01, 0.99, 97):
        assert abs(nf4.norm_ppf(float(p)) - float(ndtri(p))) < 1e-12


def test_levels_are_quantiles_of_evenly_spaced_probabilities():
    # Undo the normalization and map back through the CDF (a different function
    # from the quantile routine): the positive levels sit at evenly spaced
    # probabilities from delta down towards 1/2.
    from scipy.special import ndtr, ndtri
    delta = nf4.DELTA
    top = float(ndtri(delta))
    q64 = nf4.codebook_f64()
    probs = ndtr(q64[8:][::-1] * top)  # largest first
    assert np.allclose(probs, [delta + i * (0.5 - delta) / 8 for i in range(8)], atol=1e-12)
    probs_neg = ndtr(-q64[:7] * top)  # most negative first
    assert np.allclose(probs_neg, [delta + i * (0.5 - delta) / 7 for i in range(7)], atol=1e-12)


def _random_blocks(seed, rows, std=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((rows, 64)) * std).astype(np.float32)


@pytest.mark.parametrize("seed", range(4))
def test_quantize_equals_rational_brute_force(seed):
    w = _random_blocks(seed, 6, std=0.02)
    codes, absmax = nf4.quantize(w)
    c = nf4.unpack(codes)
    for i in range(w.shape[0]):
        a = float(np.max(np.abs(w[i].astype(np.float64))))
        assert absmax[i, 0] == np.float32(a)
        for j in range(64):
            assert c[i, j] == nf4.nearest_code_exact(float(w[i, j]), a), (i, j)


def test_brute_force_helper_on_hand_cases():
    # The rational reference itself, on values whose nearest level is obvious.
    assert nf4.nearest_code_exact(1.0, 1.0) == 15
    assert nf4.nearest_code_exact(-1.0, 1.0) == 0
    assert nf4.nearest_code_exact(0.0, 1.0) == 7
    assert nf4.nearest_code_exact(-0.09, 1.0) == 6
    assert nf4.nearest_code_exact(0.5, 2.0) == 10  # 0.25 -> level 0.2461...
    assert nf4.nearest_code_exact(0.0, 0.0) == 7


def test_forced_ties_go_to_higher_code():
    m = nf4.midpoints()
    exact = [i for i in range(15) if float(np.float32(m[i])) == m[i]]
    assert exact, "some midpoints are float32-exact"
    for i in exact:
        w = np.zeros((1, 64), dtype=np.float32)
        w[0, 0] = 1.0  # absmax 1
        w[0, 1] = np.float32(m[i])
        c = nf4.unpack(nf4.quantize(w)[0])
        assert c[0, 1] == i + 1
        assert nf4.nearest_code_exact(float(w[0, 1]), 1.0) == i + 1


def test_zero_block_and_signed_zero():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, 64:] = np.float32(-0.0)
    w[1, :64] = _random_blocks(9, 1)[0]
    codes, absmax = nf4.quantize(w)
    c = nf4.unpack(codes)
    assert np.all(c[0] == 7) and np.all(c[1, 64:] == 7)
    assert absmax[0, 0] == 0 and not np.signbit(absmax[0, 0])
    assert absmax[1, 1] == 0 and not np.signbit(absmax[1, 1])
    deq = nf4.dequantize_f32(codes, absmax)
    assert np.all(deq[0] == 0)


def test_extreme_element_codes():
    w = _random_blocks(3, 8)
    codes, absmax = nf4.quantize(w)
    c = nf4.unpack(codes)
    for i in range(8):
        j = int(np.argmax(np.abs(w[i])))
        assert c[i, j] == (15 if w[i, j] > 0 else 0)


def test_grid_round_trip():
    g = np.random.default_rng(11)
    for a in g.uniform(1e-3, 10.0, size=20).astype(np.float32):
        w = np.zeros((1, 64), dtype=np.float32)
        w[0, 0] = a
        w[0, 1:17] = (Q32.astype(np.float64) * np.float64(a)).astype(np.float32)
        codes, absmax = nf4.quantize(w)
        assert absmax[0, 0] == a
        assert list(nf4.unpack(codes)[0, 1:17]) == list(range(16))


def test_power_of_two_scale_invariance():
    w = _random_blocks(5, 4)
    c0, a0 = nf4.quantize(w)
    for k in (-6, -1, 3):
        c1, a1 = nf4.quantize(w * np.float32(2.0 ** k))
        assert np.array_equal(c0, c1)
        assert np.array_equal(a1, a0 * np.float32(2.0 ** k))


def test_packing_low_nibble_even():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = -1.0  # code 0
    w[0, 1] = 1.0   # code 15
    w[0, 2] = 0.0   # code 7
    w[0, 3] = np.float32(Q32[12])
    codes, _ = nf4.quantize(w)
    assert codes[0, 0] == 0xF0
    assert codes[0, 1] == (7 | (12 << 4))


def test_dequant_known_codes():
    c = np.arange(16, dtype=np.uint8)
    packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
    row = np.concatenate([packed] * 4)[None, :]
    one = nf4.dequantize_f32(row, np.array([[1.0]], dtype=np.float32))
    assert np.array_equal(one[0, :16].view(np.uint32), Q32.view(np.uint32))
    for k in (-10, -3, 4):
        sc = nf4.dequantize_f32(row, np.array([[2.0 ** k]], dtype=np.float32))
        assert np.array_equal(sc[0, :16], Q32 * np.float32(2.0 ** k))


def test_dequant_generic_scale_is_single_rounding():
    g = np.random.default_rng(2)
    c = g.integers(0, 16, size=64, dtype=np.uint8)
    packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)[None, :]
    for a in g.uniform(1e-4, 3.0, size=10).astype(np.float32):
        got = nf4.dequantize_f32(packed, np.array([[a]], dtype=np.float32))[0]
        for j in range(64):
            exact = Fraction(float(Q32[c[j]])) * Fraction(float(a))
            assert float(exact) == float(exact.numerator) / float(exact.denominator)
            assert got[j] == np.float32(float(exact))  # fp64 holds the product exactly


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(4)
    v = np.concatenate([g.standard_normal(4096).astype(np.float32) * 0.03,
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)],
                                 dtype=np.float32)])
    ours = nf4.f32_to_bf16_rne(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
