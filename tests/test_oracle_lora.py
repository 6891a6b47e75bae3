"""Pins for the oracle's LoRA forward and backward (CPU only).

Brute-force loops, reductions to the dequantized base matmul, finite
differences of <dY, y> and the Euler (homogeneity) identities.
"""
import numpy as np
import pytest

from oracle import lora, nf4


def _case(seed, T=5, K=128, N=6, r=3, alpha=6.0):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, K))
    Wt = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, absmax = nf4.quantize(Wt)
    D = nf4.dequantize_exact(codes, absmax)
    A = g.uniform(-1, 1, (K, r)) / np.sqrt(K)
    B = g.standard_normal((r, N)) * 0.1
    dY = g.standard_normal((T, N))
    return x, D, A, B, dY, alpha, r


def test_forward_matches_triple_loop():
    x, D, A, B, dY, alpha, r = _case(0, T=3, K=64, N=4, r=2)
    y, U = lora.forward(x, D, A, B, alpha, r)
    T, K = x.shape
    N = D.shape[0]
    s = alpha / r
    for t in range(T):
        u = [sum(x[t, k] * A[k, j] for k in range(K)) for j in range(r)]
        for j in range(r):
            assert abs(U[t, j] - u[j]) < 1e-12
        for n in range(N):
            base = sum(x[t, k] * D[n, k] for k in range(K))
            low = sum(u[j] * B[j, n] for j in range(r))
            assert abs(y[t, n] - (base + s * low)) < 1e-12


def test_b_zero_reduces_to_dequantized_base_matmul():
    # Known codes with known scale: every base weight value is written down by hand.
    T, K, N = 4, 64, 3
    codes_unpacked = np.array([[(3 * n + k) % 16 for k in range(K)] for n in range(N)], dtype=np.uint8)
    packed = (codes_unpacked[:, 0::2] | (codes_unpacked[:, 1::2] << 4)).astype(np.uint8)
    absmax = np.array([[0.5], [2.0], [0.25]], dtype=np.float32)
    D = nf4.dequantize_exact(packed, absmax)
    q = nf4.codebook_f32().astype(np.float64)
    hand = np.array([[q[(3 * n + k) % 16] * [0.5, 2.0, 0.25][n] for k in range(K)] for n in range(N)])
    assert np.array_equal(D, hand)
    g = np.random.default_rng(1)
    x = g.standard_normal((T, K))
    A = g.standard_normal((K, 4))
    y, _ = lora.forward(x, D, A, np.zeros((4, N)), 16.0, 4)
    ref = np.array([[sum(x[t, k] * hand[n, k] for k in range(K)) for n in range(N)] for t in range(T)])
    assert np.allclose(y, ref, rtol=0, atol=1e-12)


def test_zero_base_gives_scaled_lora_branch():
    x, D, A, B, dY, alpha, r = _case(2)
    Wz = np.zeros((D.shape[0], D.shape[1]), dtype=np.float32)
    codes, absmax = nf4.quantize(Wz)
    Dz = nf4.dequantize_exact(codes, absmax)
    assert np.all(Dz == 0)
    y, U = lora.forward(x, Dz, A, B, alpha, r)
    assert np.allclose(y, (alpha / r) * (x @ A) @ B, rtol=0, atol=1e-13)


def test_forward_affine_in_scale():
    x, D, A, B, dY, alpha, r = _case(3)
    y0, _ = lora.forward(x, D, A, B, 0.0, r)
    y1, _ = lora.forward(x, D, A, B, alpha, r)
    y2, _ = lora.forward(x, D, A, B, 2 * alpha, r)
    assert np.allclose(y2 - y1, y1 - y0, atol=1e-12)
    assert np.allclose(y0, x @ D.T, atol=1e-12)


def _loss(x, D, A, B, dY, alpha, r):
    return float(np.sum(dY * lora.forward(x, D, A, B, alpha, r)[0]))


@pytest.mark.parametrize("seed", [4, 5])
def test_backward_matches_finite_differences(seed):
    x, D, A, B, dY, alpha, r = _case(seed, T=3, K=64, N=5, r=2)
    dX, dA, dB = lora.backward(x, dY, D, A, B, alpha, r)
    h = 1e-3  # the loss is linear in each of x, A, B alone: central differences are exact up to roundoff
    for name, P, grad in (("x", x, dX), ("A", A, dA), ("B", B, dB)):
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args = {"x": x, "A": A, "B": B}
            args[name] = Pp
            lp = _loss(args["x"], D, args["A"], args["B"], dY, alpha, r)
            args[name] = Pm
            lm = _loss(args["x"], D, args["A"], args["B"], dY, alpha, r)
            fd[idx] = (lp - lm) / (2 * h)
        assert np.max(np.abs(fd - grad)) <= 1e-9 * max(1.0, np.max(np.abs(grad))), name


def test_euler_identities():
    x, D, A, B, dY, alpha, r = _case(6, T=7, K=192, N=9, r=4)
    y, U = lora.forward(x, D, A, B, alpha, r)
    dX, dA, dB = lora.backward(x, dY, D, A, B, alpha, r)
    lora_part = float(np.sum(dY * (y - x @ D.T)))
    assert np.isclose(np.sum(dX * x), np.sum(dY * y), rtol=1e-12)
    assert np.isclose(np.sum(dA * A), lora_part, rtol=1e-12)
    assert np.isclose(np.sum(dB * B), lora_part, rtol=1e-12)


def test_degenerate_factors():
    x, D, A, B, dY, alpha, r = _case(7)
    dX, dA, dB = lora.backward(x, dY, D, A, np.zeros_like(B), alpha, r)
    assert np.all(dA == 0)
    assert np.allclose(dX, dY @ D, atol=1e-13)
    dX, dA, dB = lora.backward(x, dY, D, np.zeros_like(A), B, alpha, r)
    assert np.all(dB == 0)


def test_rel_err_helper():
    assert lora.rel_err([1.0, -2.0], [1.0, -2.0]) == 0.0
    assert lora.rel_err([1.0, -2.5], [1.0, -2.0]) == 0.25
    assert lora.rel_err([0.0], [0.0]) == 0.0


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4049], dtype=np.uint16)
    assert list(lora.bf16_to_f64(bits)) == [1.0, -1.0, 0.0, 3.140625]


def test_factor_grads_agree_with_full_backward():
    x, D, A, B, dY, alpha, r = _case(8, T=9, K=128, N=7, r=5)
    _, dA, dB = lora.backward(x, dY, D, A, B, alpha, r)
    dA2, dB2 = lora.lora_factor_grads(x, dY, A, B, alpha, r)
    assert np.allclose(dA, dA2, rtol=0, atol=1e-13) and np.allclose(dB, dB2, rtol=0, atol=1e-13)


# ---- merge: W' = D + s (A B)^T ------------------------------------------------------

def test_merge_reproduces_the_forward():
    """x W'^T equals the forward's y: pins orientation and scale of the merge
    against the forward (itself pinned by the triple loop above)."""
    g = np.random.default_rng(31)
    T, K, N, r, alpha = 5, 12, 7, 3, 6.0
    x, D = g.standard_normal((T, K)), g.standard_normal((N, K))
    A, B = g.standard_normal((K, r)), g.standard_normal((r, N))
    y, _ = lora.forward(x, D, A, B, alpha, r)
    Wm = lora.merge(D, A, B, alpha, r)
    assert Wm.shape == (N, K)
    np.testing.assert_allclose(x @ Wm.T, y, rtol=1e-12, atol=1e-12)


def test_merge_rank_one_elementwise():
    """r = 1: W'[n, k] = D[n, k] + alpha a[k] b[n], written out element by element."""
    g = np.random.default_rng(32)
    K, N, alpha = 6, 4, 2.5
    D = g.standard_normal((N, K))
    a, b = g.standard_normal(K), g.standard_normal(N)
    Wm = lora.merge(D, a.reshape(K, 1), b.reshape(1, N), alpha, 1)
    for n in range(N):
        for k in range(K):
            assert abs(Wm[n, k] - (D[n, k] + alpha * a[k] * b[n])) <= 1e-12


def test_merge_with_zero_b_is_the_dequantized_base():
    g = np.random.default_rng(33)
    D = g.standard_normal((8, 16))
    assert np.array_equal(lora.merge(D, g.standard_normal((16, 4)), np.zeros((4, 8)), 16.0, 4), D)
