"""Pins for the oracle's optimizer step, rank-stabilized scale and double
quantization of the NF4 block scales (CPU only).

AdamW: PyTorch's own AdamW (float64) over several steps, the closed form of the
first step, zero and constant gradients. rsLoRA: the changelog's example
arguments. E4M3: values fixed by the OCP FP8 format, PyTorch's float8_e4m3fn
conversion, exact midpoints. Double quantization: error bounds, constant
blocks, block extremes, a ragged last block.
"""
import math

import numpy as np
import pytest
import torch

from oracle import dq, optim


# ---- AdamW ------------------------------------------------------------------------

def test_adamw_matches_torch_adamw_over_steps():
    g = np.random.default_rng(0)
    n = 64
    p0 = g.standard_normal(n)
    hp = dict(lr=3e-3, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.05)
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t in range(1, 7):
        grad = g.standard_normal(n) * 10.0 ** g.uniform(-9, 1, n)  # many magnitudes, near eps too
        tp.grad = torch.tensor(grad, dtype=torch.float64)
        opt.step()
        p, m, v = optim.adamw_step(p, grad, m, v, t, **hp)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_first_step_closed_form():
    # bias correction at t = 1 gives m_hat = g and v_hat = g^2
    g = np.array([3.0, -2e-7, 1e-9, -0.5, 0.0])
    p0 = np.array([1.0, -1.0, 0.25, 2.0, -3.0])
    lr, wd, eps = 0.01, 0.1, 1e-8
    p1, m1, v1 = optim.adamw_step(p0, g, np.zeros(5), np.zeros(5), 1, lr, 0.9, 0.999, eps, wd)
    expect = p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    np.testing.assert_allclose(p1, expect, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-15)


def test_adamw_zero_gradient_is_pure_decay():
    p = np.array([1.5, -0.25, 4.0])
    m = v = np.zeros(3)
    lr, wd = 0.02, 0.3
    for t in range(1, 6):
        p, m, v = optim.adamw_step(p, np.zeros(3), m, v, t, lr, 0.9, 0.999, 1e-8, wd)
    np.testing.assert_allclose(p, np.array([1.5, -0.25, 4.0]) * (1 - lr * wd) ** 5, rtol=1e-14)
    assert not m.any() and not v.any()


def test_adamw_constant_gradient_moves_lr_per_step():
    # with a constant gradient the bias-corrected moments equal g and g^2 at every step
    g = np.array([0.3, -2.0, 5e-4])
    p0 = np.array([0.0, 1.0, -1.0])
    p, m, v = p0.copy(), np.zeros(3), np.zeros(3)
    lr, eps = 1e-3, 1e-8
    for t in range(1, 11):
        p, m, v = optim.adamw_step(p, g, m, v, t, lr, 0.8, 0.95, eps, 0.0)
    np.testing.assert_allclose(p, p0 - 10 * lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-15)


def test_adamw_rejects_step_zero():
    with pytest.raises(ValueError):
        optim.adamw_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), 0, 1e-3, 0.9, 0.99, 1e-8, 0.0)


# ---- rsLoRA ------------------------------------------------------------------------

def test_rslora_scale_values():
    # the changelog's example arguments: --r 16 --lora_alpha 32
    assert optim.rslora_scale(32.0, 16) == 8.0
    assert optim.rslora_scale(1.0, 4) == 0.5
    assert optim.rslora_scale(16.0, 1) == 16.0
    for r in (3, 7, 64, 100):
        assert math.isclose(optim.rslora_scale(5.0, r) ** 2 * r, 25.0, rel_tol=1e-14)


# ---- E4M3 --------------------------------------------------------------------------

def test_e4m3_values_fixed_by_the_format():
    v = dq.e4m3_values()
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x3C] == 1.5 and v[0xC0] == -2.0 and v[0x30] == 0.5
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    finite = v[:0x7F]
    assert np.all(np.diff(finite) > 0)  # codes ascend with value


def test_e4m3_encode_matches_torch_float8():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(3000) * 10.0 ** g.uniform(-4, 2.6, 3000),
        (dq.e4m3_values()[:0x7E] + dq.e4m3_values()[1:0x7F]) / 2,  # every positive midpoint
        -(dq.e4m3_values()[:0x7E] + dq.e4m3_values()[1:0x7F]) / 2,
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -11],
    ]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(dq.e4m3_encode(x), ref)


def test_e4m3_encode_ties_and_saturation():
    c = dq.e4m3_encode(np.array([1.0625, 1.1875, 464.0, 470.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -10],
                                dtype=np.float32))
    # 1.0625 between 1.0 (0x38) and 1.125 (0x39): even; 1.1875 between 0x39 and 0x3A: even;
    # 2^-10 between 0 and 2^-9: code 0; 3 * 2^-10 between 2^-9 and 2^-8: code 2
    np.testing.assert_array_equal(c, [0x38, 0x3A, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x02])


# ---- double quantization of absmax ----------------------------------------------------

def _absmax(n, seed):
    g = np.random.default_rng(seed)
    return (np.abs(g.standard_normal(n)) * 0.02 + 0.01).astype(np.float32)


def test_dq_error_bound_and_block_structure():
    a = _absmax(3 * 256 + 44, 2)  # ragged last block
    codes, scale, offset = dq.quantize_absmax(a)
    assert codes.shape == a.shape and scale.shape == offset.shape == (4,)
    back = dq.dequantize_absmax(codes, scale, offset)
    blk = np.arange(a.size) // 256
    lo = np.minimum.reduceat(a, np.arange(0, a.size, 256))
    hi = np.maximum.reduceat(a, np.arange(0, a.size, 256))
    np.testing.assert_allclose(offset, (lo.astype(np.float64) + hi) / 2, rtol=2 ** -24)
    np.testing.assert_allclose(scale, (hi.astype(np.float64) - lo) / 2 / 448, rtol=2 ** -22)
    # E4M3 keeps 3 mantissa bits: half an ulp is 2^-4 relative (normal range) or
    # 2^-10 absolute in units of scale (subnormal range); plus float32 roundings
    centred = np.abs(a.astype(np.float64) - offset[blk])
    bound = np.maximum(centred * 2.0 ** -4, scale[blk].astype(np.float64) * 2.0 ** -10) \
        + 2.0 ** -22 * (np.abs(a) + np.abs(offset[blk]))
    assert np.all(np.abs(back.astype(np.float64) - a) <= bound)
    # every block's extremes map to the saturated codes +-448
    for b in range(4):
        seg = slice(b * 256, min(a.size, (b + 1) * 256))
        cb = codes[seg]
        assert {0x7E, 0xFE} <= set(cb.tolist())


def test_dq_constant_block_is_exact():
    a = np.full(300, 0.0375, dtype=np.float32)
    a[256:] = 0.5
    codes, scale, offset = dq.quantize_absmax(a)
    assert not scale.any() and not codes.any()
    np.testing.assert_array_equal(dq.dequantize_absmax(codes, scale, offset), a)


def test_dq_compresses_absmax_storage():
    # 8 bits per block scale plus 64 bits per 256 blocks, against 32 bits per block
    n = 4096 * 4096 // 64
    bits = (n * 8 + (n // 256) * 64) / (n * 64)
    assert bits < 0.13 < 32 / 64


# ---- AdamW, float32 evaluation and 8-bit state -------------------------------------

HP32 = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _f32(hp):
    return {k: float(np.float32(v)) for k, v in hp.items()}


def test_adamw_f32_within_float32_roundings_of_float64():
    g = np.random.default_rng(5)
    n = 4000
    p = (g.standard_normal(n) * 0.02).astype(np.float32)
    m = (g.standard_normal(n) * 1e-4).astype(np.float32)
    v = (np.abs(g.standard_normal(n)) * 1e-8).astype(np.float32)
    grad = (g.standard_normal(n) * 1e-3 * 10.0 ** g.uniform(-5, 0, n)).astype(np.float32)
    hp = _f32(HP32)
    for step in (1, 7, 1000):
        p32, m32, v32 = optim.adamw_step_f32(p, grad, m, v, step, **hp)
        p64, m64, v64 = optim.adamw_step(p.astype(np.float64), grad.astype(np.float64), m.astype(np.float64),
                                         v.astype(np.float64), step, **hp)
        upd = np.abs(p64 - p.astype(np.float64) * (1 - hp["lr"] * hp["weight_decay"]))
        assert np.all(np.abs(p32 - p64) <= 2.0 ** -20 * np.maximum(np.abs(p64), upd) + 1e-30)
        terms_m = hp["beta1"] * np.abs(m) + (1 - hp["beta1"]) * np.abs(grad)
        terms_v = hp["beta2"] * v + (1 - hp["beta2"]) * grad.astype(np.float64) ** 2
        assert np.all(np.abs(m32 - m64) <= 2.0 ** -22 * terms_m + 1e-38)
        assert np.all(np.abs(v32 - v64) <= 2.0 ** -21 * terms_v + 1e-44)


def test_adamw_f32_second_moment_decays_like_torch_at_beta2_0999():
    """Shrinking gradients at beta2 = 0.999: the float32 v follows PyTorch's float64
    exp_avg_sq; a v rounded to bf16 after every step (the 16-bit state) cannot
    decay (0.1 % per step is below half a bf16 step) and ends far above it."""
    g = np.random.default_rng(6)
    n = 256
    p0 = (g.standard_normal(n) * 0.02).astype(np.float32)
    hp = _f32(HP32)
    tp = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    vb = np.zeros(n, np.float32)  # the same recurrence with v stored as bf16
    base = (g.standard_normal(n) * 1e-2).astype(np.float32)
    for t in range(1, 401):
        grad = (base * np.float32(0.97 ** t)).astype(np.float32)
        tp.grad = torch.from_numpy(grad.astype(np.float64))
        opt.step()
        p, m, v = optim.adamw_step_f32(p, grad, m, v, t, **hp)
        _, _, vb = optim.adamw_step_f32(p, grad, m, vb, t, **hp)
        vb = (torch.from_numpy(vb).to(torch.bfloat16).float().numpy())
    v_ref = opt.state[tp]["exp_avg_sq"].numpy()
    np.testing.assert_allclose(v, v_ref, rtol=1e-4, atol=0)
    moved = np.max(np.abs(tp.detach().numpy() - p0))
    assert np.max(np.abs(p - tp.detach().numpy())) <= 1e-4 * moved
    assert np.median(vb / v_ref) > 1.3  # the bf16 state stays far above


def test_state_encoding_block_structure_and_bounds():
    g = np.random.default_rng(7)
    n = 3 * 256 + 77  # ragged last block
    x = (g.standard_normal(n) * 10.0 ** g.uniform(-3, 0, n)).astype(np.float32)
    x[256:512] = 0.0  # an all-zero block
    codes, scales = optim.encode_state(x)
    assert codes.shape == (n,) and scales.shape == (4,) and scales[1] == 0 and not codes[256:512].any()
    back = optim.decode_state(codes, scales)
    blk = np.arange(n) // 256
    amax = np.array([np.max(np.abs(x[b * 256:(b + 1) * 256])) for b in range(4)])
    np.testing.assert_allclose(scales, amax / 448.0, rtol=2.0 ** -23)
    for b in (0, 2, 3):  # each block's largest element takes the top code
        i = b * 256 + int(np.argmax(np.abs(x[b * 256:(b + 1) * 256])))
        assert codes[i] & 0x7F == 0x7E
        assert abs(back[i] - x[i]) <= 2.0 ** -22 * abs(x[i])
    # half an E4M3 step: 2^-4 relative (normal codes) or 2^-10 scale (subnormal codes),
    # plus the float32 roundings of x / scale and of the decode
    err = np.abs(back.astype(np.float64) - x)
    assert np.all(err <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scales[blk] + 2.0 ** -21 * np.abs(x))


def test_adamw8_first_step_equals_float32_step():
    """From zero state the decoded moments are exactly zero, so the first 8-bit
    step moves the parameter exactly as the float32 step."""
    g = np.random.default_rng(8)
    n = 700
    p = (g.standard_normal(n) * 0.02).astype(np.float32)
    grad = (g.standard_normal(n) * 1e-3).astype(np.float32)
    z8, zs = np.zeros(n, np.uint8), np.zeros(3, np.float32)
    p8, (mc, ms), (vc, vs), (m1, v1) = optim.adamw8_step(p, grad, z8, zs, z8, zs, 1, **_f32(HP32))
    p32, m32, v32 = optim.adamw_step_f32(p, grad, np.zeros(n, np.float32), np.zeros(n, np.float32), 1,
                                         **_f32(HP32))
    np.testing.assert_array_equal(p8, p32)
    np.testing.assert_array_equal(m1, m32)
    np.testing.assert_array_equal(mc, optim.encode_state(m32)[0])


def test_adamw8_tracks_torch_adamw():
    """Thirty steps of 8-bit AdamW against PyTorch's AdamW (float64 state) on
    gradients whose scale varies between blocks: the parameters stay within 10 % of
    their total movement (E4M3 keeps 3 mantissa bits: each decoded moment is off by
    up to 1/16 of itself, or 1/1024 of its block's scale; measured 7 %)."""
    g = np.random.default_rng(9)
    n = 2048
    p0 = (g.standard_normal(n) * 0.02).astype(np.float32)
    hp = _f32(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01))
    tp = torch.tensor(p0.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    blk_scale = np.repeat(10.0 ** g.uniform(-4, -2, n // 256), 256)
    p = p0.copy()
    mc = vc = np.zeros(n, np.uint8)
    ms = vs = np.zeros(n // 256, np.float32)
    for t in range(1, 31):
        grad = (g.standard_normal(n) * blk_scale + 0.3 * blk_scale).astype(np.float32)
        tp.grad = torch.from_numpy(grad.astype(np.float64))
        opt.step()
        p, (mc, ms), (vc, vs), _ = optim.adamw8_step(p, grad, mc, ms, vc, vs, t, **hp)
    ref = tp.detach().numpy()
    moved = np.max(np.abs(ref - p0))
    assert np.max(np.abs(p - ref)) <= 0.10 * moved
