"""The rank-r gradients alone (lora_nf4_grad_ab): dA = x^T G and dB = s U^T dY from
bf16 G and U, against the oracle.

G = bf16(s dY B^T) and U = bf16(x A) are formed on the host from the seeded bf16
inputs. Two comparisons per case:
  - against the products of exactly those bf16 inputs in float64 (only the float32
    sums over T and the bf16 rounding of dA, dB stand between them: within 5e-3 of
    max |ref|, the bf16 rounding alone being at most 2^-8 of each element);
  - against the oracle's dA, dB of the linear (oracle.lora.lora_factor_grads, from x,
    dY, A, B in float64, G and U unrounded) within the linear's tolerance 1e-2.
Cases: the one-launch rank-r kernel (r % 8 == 0, r <= 64) on ragged T and d_out
(one to several token splits), the generic split-T kernels (r = 12, 72), the
register-dequantizing backward's shape (q_proj at 8192 tokens, r = 16), the empty
batch, and bitwise run-to-run equality.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import lora as olora

pytestmark = pytest.mark.gpu
TOL = 1e-2
TOL_PRODUCT = 5e-3


@pytest.fixture(scope="module")
def q():
    import qlora_linear_amd as q
    q.library()
    return q


def _f64(bits):
    return olora.bf16_to_f64(bits)


def _inputs(seed, T, K, N, r, alpha):
    inp = synth.custom_inputs(seed, T, K, N, r, dy_std=0.1)
    s = alpha / r
    x, dy, A, B = (_f64(inp[k]) for k in ("x", "dY", "A", "B"))
    g_bits = synth.f32_to_bf16_bits((s * (dy @ B.T)).astype(np.float32))
    u_bits = synth.f32_to_bf16_bits((x @ A).astype(np.float32))
    return inp, g_bits, u_bits


CASES = [(300, 256, 320, 16), (1000, 512, 264, 8), (64, 128, 72, 32), (4100, 256, 520, 64),
         (257, 128, 72, 12), (130, 192, 136, 72)]


@pytest.mark.parametrize("T,K,N,r", CASES)
def test_grad_ab_matches_oracle(q, T, K, N, r):
    from tests.gpu_util import dev_bf16, host_f64
    alpha = 16.0
    inp, g_bits, u_bits = _inputs(40 + r, T, K, N, r, alpha)
    x, dy, g, u = dev_bf16(inp["x"]), dev_bf16(inp["dY"]), dev_bf16(g_bits), dev_bf16(u_bits)
    dA, dB = q.lora_nf4_grad_ab(x, g, dy, u, alpha)
    torch.cuda.synchronize()
    s = alpha / r
    xf, dyf, gf, uf = _f64(inp["x"]), _f64(inp["dY"]), _f64(g_bits), _f64(u_bits)
    assert olora.rel_err(host_f64(dA), xf.T @ gf) <= TOL_PRODUCT, ("dA", T, K, N, r)
    assert olora.rel_err(host_f64(dB), s * (uf.T @ dyf)) <= TOL_PRODUCT, ("dB", T, K, N, r)
    dA_ref, dB_ref = olora.lora_factor_grads(xf, dyf, _f64(inp["A"]), _f64(inp["B"]), alpha, r)
    assert olora.rel_err(host_f64(dA), dA_ref) <= TOL
    assert olora.rel_err(host_f64(dB), dB_ref) <= TOL
    dA2, dB2 = q.lora_nf4_grad_ab(x, g, dy, u, alpha)
    torch.cuda.synchronize()
    assert torch.equal(dA, dA2) and torch.equal(dB, dB2)


def test_grad_ab_full_size_q_proj(q):
    """Llama-3-8B q_proj at 8192 tokens, r = 16: the shape the benchmark times."""
    from tests.gpu_util import dev_bf16, host_f64
    w = next(x for x in synth.WORKLOADS if x.name == "llama3-8b-q_proj")
    inp = synth.projection_inputs(w, 0)
    T, r, alpha = w.tokens, w.r, w.alpha
    s = alpha / r
    x, dy, A, B = (_f64(inp[k]) for k in ("x", "dY", "A", "B"))
    g_bits = synth.f32_to_bf16_bits((s * (dy @ B.T)).astype(np.float32))
    u_bits = synth.f32_to_bf16_bits((x @ A).astype(np.float32))
    dA, dB = q.lora_nf4_grad_ab(dev_bf16(inp["x"]), dev_bf16(g_bits), dev_bf16(inp["dY"]), dev_bf16(u_bits), alpha)
    torch.cuda.synchronize()
    assert olora.rel_err(host_f64(dA), x.T @ _f64(g_bits)) <= TOL_PRODUCT
    assert olora.rel_err(host_f64(dB), s * (_f64(u_bits).T @ dy)) <= TOL_PRODUCT
    dA_ref, dB_ref = olora.lora_factor_grads(x, dy, A, B, alpha, r)
    assert olora.rel_err(host_f64(dA), dA_ref) <= TOL
    assert olora.rel_err(host_f64(dB), dB_ref) <= TOL


def test_grad_ab_empty_batch(q):
    import ctypes
    lib = q.library()
    K, N, r = 128, 64, 16
    dA = torch.full((K, r), 1.0, dtype=torch.bfloat16, device="cuda")
    dB = torch.full((r, N), 1.0, dtype=torch.bfloat16, device="cuda")
    st = lib.lora_nf4_grad_ab(0, K, N, r, 16.0, None, None, None, None, dA.data_ptr(), dB.data_ptr(), None,
                              ctypes.c_size_t(0), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert not dA.float().any() and not dB.float().any()
