"""Merged base weight W' = D + s (A B)^T on the GPU against the fp64 oracle.

float32 output: within 1e-6 of the exact value, relative to max|W'| (one rounding
of q * absmax, float32 accumulation of r products, one rounding of the sum).
bf16 output: every element within one bf16 ulp of the exact value, and at least
99 % equal to its correctly rounded bf16 (a float32 intermediate can flip a
rounding only when the exact value sits within ~2^-24 relative of a midpoint).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import lora as olora
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import qlora_linear_amd as q
    q.library()
    return q


def _bf16_ulp(v):
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


# (d_in, d_out, r, alpha): partial tiles in both directions, ranks 1 .. 256 (above
# 128 in two rank passes), d_out not a multiple of 8 (rows of B unaligned)
SHAPES = [(256, 64, 16, 16.0), (320, 72, 8, 16.0), (192, 200, 24, 32.0), (64, 8, 1, 2.0),
          (512, 100, 128, 16.0), (4096, 4096, 16, 16.0), (320, 13, 24, 16.0), (128, 1, 7, 16.0),
          (384, 77, 256, 16.0), (256, 200, 160, 32.0)]


@pytest.mark.parametrize("K,N,r,alpha", SHAPES)
def test_merge_matches_oracle(q, K, N, r, alpha):
    from tests.gpu_util import dev_bf16
    inp = synth.custom_inputs(11, 8, K, N, r)
    codes_h, absmax_h = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
    ref = olora.merge(onf4.dequantize_exact(codes_h, absmax_h), olora.bf16_to_f64(inp["A"]),
                      olora.bf16_to_f64(inp["B"]), alpha, r)
    codes, absmax = q.nf4_quantize(dev_bf16(inp["W"]))
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    w32 = q.lora_nf4_merge(codes, absmax, A, B, alpha, dtype=torch.float32).cpu().numpy().astype(np.float64)
    wbf = q.lora_nf4_merge(codes, absmax, A, B, alpha).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.max(np.abs(w32 - ref)) <= 1e-6 * np.max(np.abs(ref))
    got = olora.bf16_to_f64(wbf)
    assert np.all(np.abs(got - ref) <= _bf16_ulp(ref))
    exact = olora.bf16_to_f64(synth.f32_to_bf16_bits(ref.astype(np.float32)))
    assert np.mean(got == exact) >= 0.99
