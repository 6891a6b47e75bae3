"""NF4 quantize / dequantize on the GPU: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import qlora_linear_amd as q
    q.library()
    return q


def _gpu_quant(q, w_bits=None, w_f32=None):
    if w_bits is not None:
        from tests.gpu_util import dev_bf16
        w = dev_bf16(w_bits)
    else:
        w = torch.from_numpy(w_f32).cuda()
    codes, absmax = q.nf4_quantize(w)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), absmax.cpu().numpy()


def _check_exact(codes, absmax, w_f32):
    rc, ra = onf4.quantize(w_f32)
    assert codes.shape == rc.shape and absmax.shape == ra.shape
    bad = np.argwhere(codes != rc)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    assert np.array_equal(absmax.view(np.uint32), ra.view(np.uint32))


@pytest.mark.parametrize("wi,pi", [(0, 0), (1, 0), (2, 1)])
def test_quantize_workload_weights_bf16(lib, wi, pi):
    w = synth.WORKLOADS[wi]
    bits = synth.projection_inputs(w, pi, tensors=("W",))["W"]
    codes, absmax = _gpu_quant(lib, w_bits=bits)
    _check_exact(codes, absmax, synth.bf16_bits_to_f32(bits))


def test_quantize_f32_and_edge_blocks(lib):
    g = np.random.default_rng(7)
    w = (g.standard_normal((33, 192)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                      # zero block
    w[1, 64:128] = -0.0                  # negative-zero block
    m = onf4.midpoints()
    ties = [float(np.float32(v)) for v in m if float(np.float32(v)) == v]
    w[2, :64] = 0.0
    w[2, 0] = 1.0                        # absmax 1 ...
    for i, t in enumerate(ties):
        w[2, 1 + i] = t                  # ... and exact ties
    w[3, :64] = 1e-30                    # tiny absmax
    w[4, :64] = -3.0e38                  # large magnitude
    w[5, 5] = 123.0
    w[6, :64] = np.linspace(-1, 1, 64, dtype=np.float32)
    codes, absmax = _gpu_quant(lib, w_f32=w)
    _check_exact(codes, absmax, w)


def test_quantize_ragged_rows(lib):
    g = np.random.default_rng(8)
    for rows, cols in [(1, 64), (3, 64), (7, 320), (129, 128)]:
        w = (g.standard_normal((rows, cols)) * 0.02).astype(np.float32)
        codes, absmax = _gpu_quant(lib, w_f32=w)
        _check_exact(codes, absmax, w)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_bit_exact(lib, dtype):
    g = np.random.default_rng(9)
    rows, cols = 77, 256
    codes = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    absmax = np.abs(g.standard_normal((rows, cols // 64)) * 0.05).astype(np.float32)
    absmax[0, 0] = 0.0
    absmax[1, 1] = 1.0
    absmax[2, 2] = 2.0 ** -130           # subnormal products
    out = lib.nf4_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(absmax).cuda(), dtype)
    torch.cuda.synchronize()
    if dtype == torch.float32:
        ref = onf4.dequantize_f32(codes, absmax)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    else:
        ref = onf4.dequantize_bf16(codes, absmax)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref)


def test_quantize_dequantize_full_qproj_weight(lib):
    """Full 4096 x 4096 weight: codes, absmax and the bf16 dequantization bit-exact."""
    w = synth.WORKLOADS[1]
    bits = synth.projection_inputs(w, 0, tensors=("W",))["W"]
    from tests.gpu_util import dev_bf16
    codes, absmax = lib.nf4_quantize(dev_bf16(bits))
    deq = lib.nf4_dequantize(codes, absmax, torch.bfloat16)
    torch.cuda.synchronize()
    rc, ra = onf4.quantize(synth.bf16_bits_to_f32(bits))
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    got = deq.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, onf4.dequantize_bf16(rc, ra))
