"""Training-step companions on the GPU against the oracle: the AdamW step of a
LoRA factor and the double quantization of the NF4 block scales.

AdamW: one step from seeded states at several step numbers. float32 master
weights within 2^-20 of the larger of |p| and the update (a handful of float32
roundings); bf16 moments within one bf16 ulp (2^-8 relative) of the exact
values, plus float32 cancellation error relative to the two terms of each
moment update; the bf16 parameter copy is exactly the nearest-even bf16 of the
returned master value. Double quantization: codes, scales and offsets
bit-exact (every step is a float32 operation with a fixed rounding), the
dequantized scales bit-exact, and a forward through the dequantized scales
within the linear's own tolerance.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dq as odq
from oracle import lora as olora
from oracle import nf4 as onf4
from oracle import optim as ooptim

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import qlora_linear_amd as q
    q.library()
    return q


def _bf16_dev(bits):
    from tests.gpu_util import dev_bf16
    return dev_bf16(bits)


def _bits(t):
    from tests.gpu_util import host_bits
    return host_bits(t)


HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.mark.parametrize("n,step", [(13, 1), (4096 * 16 + 5, 3), (4096 * 16, 1000), (8, 2)])
def test_adamw_step_matches_oracle(q, n, step):
    inp = synth.optimizer_inputs(7 + step, n)
    f32 = lambda v: float(np.float32(v))  # hyper-parameters cross the ABI as float32
    hp = {k: f32(v) for k, v in HP.items()}
    p_ref, m_ref, v_ref = ooptim.adamw_step(inp["p"].astype(np.float64), olora.bf16_to_f64(inp["grad"]),
                                            olora.bf16_to_f64(inp["m"]), olora.bf16_to_f64(inp["v"]), step,
                                            hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
    p = torch.from_numpy(inp["p"].copy()).cuda()
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    g, m, v = _bf16_dev(inp["grad"]), _bf16_dev(inp["m"]), _bf16_dev(inp["v"])
    q.lora_adamw_step(p, pb, g, m, v, step, hp["lr"], (hp["beta1"], hp["beta2"]), hp["eps"], hp["weight_decay"])
    torch.cuda.synchronize()
    p_got = p.cpu().numpy().astype(np.float64)
    upd = np.abs(p_ref - inp["p"] * (1 - hp["lr"] * hp["weight_decay"]))
    assert np.all(np.abs(p_got - p_ref) <= 2.0 ** -20 * np.maximum(np.abs(p_ref), upd) + 1e-30)
    # float32 evaluation of beta m + (1 - beta) g can cancel: its error is relative
    # to the two terms; the bf16 store then adds half an ulp of the result
    g64, m64, v64 = (olora.bf16_to_f64(inp[k]) for k in ("grad", "m", "v"))
    terms_m = hp["beta1"] * np.abs(m64) + (1 - hp["beta1"]) * np.abs(g64)
    terms_v = hp["beta2"] * v64 + (1 - hp["beta2"]) * g64 * g64
    for got_t, ref, terms in ((m, m_ref, terms_m), (v, v_ref, terms_v)):
        got = olora.bf16_to_f64(_bits(got_t))
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * terms + 1e-38)
    np.testing.assert_array_equal(_bits(pb), synth.f32_to_bf16_bits(p.cpu().numpy()))
    assert np.array_equal(_bits(g), inp["grad"])  # the gradient is read-only


def test_adamw_chain_tracks_torch_adamw(q):
    """Ten steps on the GPU against PyTorch's AdamW in float64 on the CPU (whose
    moments are not rounded to bf16): the master weights stay within a few
    bf16-state roundings of the float64 trajectory."""
    n = 4096
    inp = synth.optimizer_inputs(3, n)
    p = torch.from_numpy(inp["p"].copy()).cuda()
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    tp = torch.tensor(inp["p"].astype(np.float64), requires_grad=True)
    lr = float(np.float32(1e-3))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(float(np.float32(0.9)), float(np.float32(0.99))),
                            eps=float(np.float32(1e-8)), weight_decay=float(np.float32(0.1)))
    grads = [synth.optimizer_inputs(100 + t, n)["grad"] for t in range(10)]
    for t, gb in enumerate(grads, start=1):
        q.lora_adamw_step(p, pb, _bf16_dev(gb), m, v, t, lr, (0.9, 0.99), 1e-8, 0.1)
        tp.grad = torch.from_numpy(olora.bf16_to_f64(gb))
        opt.step()
    torch.cuda.synchronize()
    moved = np.abs(tp.detach().numpy() - inp["p"])
    err = np.abs(p.cpu().numpy().astype(np.float64) - tp.detach().numpy())
    assert np.max(err) <= 0.05 * np.max(moved)


@pytest.mark.parametrize("rows,cols", [(1003, 4096), (4096, 4096), (3, 64)])
def test_absmax_double_quant_bit_exact(q, rows, cols):
    w = synth.normal_bf16(synth.rng(9, rows, cols), (rows, cols), 0.02)
    _, absmax_h = onf4.quantize(synth.bf16_bits_to_f32(w))
    qc_ref, sc_ref, off_ref = odq.quantize_absmax(absmax_h)
    back_ref = odq.dequantize_absmax(qc_ref, sc_ref, off_ref)
    _, absmax = q.nf4_quantize(_bf16_dev(w))
    qc, sc, off = q.nf4_absmax_quantize(absmax)
    back = q.nf4_absmax_dequantize(qc, sc, off)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qc.cpu().numpy(), qc_ref)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), sc_ref.view(np.uint32))
    np.testing.assert_array_equal(off.cpu().numpy().view(np.uint32), off_ref.view(np.uint32))
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint32), back_ref.view(np.uint32))


def test_forward_through_double_quantized_scales(q):
    T, K, N, r, alpha = 300, 512, 320, 16, 16.0
    inp = synth.custom_inputs(21, T, K, N, r)
    codes_h, absmax_h = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
    a2_h = odq.dequantize_absmax(*odq.quantize_absmax(absmax_h)).reshape(absmax_h.shape)
    y_ref, _ = olora.forward(olora.bf16_to_f64(inp["x"]), onf4.dequantize_exact(codes_h, a2_h),
                             olora.bf16_to_f64(inp["A"]), olora.bf16_to_f64(inp["B"]), alpha, r)
    codes, absmax = q.nf4_quantize(_bf16_dev(inp["W"]))
    a2 = q.nf4_absmax_dequantize(*q.nf4_absmax_quantize(absmax)).view_as(absmax)
    y, _ = q.lora_nf4_fwd(_bf16_dev(inp["x"]), codes, a2, _bf16_dev(inp["A"]), _bf16_dev(inp["B"]), alpha)
    torch.cuda.synchronize()
    got = olora.bf16_to_f64(_bits(y))
    assert olora.rel_err(got, y_ref) <= 1e-2
    # the double-quantized scales change the weight by at most 2^-4 of a block's spread
    d_full = onf4.dequantize_exact(codes_h, absmax_h)
    d_dq = onf4.dequantize_exact(codes_h, a2_h)
    assert np.max(np.abs(d_dq - d_full)) <= np.max(np.abs(d_full)) * 0.1
