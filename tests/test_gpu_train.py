"""Training-step companions on the GPU against the oracle: the AdamW step of a
LoRA factor and the double quantization of the NF4 block scales.

AdamW: the float32-state and 8-bit-state kernels against the oracle's float32
evaluation, bit for bit (one step from seeded state at several step numbers; a
400-step chain at beta2 = 0.999; five 8-bit steps); the update fused into the
backward's rank-r reduction against the float64 backward and AdamW within the
linear's rounding. Double quantization: codes, scales and offsets
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


def _hp32(hp):
    return {k: float(np.float32(v)) for k, v in hp.items()}  # the values that cross the ABI


def _call_hp(hp):
    return dict(lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"], weight_decay=hp["weight_decay"])


@pytest.mark.parametrize("n,step", [(13, 1), (4096 * 16 + 5, 3), (4096 * 16, 1000), (8, 2)])
def test_adamw_step_bit_exact(q, n, step):
    """float32 moments: master, copy and both moments equal, bit for bit, the
    oracle's float32 evaluation (which itself is pinned to the float64 AdamW)."""
    inp = synth.optimizer_inputs(7 + step, n)
    hp = _hp32(HP)
    g32 = synth.bf16_bits_to_f32(inp["grad"])
    p_ref, m_ref, v_ref = ooptim.adamw_step_f32(inp["p"], g32, inp["m"], inp["v"], step, **hp)
    p = torch.from_numpy(inp["p"].copy()).cuda()
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    m, v = torch.from_numpy(inp["m"].copy()).cuda(), torch.from_numpy(inp["v"].copy()).cuda()
    g = _bf16_dev(inp["grad"])
    q.lora_adamw_step(p, pb, g, m, v, step, **_call_hp(hp))
    torch.cuda.synchronize()
    for got, ref in ((p, p_ref), (m, m_ref), (v, v_ref)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    np.testing.assert_array_equal(_bits(pb), synth.f32_to_bf16_bits(p_ref))
    assert np.array_equal(_bits(g), inp["grad"])  # the gradient is read-only


def test_adamw_chain_second_moment_decays_at_beta2_0999(q):
    """400 steps at beta2 = 0.999 with gradients shrinking 3 % per step: the GPU's
    float32 state equals the oracle's float32 chain bit for bit at the end (the
    oracle chain itself tracks PyTorch's AdamW; a 16-bit v would not decay)."""
    n = 4096 + 37
    g0 = synth.optimizer_inputs(31, n)
    hp = _hp32(HP)
    p = torch.from_numpy(g0["p"].copy()).cuda()
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    pr, mr, vr = g0["p"].copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    base = synth.bf16_bits_to_f32(g0["grad"]) * np.float32(10.0)
    for t in range(1, 401):
        gb = synth.f32_to_bf16_bits(base * np.float32(0.97 ** t))
        q.lora_adamw_step(p, pb, _bf16_dev(gb), m, v, t, **_call_hp(hp))
        pr, mr, vr = ooptim.adamw_step_f32(pr, synth.bf16_bits_to_f32(gb), mr, vr, t, **hp)
    torch.cuda.synchronize()
    for got, ref in ((p, pr), (m, mr), (v, vr)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n", [4096 * 16 + 77, 256, 13])
def test_adamw8_chain_bit_exact(q, n):
    """8-bit blockwise moments: five steps from zero state; codes, scales, master and
    copy equal the oracle's bit for bit after every step (a ragged last block,
    one block, less than one block)."""
    hp = _hp32(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01))
    inp = synth.optimizer_inputs(50, n)
    p = torch.from_numpy(inp["p"].copy()).cuda()
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    state = q.adamw8_state(n)
    pr = inp["p"].copy()
    nb = (n + 255) // 256
    mc, ms, vc, vs = np.zeros(n, np.uint8), np.zeros(nb, np.float32), np.zeros(n, np.uint8), np.zeros(nb, np.float32)
    for t in range(1, 6):
        gb = synth.optimizer_inputs(60 + t, n)["grad"]
        q.lora_adamw8_step(p, pb, _bf16_dev(gb), state, t, **_call_hp(hp))
        pr, (mc, ms), (vc, vs), _ = ooptim.adamw8_step(pr, synth.bf16_bits_to_f32(gb), mc, ms, vc, vs, t, **hp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(state[0].cpu().numpy(), mc)
        np.testing.assert_array_equal(state[2].cpu().numpy(), vc)
        np.testing.assert_array_equal(state[1].cpu().numpy().view(np.uint32), ms.view(np.uint32))
        np.testing.assert_array_equal(state[3].cpu().numpy().view(np.uint32), vs.view(np.uint32))
        np.testing.assert_array_equal(p.cpu().numpy().view(np.uint32), pr.view(np.uint32))
    np.testing.assert_array_equal(_bits(pb), synth.f32_to_bf16_bits(pr))


@pytest.mark.parametrize("T,K,N,r", [(300, 256, 192, 16), (8192, 4096, 4096, 16), (16, 512, 384, 8),
                                     (4100, 512, 256, 64)])
def test_bwd_adamw_fused_matches_oracle(q, T, K, N, r):
    """The backward with AdamW applied in its rank-r reduction against the oracle
    (float64 gradients from the oracle's backward, then the float64 AdamW step)
    from seeded state at step 5 whose moments have the gradients' own scale (m ~
    N(0, sigma), v ~ sigma^2 U(0.5, 1.5), sigma the rms of the oracle's gradient:
    AdamW divides by sqrt(v), so a near-zero v would magnify any rounding of the
    gradient without bound): the moments within 1 % of their largest value and
    the parameter within 2 % of its largest update (the gradients carry the
    linear's bf16 roundings, about 2^-8 relative); A and B are bf16 of the new
    masters; dX as lora_nf4_bwd gives it."""
    from tests.gpu_util import dev_bf16
    alpha, step = 16.0, 5
    hp = _hp32(HP)
    inp = synth.custom_inputs(71, T, K, N, r)
    x, W, A, B, dY = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
    codes, absmax = q.nf4_quantize(W)
    f = olora.bf16_to_f64
    D = onf4.dequantize_exact(*onf4.quantize(synth.bf16_bits_to_f32(inp["W"])))
    _, dA_ref, dB_ref = olora.backward(f(inp["x"]), f(inp["dY"]), D, f(inp["A"]), f(inp["B"]), alpha, r)
    rng = np.random.default_rng(90 + T)

    def state_like(gr):
        sig = float(np.sqrt(np.mean(gr * gr)))
        return {"m": (rng.standard_normal(gr.size) * sig).astype(np.float32),
                "v": (sig * sig * rng.uniform(0.5, 1.5, gr.size)).astype(np.float32)}

    st_a, st_b = state_like(dA_ref), state_like(dB_ref)
    a_master = torch.from_numpy(synth.bf16_bits_to_f32(inp["A"]).ravel().copy()).cuda().view(K, r)
    b_master = torch.from_numpy(synth.bf16_bits_to_f32(inp["B"]).ravel().copy()).cuda().view(r, N)
    state = (a_master, torch.from_numpy(st_a["m"]).cuda().view(K, r), torch.from_numpy(st_a["v"]).cuda().view(K, r),
             b_master, torch.from_numpy(st_b["m"]).cuda().view(r, N), torch.from_numpy(st_b["v"]).cuda().view(r, N))
    _, u = q.lora_nf4_fwd(x, codes, absmax, A, B, alpha, save_u=True)
    dx_ref_gpu, _, _ = q.lora_nf4_bwd(x, dY, codes, absmax, A, B, alpha, u_saved=u)
    A_in, B_in = A.clone(), B.clone()
    dx = q.lora_nf4_bwd_adamw(x, dY, codes, absmax, A, B, alpha, state, step, **_call_hp(hp), u_saved=u)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref_gpu)  # dX read A and B before the update
    for grad_ref, st, master0, shape, got in (
            (dA_ref, st_a, inp["A"], (K, r), (state[0], state[1], state[2], A)),
            (dB_ref, st_b, inp["B"], (r, N), (state[3], state[4], state[5], B))):
        p0 = synth.bf16_bits_to_f32(master0).astype(np.float64).reshape(shape)
        p_ref, m_ref, v_ref = ooptim.adamw_step(p0, grad_ref, st["m"].reshape(shape).astype(np.float64),
                                                st["v"].reshape(shape).astype(np.float64), step, **hp)
        p_got, m_got, v_got = (t.cpu().numpy().astype(np.float64) for t in got[:3])
        upd = np.max(np.abs(p_ref - p0 * (1 - hp["lr"] * hp["weight_decay"])))
        assert np.max(np.abs(p_got - p_ref)) <= 0.02 * upd
        assert np.max(np.abs(m_got - m_ref)) <= 0.01 * np.max(np.abs(m_ref))
        assert np.max(np.abs(v_got - v_ref)) <= 0.02 * np.max(np.abs(v_ref))
        np.testing.assert_array_equal(_bits(got[3]).ravel(), synth.f32_to_bf16_bits(got[0].cpu().numpy()).ravel())
    assert not torch.equal(A, A_in) and not torch.equal(B, B_in)


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
