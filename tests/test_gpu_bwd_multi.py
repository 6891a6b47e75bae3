"""Backward of several projections that share x (lora_nf4_bwd_multi) against the
oracle: dX summed over the projections, dA and dB of each, within the linear's
tolerance (max|err| / max|ref| <= 1e-2).

Cases cover the fused path (every d_out a multiple of 64, T > 128: one dX
launch over the concatenated d_out; for n r <= 64 one rank-r launch for every
dA and dB, up to 192 one for every dA and one for every dB, wider sums one per
projection; n r > 64 in several epilogue passes) with 2, 3,
4 and 8 projections and ranks 8 .. 64, ragged token counts and partial d_in
tiles, G from a pass of its own (rank > 16, from 4096 tokens), from 1024 tokens on weights dequantized into the workspace; and the
per-projection path (a d_out not a multiple of 64, up to 128 tokens,
no dX). One case runs the Qwen-14B-shaped q/k/v at full size
(8192 tokens, 5120 -> 5120 each, r = 16) and checks sampled rows of dX and
sampled columns of dA and dB against the oracle; another runs the Llama-3-70B
gate and up projections (8192 -> 28672, 4096 tokens) the same way.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import lora as olora
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def q():
    import qlora_linear_amd as q
    q.library()
    return q


def _f64(bits):
    return olora.bf16_to_f64(bits)


def _dev_inputs(q, ins):
    from tests.gpu_util import dev_bf16
    x = dev_bf16(ins[0]["x"])
    codes, absmax, A, B, dy = [], [], [], [], []
    for inp in ins:
        c, a = q.nf4_quantize(dev_bf16(inp["W"]))
        codes.append(c), absmax.append(a)
        A.append(dev_bf16(inp["A"])), B.append(dev_bf16(inp["B"])), dy.append(dev_bf16(inp["dY"]))
    return x, codes, absmax, A, B, dy


# (T, d_in, d_outs, r, with u_saved, with dx)
CASES = [
    (300, 256, (256, 64, 64), 16, True, True),      # fused, q/k/v-like, RE = 48
    (260, 192, (128, 64), 24, False, True),         # fused, r = 24 (two projections), U recomputed
    (257, 320, (64, 64, 128, 64), 16, True, True),  # fused, four projections, RE = 64
    (140, 128, (64, 192), 8, True, True),           # fused, r = 8
    (150, 128, (72, 136), 16, True, True),          # d_out % 64 != 0: per projection
    (8, 192, (64, 64, 64), 16, True, True),         # few tokens: per projection (weight streaming)
    (150, 192, (64, 128), 40, True, True),          # fused, n r = 80 > 64: two epilogue passes, dA per projection
    (100, 256, (128, 64, 64), 16, True, True),      # up to 128 tokens: per projection (split-K dX)
    (260, 256, (128, 64, 64), 64, True, True),      # fused, rank 64 q/k/v-like: n r = 192
    # from 4096 tokens at rank > 16 (d_out % 256 == 0): G from a G pass, dX tiles without it
    (4100, 256, (256, 512, 256), 64, True, True),
    (4096, 320, (256, 256), 24, False, True),       # U recomputed, ragged d_in tile
    (4100, 256, (256, 256, 256), 48, True, False),  # no dX: the G pass alone feeds dA
    (200, 128, (64, 64, 64), 32, False, True),      # fused, n r = 96, U recomputed
    (300, 256, (256, 64, 64), 16, True, False),     # fused, dX not requested
    (1100, 320, (128, 64, 64), 16, True, True),     # fused, dX on the dequantized weights (128 tiles)
    (4100, 256, (128, 64, 64), 64, False, True),    # the same at rank 64, U recomputed
    (300, 256, (64,) * 8, 8, True, True),           # eight projections, n r = 64: nine rank-r jobs in one launch
    (260, 128, (64,) * 8, 16, True, True),          # eight projections, n r = 128: every dA, then every dB
]


@pytest.mark.parametrize("T,K,Ns,r,with_u,with_dx", CASES)
def test_bwd_multi_matches_oracle(q, T, K, Ns, r, with_u, with_dx):
    from tests.gpu_util import host_f64
    alpha = 16.0
    ins = [synth.custom_inputs(30 + g, T, K, N, r, dy_std=0.1) for g, N in enumerate(Ns)]
    for inp in ins[1:]:
        inp["x"] = ins[0]["x"]  # one shared input
    x, codes, absmax, A, B, dy = _dev_inputs(q, ins)
    us = q.lora_nf4_fwd_multi(x, codes, absmax, A, B, alpha)[1] if with_u else None
    dx, dAs, dBs = q.lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, alpha, u_saved=us, need_dx=with_dx)
    torch.cuda.synchronize()
    xr = _f64(ins[0]["x"])
    dx_ref = np.zeros_like(xr)
    for g, inp in enumerate(ins):
        c, a = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
        dX, dA, dB = olora.backward(xr, _f64(inp["dY"]), onf4.dequantize_exact(c, a), _f64(inp["A"]),
                                    _f64(inp["B"]), alpha, r)
        dx_ref += dX
        assert olora.rel_err(host_f64(dAs[g]), dA) <= TOL, ("dA", g)
        assert olora.rel_err(host_f64(dBs[g]), dB) <= TOL, ("dB", g)
    if with_dx:
        assert olora.rel_err(host_f64(dx), dx_ref) <= TOL
    else:
        assert dx is None


def test_bwd_multi_dx_dequantized_matches_in_loop(q):
    """With weight staging on, from 1024 tokens (128 x 128 tiles) the fused dX reads
    weights dequantized into the workspace; rows 0 .. 1022 match the in-loop path at
    1023 tokens bit for bit (rows are independent, the summation order is the same),
    and the default (in-loop at every token count) gives those bits too."""
    T, K, Ns, r = 1100, 320, (128, 64, 64), 16
    ins = [synth.custom_inputs(40 + g, T, K, N, r, dy_std=0.1) for g, N in enumerate(Ns)]
    x, codes, absmax, A, B, dy = _dev_inputs(q, ins)
    with q.weight_staging(True):
        dx, _, _ = q.lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, 16.0)
        dx1, _, _ = q.lora_nf4_bwd_multi(x[:1023].contiguous(), [d[:1023].contiguous() for d in dy], codes,
                                         absmax, A, B, 16.0)
        torch.cuda.synchronize()
    assert torch.equal(dx[:1023], dx1)
    dx0, _, _ = q.lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, 16.0)
    torch.cuda.synchronize()
    assert torch.equal(dx0, dx)


def test_bwd_multi_empty_batch(q):
    from tests.gpu_util import dev_bf16
    K, Ns, r = 128, (64, 64), 16
    ins = [synth.custom_inputs(50 + g, 4, K, N, r) for g, N in enumerate(Ns)]
    _, codes, absmax, A, B, _ = _dev_inputs(q, ins)
    x = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    dy = [torch.empty((0, N), dtype=torch.bfloat16, device="cuda") for N in Ns]
    dx, dAs, dBs = q.lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, 16.0)
    torch.cuda.synchronize()
    assert dx.shape == (0, K)
    for t in dAs + dBs:
        assert not t.float().abs().sum().item()


def test_bwd_multi_full_size_qwen_qkv(q):
    """Qwen-14B q, k, v (5120 -> 5120 each) at 8192 tokens, r = 16, as the fused path
    runs them: sampled dX rows and dA / dB columns against the oracle."""
    from tests.gpu_util import host_f64
    w = next(x for x in synth.WORKLOADS if x.name == "qwen14b-attn")
    ins = [synth.projection_inputs(w, pi) for pi in range(3)]
    for inp in ins[1:]:
        inp["x"] = ins[0]["x"]
    x, codes, absmax, A, B, dy = _dev_inputs(q, ins)
    us = q.lora_nf4_fwd_multi(x, codes, absmax, A, B, w.alpha)[1]
    dx, dAs, dBs = q.lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, w.alpha, u_saved=us)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    T, K = ins[0]["x"].shape
    rows = np.sort(rng.choice(T, 6, replace=False))
    cols = np.sort(rng.choice(K, 6, replace=False))
    xr = _f64(ins[0]["x"])
    s = w.alpha / w.r
    dx_ref = np.zeros((rows.size, K))
    for g, inp in enumerate(ins):
        c, a = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
        D = onf4.dequantize_exact(c, a)
        Ag, Bg, dYg = _f64(inp["A"]), _f64(inp["B"]), _f64(inp["dY"])
        G = s * (dYg @ Bg.T)                      # [T, r]
        dx_ref += dYg[rows] @ D + G[rows] @ Ag.T
        dA_ref = xr[:, cols].T @ G                # dA rows k = cols
        U = xr @ Ag
        ncols = np.sort(rng.choice(dYg.shape[1], 6, replace=False))
        dB_ref = s * (U.T @ dYg[:, ncols])
        got_dA = host_f64(dAs[g])[cols]
        got_dB = host_f64(dBs[g])[:, ncols]
        assert olora.rel_err(got_dA, dA_ref) <= TOL, ("dA", g)
        assert olora.rel_err(got_dB, dB_ref) <= TOL, ("dB", g)
    got = host_f64(dx)[rows]
    assert olora.rel_err(got, dx_ref) <= TOL


def test_bwd_multi_full_size_70b_gate_up(q):
    """Llama-3-70B gate and up (8192 -> 28672 each) at 4096 tokens, r = 16, sharing
    x as the fused path runs them (the benchmark's --fuse grouping): sampled dX rows
    (the sum over both projections) and sampled dA / dB columns against the oracle."""
    from tests.gpu_util import host_f64
    w = next(x for x in synth.WORKLOADS if x.name == "llama3-70b-layer")
    names = [p.name for p in w.projections]
    pis = [names.index("gate_proj"), names.index("up_proj")]
    ins = [synth.projection_inputs(w, pi) for pi in pis]
    ins[1]["x"] = ins[0]["x"]
    x, codes, absmax, A, B, dy = _dev_inputs(q, ins)
    us = q.lora_nf4_fwd_multi(x, codes, absmax, A, B, w.alpha)[1]
    dx, dAs, dBs = q.lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, w.alpha, u_saved=us)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    T, K = ins[0]["x"].shape
    rows = np.sort(rng.choice(T, 6, replace=False))
    cols = np.sort(rng.choice(K, 6, replace=False))
    xr = _f64(ins[0]["x"])
    s = w.alpha / w.r
    dx_ref = np.zeros((rows.size, K))
    for g, inp in enumerate(ins):
        c, a = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
        D = onf4.dequantize_exact(c, a)
        Ag, Bg, dYg = _f64(inp["A"]), _f64(inp["B"]), _f64(inp["dY"])
        G = s * (dYg @ Bg.T)
        dx_ref += dYg[rows] @ D + G[rows] @ Ag.T
        del D
        dA_ref = xr[:, cols].T @ G
        U = xr @ Ag
        ncols = np.sort(rng.choice(dYg.shape[1], 6, replace=False))
        dB_ref = s * (U.T @ dYg[:, ncols])
        assert olora.rel_err(host_f64(dAs[g])[cols], dA_ref) <= TOL, ("dA", g)
        assert olora.rel_err(host_f64(dBs[g])[:, ncols], dB_ref) <= TOL, ("dB", g)
    assert olora.rel_err(host_f64(dx)[rows], dx_ref) <= TOL
