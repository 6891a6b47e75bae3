"""Fused NF4-LoRA forward and backward on the GPU against the fp64 oracle.

Bar: max|gpu - ref| / max|ref| <= 1e-2 for y, dX, dA, dB (bf16 outputs, fp32
accumulation); U saved by the forward to the same bar. Small shapes compare
every element; full workload sizes compare sampled rows of y and dX and the
full dA and dB.
"""
import ctypes

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


def _run_gpu(q, inp, alpha, u_saved=True, need_dx=True):
    from tests.gpu_util import dev_bf16
    x, W, A, B, dY = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
    codes, absmax = q.nf4_quantize(W)
    y, u = q.lora_nf4_fwd(x, codes, absmax, A, B, alpha, save_u=True)
    dx, dA, dB = q.lora_nf4_bwd(x, dY, codes, absmax, A, B, alpha,
                                u_saved=u if u_saved else None, need_dx=need_dx)
    torch.cuda.synchronize()
    return y, u, dx, dA, dB


def _oracle_D(inp):
    codes, absmax = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
    return onf4.dequantize_exact(codes, absmax)


def _check_full(q, inp, alpha, r, label):
    from tests.gpu_util import host_f64
    y, u, dx, dA, dB = _run_gpu(q, inp, alpha)
    x, A, B, dY = (_f64(inp[k]) for k in ("x", "A", "B", "dY"))
    D = _oracle_D(inp)
    y_ref, U_ref = olora.forward(x, D, A, B, alpha, r)
    dX_ref, dA_ref, dB_ref = olora.backward(x, dY, D, A, B, alpha, r)
    errs = {
        "y": olora.rel_err(host_f64(y), y_ref),
        "u": olora.rel_err(host_f64(u), U_ref),
        "dx": olora.rel_err(host_f64(dx), dX_ref),
        "dA": olora.rel_err(host_f64(dA), dA_ref),
        "dB": olora.rel_err(host_f64(dB), dB_ref),
    }
    print(label, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (label, k, v)
    return errs


def test_tiny_workload(q):
    w = synth.WORKLOADS[0]
    inp = synth.projection_inputs(w, 0)
    _check_full(q, inp, w.alpha, w.r, "tiny")


# (T, d_in, d_out, r): ragged token counts, partial tiles in every dimension,
# ranks from 1 to the maximum (256), d_out from 1; the last four split the reduction of the tiled
# kernels across workgroups: the forward's over d_in (few tiles, d_in >= 1024),
# then dX's over d_out (few tiles, d_out >= 2048).
ODD = [(1, 64, 64, 1), (63, 128, 192, 8), (65, 192, 64, 16), (200, 320, 136, 64),
       (130, 256, 8, 128), (257, 64, 520, 24), (129, 384, 264, 17), (17, 640, 1000, 40),
       (260, 192, 296, 48), (300, 2048, 200, 16), (200, 1536, 136, 64), (300, 256, 2048, 16),
       (200, 192, 2056, 64),
       # d_out not a multiple of 8 (generic kernels, unaligned rows of dY, y and B) and
       # ranks above 128 (rank tiles of 12 and 16, epilogues in passes of 64 columns)
       (40, 128, 13, 16), (300, 192, 7, 24), (5, 64, 1, 8), (129, 320, 1001, 64), (70, 256, 200, 256),
       (130, 128, 64, 200), (1, 64, 13, 256), (260, 192, 136, 160)]


@pytest.mark.parametrize("T,K,N,r", ODD)
def test_odd_shapes(q, T, K, N, r):
    inp = synth.custom_inputs(1, T, K, N, r)
    _check_full(q, inp, 16.0, r, f"odd T={T} K={K} N={N} r={r}")


# Few tokens (r % 8 == 0, r <= 64): the one-launch weight-streaming forward (T <=
# 32, d_out <= 4096), the split-K weight-streaming forward (T <= 128 otherwise),
# and the split-K weight-streaming dX (T <= 128). Cases cover a single half-filled
# reduction step (d_in = 64), a half-filled last step (d_in % 128 == 64), d_out
# not a multiple of the 16- or 64-row block, one, two, four and eight 16-token
# blocks, one and many d_in splits, every rank block count, and wide d_out (up to
# 32776) at few tokens. The wide-d_out cases up to 32 tokens run the dX that reads
# each column's codes with the 4-bit transposing LDS read (slices of eight or more
# steps), the last two with a last 128-column block half past d_in.
FEW = [(1, 64, 16, 8), (1, 4096, 64, 16), (5, 192, 40, 16), (9, 64, 8, 56), (16, 256, 48, 24),
       (17, 320, 136, 64), (32, 448, 1000, 32), (32, 128, 8, 8), (16, 4096, 4096, 16),
       (32, 4096, 1024, 64), (48, 192, 72, 24), (64, 4096, 4096, 16), (100, 320, 200, 64),
       (128, 448, 1000, 32), (127, 2048, 136, 8), (1, 320, 4104, 16), (8, 192, 5000, 64),
       (32, 2048, 4160, 40), (3, 1024, 28672, 16), (16, 1024, 32776, 8), (20, 1024, 20488, 32),
       (12, 1024, 16392, 64), (7, 3072, 12296, 48), (1, 2048, 9000, 24), (25, 3072, 520, 16),
       (5, 320, 16392, 16), (9, 192, 12352, 64)]


@pytest.mark.parametrize("T,K,N,r", FEW)
def test_few_token_shapes(q, T, K, N, r):
    inp = synth.custom_inputs(5, T, K, N, r)
    _check_full(q, inp, 16.0, r, f"few T={T} K={K} N={N} r={r}")


@pytest.mark.parametrize("r", [16, 64])
def test_forward_tile_edges_agree(q, r):
    """The forward runs 256 x 256 tiles when they fill the GPU and 128 x 128 tiles
    otherwise; both accumulate every output in the same order. d_out = 32808 at 300
    tokens gives 2 x 129 = 258 tiles of 256 (256 path, ragged in both dimensions);
    the first 1000 columns alone give 8 (128 path). Same bits, and the oracle."""
    from tests.gpu_util import dev_bf16, host_f64
    T, K, N, Nsub = 300, 256, 32808, 1000
    inp = synth.custom_inputs(11, T, K, N, r)
    x, W, A, B = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B"))
    codes, absmax = q.nf4_quantize(W)
    y, u = q.lora_nf4_fwd(x, codes, absmax, A, B, 16.0)
    ys, us = q.lora_nf4_fwd(x, codes[:Nsub].contiguous(), absmax[:Nsub].contiguous(), A,
                            B[:, :Nsub].contiguous(), 16.0)
    torch.cuda.synchronize()
    assert torch.equal(ys, y[:, :Nsub]) and torch.equal(us, u)
    cols = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
    Wc = synth.bf16_bits_to_f32(inp["W"])[cols]
    c, a = onf4.quantize(Wc)
    y_ref, u_ref = olora.forward(_f64(inp["x"]), onf4.dequantize_exact(c, a), _f64(inp["A"]),
                                 _f64(inp["B"])[:, cols], 16.0, r)
    assert olora.rel_err(host_f64(y)[:, cols], y_ref) <= TOL
    assert olora.rel_err(host_f64(u), u_ref) <= TOL


# With weight staging on, from 1024 tokens the forward dequantizes the weight once
# into its workspace and runs the tiles on bf16; the values are those of the
# in-loop dequantization. Ragged T, d_in and d_out (odd step counts), every rank
# block.
DQ = [(1100, 320, 200, 16), (1030, 448, 520, 64), (2080, 192, 264, 24), (1040, 256, 136, 40)]


@pytest.mark.parametrize("T,K,N,r", DQ)
def test_forward_dequantized_matches_in_loop(q, T, K, N, r):
    """Rows 0 .. 1022 through the dequantize-then-GEMM path (T >= 1024) and
    through the in-loop dequantization (T = 1023): each output row depends on its
    own input row only, in the same order, so the bits agree; and the oracle."""
    from tests.gpu_util import dev_bf16, host_f64
    inp = synth.custom_inputs(12, T, K, N, r)
    x, W, A, B = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B"))
    codes, absmax = q.nf4_quantize(W)
    with q.weight_staging(True):
        assert q.lora_nf4_fwd_workspace_bytes(T, K, N, r) >= K * N * 2
        assert q.lora_nf4_fwd_workspace_bytes(1023, K, N, r) == 0
        y, u = q.lora_nf4_fwd(x, codes, absmax, A, B, 16.0)
        y1, u1 = q.lora_nf4_fwd(x[:1023].contiguous(), codes, absmax, A, B, 16.0)
        torch.cuda.synchronize()
    y0, u0 = q.lora_nf4_fwd(x, codes, absmax, A, B, 16.0)  # default: in-loop at every T
    torch.cuda.synchronize()
    assert torch.equal(y0[:1023], y1) and torch.equal(u0[:1023], u1)
    assert torch.equal(y[:1023], y1) and torch.equal(u[:1023], u1)
    y_ref, u_ref = olora.forward(_f64(inp["x"]), _oracle_D(inp), _f64(inp["A"]), _f64(inp["B"]), 16.0, r)
    assert olora.rel_err(host_f64(y), y_ref) <= TOL
    assert olora.rel_err(host_f64(u), u_ref) <= TOL


# With weight staging on, from 4096 tokens at rank > 16 the dequantize-then-GEMM
# forward takes U = x A
# from a separate pass (d_in split over four waves, fixed-order sum; the tile
# kernel reads bf16(s U) in its epilogue): ranks 24 (half the 32-wide block), 40
# and 64, ragged T, d_in and d_out; the full oracle on every output.
UPASS = [(4100, 320, 200, 64), (4130, 192, 136, 24), (4096, 448, 72, 40)]


@pytest.mark.parametrize("T,K,N,r", UPASS)
def test_forward_u_pass(q, T, K, N, r):
    inp = synth.custom_inputs(15, T, K, N, r)
    with q.weight_staging(True):
        assert q.lora_nf4_fwd_workspace_bytes(T, K, N, r) >= K * N * 2 + T * r * 2
        _check_full(q, inp, 16.0, r, f"u-pass T={T} K={K} N={N} r={r}")


# From 4096 tokens, where the grid takes 256 x 256 tiles and d_in % 256 == 0, the
# forward runs the register-dequantizing kernel (packed codes straight into MFMA
# fragments, x through a four-stage LDS ring, U from the U pass): ragged T and
# d_out (partial tiles in both directions), ranks 8 .. 64, one to four groups of
# four K-steps; the full oracle on every output, and bitwise determinism.
RW = [(4100, 512, 2056, 16), (4350, 768, 2104, 24), (4096, 1024, 4104, 64), (8192, 256, 1032, 8)]


@pytest.mark.parametrize("T,K,N,r", RW)
def test_forward_register_dequant(q, T, K, N, r):
    inp = synth.custom_inputs(16, T, K, N, r)
    assert q.lora_nf4_fwd_workspace_bytes(T, K, N, r) < K * N * 2  # no dequantized weight
    _check_full(q, inp, 16.0, r, f"rw T={T} K={K} N={N} r={r}")
    r1 = _run_gpu(q, inp, 16.0)
    r2 = _run_gpu(q, inp, 16.0)
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


# From 4096 tokens at rank 16, d_in and d_out multiples of 256, dX runs on
# register-dequantized 256 x 256 tiles: the packed weight transposed once into the
# workspace (codes^T, absmax^T), its codes straight into MFMA fragments, G = s dY
# B^T in the same loop. Ragged T, one to three column tiles, one to four groups of
# four d_out steps; the full oracle on every output, bitwise determinism, and the
# dX-less call (G only) giving the same dA and dB bits.
RWX = [(4100, 512, 256, 16), (4350, 768, 1024, 16), (8192, 256, 512, 16)]


@pytest.mark.parametrize("T,K,N,r", RWX)
def test_dx_register_dequant(q, T, K, N, r):
    inp = synth.custom_inputs(17, T, K, N, r, dy_std=0.1)
    _check_full(q, inp, 16.0, r, f"rwx T={T} K={K} N={N} r={r}")
    r1 = _run_gpu(q, inp, 16.0)
    r2 = _run_gpu(q, inp, 16.0)
    assert all(torch.equal(a, b) for a, b in zip(r1[2:], r2[2:]))
    _, _, dx3, dA3, dB3 = _run_gpu(q, inp, 16.0, need_dx=False)
    assert dx3 is None and torch.equal(dA3, r1[3]) and torch.equal(dB3, r1[4])


# From 4096 tokens at rank > 16 with d_out a multiple of 256 (and dX not split over
# d_out), G = s dY B^T comes from a pass of its own over dY and the dX tiles run
# without G in their K loop, reading it back in the epilogue: ranks 24, 40 and 64,
# ragged T and d_in; the full oracle on every output, and the dX-less call (the G
# pass alone) giving the same dA and dB bits.
GPASS = [(4100, 320, 512, 24), (4096, 768, 256, 64), (8200, 256, 1024, 40)]


@pytest.mark.parametrize("T,K,N,r", GPASS)
def test_dx_with_g_pass(q, T, K, N, r):
    inp = synth.custom_inputs(18, T, K, N, r, dy_std=0.1)
    _check_full(q, inp, 16.0, r, f"gpass T={T} K={K} N={N} r={r}")
    r1 = _run_gpu(q, inp, 16.0)
    _, _, dx3, dA3, dB3 = _run_gpu(q, inp, 16.0, need_dx=False)
    assert dx3 is None and torch.equal(dA3, r1[3]) and torch.equal(dB3, r1[4])


# With weight staging on, from 4096 tokens on 256 x 256 dX tiles (1024 on 128 x 128
# tiles) the dX kernel runs on the weight dequantized once into the workspace; by
# default the same shapes run the in-loop kernels (or, at rank 16 on whole tiles,
# the register path above). Large token counts,
# ragged T and d_in, one to eight d_out steps, ranks 8 and 16; the full oracle on
# every output.
DQ_BWD = [(8200, 320, 192, 16), (8230, 192, 128, 8), (9000, 128, 64, 16), (8300, 448, 512, 16)]


@pytest.mark.parametrize("T,K,N,r", DQ_BWD)
@pytest.mark.parametrize("staged", [True, False])
def test_backward_dequantized(q, T, K, N, r, staged):
    inp = synth.custom_inputs(13, T, K, N, r)
    with q.weight_staging(staged):
        _check_full(q, inp, 16.0, r, f"{'dq' if staged else 'in-loop'}-bwd T={T} K={K} N={N} r={r}")


# The same path against the in-loop dequantization: rows of dX are independent,
# so rows 0 .. T_in - 1 match, bit for bit, a call at T_in tokens, just under the
# threshold on the same tile edge. Ragged d_in and d_out, ranks 16 .. 64; the
# full oracle on every output.
DQX = [(1100, 4160, 200, 24, 1023), (4100, 4096, 192, 64, 4095), (4096, 4160, 136, 16, 4095)]


@pytest.mark.parametrize("T,K,N,r,T_in", DQX)
def test_dx_dequantized_matches_in_loop(q, T, K, N, r, T_in):
    from tests.gpu_util import dev_bf16
    inp = synth.custom_inputs(14, T, K, N, r, dy_std=0.1)
    x, W, A, B, dY = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
    codes, absmax = q.nf4_quantize(W)
    with q.weight_staging(True):
        dx, _, _ = q.lora_nf4_bwd(x, dY, codes, absmax, A, B, 16.0)
        dx1, _, _ = q.lora_nf4_bwd(x[:T_in].contiguous(), dY[:T_in].contiguous(), codes, absmax, A, B, 16.0)
        torch.cuda.synchronize()
        assert torch.equal(dx[:T_in], dx1)
        _check_full(q, inp, 16.0, r, f"dqx T={T} K={K} N={N} r={r}")


@pytest.mark.parametrize("r", [16, 64])
def test_dx_tile_edges_agree(q, r):
    """The input gradient's tile edge follows the same round count: 500 tokens x
    d_in 32704 is 2 x 128 tiles of 256 (one round; 256 path, ragged tokens), its
    first 1024 columns alone 4 x 8 tiles of 128. dX columns depend only on their
    own weight columns and rows of A: same bits, and the oracle on sampled columns."""
    from tests.gpu_util import dev_bf16, host_f64
    T, K, N, Ksub, alpha = 500, 32704, 64, 1024, 16.0
    inp = synth.custom_inputs(12, T, K, N, r, dy_std=0.1)
    x, W, A, B, dY = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
    codes, absmax = q.nf4_quantize(W)
    dx, _, _ = q.lora_nf4_bwd(x, dY, codes, absmax, A, B, alpha)
    dxs, _, _ = q.lora_nf4_bwd(x[:, :Ksub].contiguous(), dY, codes[:, :Ksub // 2].contiguous(),
                               absmax[:, :Ksub // 64].contiguous(), A[:Ksub].contiguous(), B, alpha)
    torch.cuda.synchronize()
    assert torch.equal(dxs, dx[:, :Ksub])
    cols = np.unique(np.concatenate([np.arange(0, K, 211), [K - 1]]))
    c, a = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))
    D = onf4.dequantize_exact(c, a)
    dYr, Ar, Br = _f64(inp["dY"]), _f64(inp["A"]), _f64(inp["B"])
    G = (alpha / r) * (dYr @ Br.T)
    dx_ref = dYr @ D[:, cols] + G @ Ar[cols].T
    assert olora.rel_err(host_f64(dx)[:, cols], dx_ref) <= TOL


@pytest.mark.parametrize("T,K,N,r", [(300, 256, 192, 16), (7, 320, 200, 24), (8200, 256, 192, 16),
                                     (48, 4096, 1024, 16), (4100, 512, 256, 64), (4352, 512, 512, 16)])
def test_recompute_u_and_skip_dx_paths(q, T, K, N, r):
    """The backward with u_saved = NULL recomputes U = x A itself; its dX, dA and dB
    are checked against the oracle directly (tiled, few-token, split-K and
    large-token shapes), and the dX-less call gives the same dA and dB bits."""
    from tests.gpu_util import host_f64
    alpha = 32.0
    inp = synth.custom_inputs(2, T, K, N, r)
    y, u, dx, dA, dB = _run_gpu(q, inp, alpha, u_saved=True)
    _, _, dx2, dA2, dB2 = _run_gpu(q, inp, alpha, u_saved=False)
    _, _, dx3, dA3, dB3 = _run_gpu(q, inp, alpha, u_saved=True, need_dx=False)
    assert dx3 is None
    x, A, B, dY = (_f64(inp[k]) for k in ("x", "A", "B", "dY"))
    dX_ref, dA_ref, dB_ref = olora.backward(x, dY, _oracle_D(inp), A, B, alpha, r)
    errs = {"dx": olora.rel_err(host_f64(dx2), dX_ref), "dA": olora.rel_err(host_f64(dA2), dA_ref),
            "dB": olora.rel_err(host_f64(dB2), dB_ref)}
    print(f"recompute-U T={T} K={K} N={N} r={r}", {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    assert torch.equal(dA3, dA) and torch.equal(dB3, dB)


@pytest.mark.parametrize("T", [1000, 100, 16])
def test_bitwise_deterministic(q, T):
    inp = synth.custom_inputs(3, T, 512, 384, 16)
    r1 = _run_gpu(q, inp, 16.0)
    r2 = _run_gpu(q, inp, 16.0)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_empty_batch(q):
    """T = 0: the forward is a no-op and the backward's dA, dB are zero (empty sums)."""
    from tests.gpu_util import dev_bf16
    inp = synth.custom_inputs(9, 4, 256, 64, 16)
    codes, absmax = q.nf4_quantize(dev_bf16(inp["W"]))
    A, B = dev_bf16(inp["A"]), dev_bf16(inp["B"])
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    dy = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    y, u = q.lora_nf4_fwd(x, codes, absmax, A, B, 16.0)
    assert y.shape == (0, 64) and u.shape == (0, 16)
    dx, dA, dB = q.lora_nf4_bwd(x, dy, codes, absmax, A, B, 16.0)
    torch.cuda.synchronize()
    assert dx.shape == (0, 256)
    assert not dA.any() and not dB.any()


def test_operand_beyond_two_gib(q):
    """x and dX of 2 GiB each (past the buffer-descriptor range: the generic
    kernels) on sampled rows and sampled dA / dB entries against the oracle."""
    from tests.gpu_util import dev_bf16, host_f64
    T, K, N, r, alpha = 262144, 4096, 64, 8, 16.0
    g = torch.Generator(device="cuda").manual_seed(123)
    x = torch.randn((T, K), generator=g, device="cuda").to(torch.bfloat16)
    dy = (torch.randn((T, N), generator=g, device="cuda") * 0.01).to(torch.bfloat16)
    small = synth.custom_inputs(12, 1, K, N, r)
    codes, absmax = q.nf4_quantize(dev_bf16(small["W"]))
    A, B = dev_bf16(small["A"]), dev_bf16(small["B"])
    assert x.numel() * 2 >= 2 ** 31
    y, u = q.lora_nf4_fwd(x, codes, absmax, A, B, alpha)
    dx, dA, dB = q.lora_nf4_bwd(x, dy, codes, absmax, A, B, alpha, u_saved=u)
    torch.cuda.synchronize()
    D = _oracle_D(small)
    Af, Bf = _f64(small["A"]), _f64(small["B"])
    s = alpha / r
    rows = torch.tensor([0, 1, 777, 65536, 131071, 200000, T - 2, T - 1], device="cuda")
    xr, dyr = host_f64(x[rows]), host_f64(dy[rows])
    y_ref, u_ref = olora.forward(xr, D, Af, Bf, alpha, r)
    dx_ref, _, _ = olora.backward(xr, dyr, D, Af, Bf, alpha, r)
    assert olora.rel_err(host_f64(y[rows]), y_ref) <= TOL
    assert olora.rel_err(host_f64(u[rows]), u_ref) <= TOL
    assert olora.rel_err(host_f64(dx[rows]), dx_ref) <= TOL
    # dA[k, j] = sum_t x[t, k] G[t, j] and dB[j, n] = s sum_t U[t, j] dY[t, n] over
    # all T: exact G from dY; U from the forward's saved U (checked on rows above)
    G = s * (host_f64(dy) @ Bf.T)
    ks = [0, 1, 1234, K - 1]
    xk = host_f64(x[:, ks])
    dA_ref = xk.T @ G
    assert olora.rel_err(host_f64(dA[ks]), dA_ref) <= TOL
    dB_ref = s * (host_f64(u).T @ host_f64(dy))
    assert olora.rel_err(host_f64(dB), dB_ref) <= TOL


@pytest.mark.parametrize("T,K,N,r", [(131, 192, 200, 12), (7, 320, 72, 24), (100, 448, 200, 16),
                                     (260, 1024, 136, 16), (1040, 320, 200, 16), (8200, 320, 192, 16)])
def test_guard_bands_untouched(q, T, K, N, r):
    """Outputs written through the C ABI stay inside their buffers."""
    from tests.gpu_util import Guarded, dev_bf16
    inp = synth.custom_inputs(4, T, K, N, r)
    x, W, A, B, dY = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
    codes, absmax = q.nf4_quantize(W)
    gy, gu, gdx, gda, gdb = Guarded(T * N * 2), Guarded(T * r * 2), Guarded(T * K * 2), \
        Guarded(K * r * 2), Guarded(r * N * 2)
    lib = q.library()
    stream = torch.cuda.current_stream().cuda_stream
    fbytes = lib.lora_nf4_fwd_workspace_bytes(T, K, N, r)
    gws = Guarded(fbytes) if fbytes else None
    st = lib.lora_nf4_fwd(T, K, N, r, 16.0, x.data_ptr(), codes.data_ptr(), absmax.data_ptr(),
                          A.data_ptr(), B.data_ptr(), gy.ptr, gu.ptr, gws.ptr if gws else None,
                          ctypes.c_size_t(fbytes), stream)
    assert st == 0
    nbytes = lib.lora_nf4_bwd_workspace_bytes(T, K, N, r)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = lib.lora_nf4_bwd(T, K, N, r, 16.0, x.data_ptr(), dY.data_ptr(), codes.data_ptr(),
                          absmax.data_ptr(), A.data_ptr(), B.data_ptr(), gu.ptr, gdx.ptr, gda.ptr,
                          gdb.ptr, ws.data_ptr(), ctypes.c_size_t(nbytes), stream)
    assert st == 0
    torch.cuda.synchronize()
    for g in (gy, gu, gdx, gda, gdb) + ((gws,) if gws else ()):
        assert g.canaries_intact()
    y_ref, _ = olora.forward(_f64(inp["x"]), _oracle_D(inp), _f64(inp["A"]), _f64(inp["B"]), 16.0, r)
    from tests.gpu_util import host_f64
    assert olora.rel_err(host_f64(gy.view(torch.bfloat16, (T, N))), y_ref) <= TOL


def _sample_rows(T, n=48, seed=0):
    g = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, T - 1], g.choice(T, size=n, replace=False)]))
    return rows


# every distinct projection shape of the five workloads: 8B q (4096 -> 4096, r = 16),
# 8B k/o at r = 64, Qwen-14B (5120 -> 5120), and the 70B q (8192 -> 8192), k, gate
# (8192 -> 28672) and down (28672 -> 8192) projections at 4096 tokens
FULL = [(1, 0), (2, 1), (2, 3), (3, 0), (4, 0), (4, 1), (4, 4), (4, 6)]


@pytest.mark.parametrize("T", [1, 16, 32])
def test_full_size_few_tokens_70b_gate(q, T):
    """Llama-3-70B gate (8192 -> 28672, r = 16) at 1, 16 and 32 tokens (the
    workload's draws at that token count): the few-token forward and dX in the
    launch configuration the benchmark's small-token leg times, every output
    against the oracle."""
    from tests.gpu_util import host_f64
    w = synth.WORKLOADS[4]
    inp = synth.projection_inputs(w, 4, tokens=T)
    y, u, dx, dA, dB = _run_gpu(q, inp, w.alpha)
    x, A, B, dY = (_f64(inp[k]) for k in ("x", "A", "B", "dY"))
    D = _oracle_D(inp)
    y_ref, U_ref = olora.forward(x, D, A, B, w.alpha, w.r)
    dX_ref, dA_ref, dB_ref = olora.backward(x, dY, D, A, B, w.alpha, w.r)
    errs = {"y": olora.rel_err(host_f64(y), y_ref), "u": olora.rel_err(host_f64(u), U_ref),
            "dx": olora.rel_err(host_f64(dx), dX_ref), "dA": olora.rel_err(host_f64(dA), dA_ref),
            "dB": olora.rel_err(host_f64(dB), dB_ref)}
    print("70b gate", T, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (T, k, v)


@pytest.mark.parametrize("wi,pi", FULL)
def test_full_size_sampled(q, wi, pi):
    """Full workload sizes, in the launch configuration the benchmark times."""
    from tests.gpu_util import host_f64
    w = synth.WORKLOADS[wi]
    p = w.projections[pi]
    inp = synth.projection_inputs(w, pi)
    y, u, dx, dA, dB = _run_gpu(q, inp, w.alpha)
    rows = _sample_rows(w.tokens)
    x, A, B, dY = (_f64(inp[k]) for k in ("x", "A", "B", "dY"))
    D = _oracle_D(inp)
    y_ref, U_ref = olora.forward(x[rows], D, A, B, w.alpha, w.r)
    dX_ref, _, _ = olora.backward(x[rows], dY[rows], D, A, B, w.alpha, w.r)
    dA_ref, dB_ref = olora.lora_factor_grads(x, dY, A, B, w.alpha, w.r)
    rows_t = torch.from_numpy(rows).cuda()
    errs = {
        "y": olora.rel_err(host_f64(y[rows_t]), y_ref),
        "u": olora.rel_err(host_f64(u[rows_t]), U_ref),
        "dx": olora.rel_err(host_f64(dx[rows_t]), dX_ref),
        "dA": olora.rel_err(host_f64(dA), dA_ref),
        "dB": olora.rel_err(host_f64(dB), dB_ref),
    }
    print(w.name, p.name, {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v <= TOL, (w.name, p.name, k, v)


# Multi-projection forward: the same values as one lora_nf4_fwd per projection
# (bitwise: each output tile runs the same kernel code on the same data), on the
# tiled path (one launch; from 1024 tokens with every weight dequantized into the
# workspace), the few-token paths and the K-split tiled forward (one workspace
# shared by the projections in turn) and the generic path.
MULTI = [(300, 256, (256, 64, 64), 16), (200, 320, (200, 40, 8), 24), (8, 192, (64, 16, 16), 16),
         (150, 128, (72, 136), 12), (100, 256, (128, 64, 64), 16), (300, 2048, (256, 64, 64), 16),
         (1100, 320, (200, 72, 136), 16)]


@pytest.mark.parametrize("T,K,Ns,r", MULTI)
def test_fwd_multi_matches_single(q, T, K, Ns, r):
    from tests.gpu_util import dev_bf16, host_f64
    ins = [synth.custom_inputs(6 + g, T, K, N, r) for g, N in enumerate(Ns)]
    x = dev_bf16(ins[0]["x"])
    codes, absmax, A, B = [], [], [], []
    for inp in ins:
        c, a = q.nf4_quantize(dev_bf16(inp["W"]))
        codes.append(c), absmax.append(a), A.append(dev_bf16(inp["A"])), B.append(dev_bf16(inp["B"]))
    ys, us = q.lora_nf4_fwd_multi(x, codes, absmax, A, B, 16.0)
    for g in range(len(Ns)):
        y1, u1 = q.lora_nf4_fwd(x, codes[g], absmax[g], A[g], B[g], 16.0)
        torch.cuda.synchronize()
        assert torch.equal(ys[g], y1) and torch.equal(us[g], u1), (T, K, Ns, r, g)
    # and against the oracle for the first projection
    D = _oracle_D(ins[0])
    y_ref, u_ref = olora.forward(_f64(ins[0]["x"]), D, _f64(ins[0]["A"]), _f64(ins[0]["B"]), 16.0, r)
    assert olora.rel_err(host_f64(ys[0]), y_ref) <= TOL
    assert olora.rel_err(host_f64(us[0]), u_ref) <= TOL


def test_fwd_multi_full_size_qkv(q):
    """Llama-3-8B q, k, v (4096 -> 4096, 1024, 1024) at 8192 tokens, r = 64, one shared x."""
    from tests.gpu_util import dev_bf16
    w = next(x for x in synth.WORKLOADS if x.name == "llama3-8b-attn-r64")
    ins = [synth.projection_inputs(w, pi) for pi in range(3)]
    x = dev_bf16(ins[0]["x"])
    codes, absmax, A, B = [], [], [], []
    for inp in ins:
        c, a = q.nf4_quantize(dev_bf16(inp["W"]))
        codes.append(c), absmax.append(a), A.append(dev_bf16(inp["A"])), B.append(dev_bf16(inp["B"]))
    ys, us = q.lora_nf4_fwd_multi(x, codes, absmax, A, B, w.alpha)
    # the shared launch runs 256 x 256 register-dequantizing tiles over all three
    # projections; a separate k or v call (1024 columns) runs 128 x 128 tiles, whose
    # summation order differs: equal U (the same U pass), y within the tolerance of
    # each other, and sampled rows against the oracle
    rows = _sample_rows(w.tokens, n=6, seed=3)
    rows_t = torch.from_numpy(rows).cuda()
    from tests.gpu_util import host_f64
    for g in range(3):
        y1, u1 = q.lora_nf4_fwd(x, codes[g], absmax[g], A[g], B[g], w.alpha)
        torch.cuda.synchronize()
        assert torch.equal(us[g], u1), g
        assert olora.rel_err(host_f64(ys[g]), host_f64(y1)) <= TOL, g
        y_ref, _ = olora.forward(_f64(ins[0]["x"][rows]), _oracle_D(ins[g]), _f64(ins[g]["A"]), _f64(ins[g]["B"]),
                                 w.alpha, w.r)
        assert olora.rel_err(host_f64(ys[g][rows_t]), y_ref) <= TOL, g
