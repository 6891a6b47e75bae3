"""lora_nf4_bwd_noalloc (the backward whose workspace is the library's own device
scratch) against lora_nf4_bwd with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, then a shape whose dequantized-
weight plan exceeds the scratch (the no-dequantized-weight plan runs instead).
Both plans give the same bits, so every output must match exactly."""
import ctypes

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import qlora_linear_amd as q
    q.library()
    return q


def _inputs(q, seed, T, K, N, r):
    from tests.gpu_util import dev_bf16
    inp = synth.custom_inputs(seed, T, K, N, r, dy_std=0.01)
    x, W, A, B, dY = (dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
    codes, absmax = q.nf4_quantize(W)
    return x, dY, codes, absmax, A, B


def _noalloc(q, x, dy, codes, absmax, A, B, alpha, u):
    T, K = x.shape
    N, r = B.shape[1], A.shape[1]
    dx = torch.full((T, K), 7.0, dtype=torch.bfloat16, device="cuda")
    dA = torch.full((K, r), 7.0, dtype=torch.bfloat16, device="cuda")
    dB = torch.full((r, N), 7.0, dtype=torch.bfloat16, device="cuda")
    st = q.library().lora_nf4_bwd_noalloc(
        T, K, N, r, alpha, x.data_ptr(), dy.data_ptr(), codes.data_ptr(), absmax.data_ptr(), A.data_ptr(),
        B.data_ptr(), None if u is None else u.data_ptr(), dx.data_ptr(), dA.data_ptr(), dB.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, q.status_string(st)
    return dx, dA, dB


# (T, d_in, d_out, r, with saved U): q_proj at 8192 tokens (its workspace, with the
# dequantized weight, fits the scratch), then a smaller ragged call, then 4096 x
# (4096 -> 14336), whose dequantized weight (112 MiB) does not fit
CALLS = [(8192, 4096, 4096, 16, True), (300, 256, 192, 16, False), (4096, 4096, 14336, 16, True)]


def test_noalloc_matches_workspace_entry_point(q):
    lib = q.library()
    for i, (T, K, N, r, with_u) in enumerate(CALLS):
        print(f"noalloc call {i}: T={T} K={K} N={N} r={r} u={with_u}", flush=True)
        x, dy, codes, absmax, A, B = _inputs(q, 60 + i, T, K, N, r)
        u = q.lora_nf4_fwd(x, codes, absmax, A, B, 16.0)[1] if with_u else None
        ref = q.lora_nf4_bwd(x, dy, codes, absmax, A, B, 16.0, u_saved=u)
        got = _noalloc(q, x, dy, codes, absmax, A, B, 16.0, u)
        torch.cuda.synchronize()
        for name, a, b in zip(("dx", "dA", "dB"), got, ref):
            assert torch.equal(a, b), (i, name)
    # past the scratch: rejected before any launch
    ws = lib.lora_nf4_bwd_workspace_bytes(1 << 20, 8192, 28672, 256)
    assert ws > (64 << 20)
