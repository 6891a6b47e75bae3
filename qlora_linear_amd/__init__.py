"""Fused NF4-LoRA linear for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``liblora_nf4.so`` (C ABI in include/lora_nf4.h). Each
function only marshals arguments: it checks tensor placement and dtypes,
allocates outputs with PyTorch (device memory is PyTorch's job here) and calls
the C entry point of the same name on the current HIP stream. Every step of the
computation runs in the library's HIP kernels; there is no fallback. If the
library has not been built, the first call raises.

    codes, absmax = nf4_quantize(w)                    # w [d_out, d_in] fp32/bf16
    y, u = lora_nf4_fwd(x, codes, absmax, A, B, lora_alpha)
    dx, dA, dB = lora_nf4_bwd(x, dy, codes, absmax, A, B, lora_alpha, u_saved=u)
    ys, us = lora_nf4_fwd_multi(x, [cq, ck, cv], [aq, ak, av], [Aq, Ak, Av], [Bq, Bk, Bv], alpha)
    dx, dAs, dBs = lora_nf4_bwd_multi(x, dys, [cq, ck, cv], [aq, ak, av], [Aq, Ak, Av], [Bq, Bk, Bv],
                                      alpha, u_saved=us)              # dx summed over q/k/v
    w_merged = lora_nf4_merge(codes, absmax, A, B, lora_alpha)   # bf16 [d_out, d_in]
    lora_adamw_step(A_master, A, dA, mA, vA, step, lr)           # in place, A = bf16(A_master)
    q, sc, off = nf4_absmax_quantize(absmax)                     # 8-bit block scales
    absmax2 = nf4_absmax_dequantize(q, sc, off).view_as(absmax)
    alpha_rs = rslora_alpha(lora_alpha, r)                       # scale alpha / sqrt(r)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LoraNF4Error", "library", "library_path", "nf4_quantize", "nf4_dequantize",
    "lora_nf4_fwd", "lora_nf4_fwd_multi", "lora_nf4_bwd", "lora_nf4_bwd_workspace_bytes", "lora_nf4_merge",
    "status_string", "EXPORTED_SYMBOLS", "LN_MAX_RANK", "LN_MAX_PROJ",
    "lora_adamw_step", "rslora_alpha", "nf4_absmax_quantize", "nf4_absmax_dequantize",
    "lora_nf4_bwd_multi", "lora_nf4_bwd_multi_workspace_bytes", "lora_nf4_bwd_noalloc",
    "set_weight_staging", "weight_staging", "lora_adamw8_step", "adamw8_state", "lora_nf4_bwd_adamw",
    "lora_nf4_grad_ab", "lora_nf4_grad_ab_workspace_bytes",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "liblora_nf4.so")

LN_OK, LN_F32, LN_BF16 = 0, 0, 1
LN_MAX_RANK = 256
LN_MAX_PROJ = 8
EXPORTED_SYMBOLS = ("nf4_quantize", "nf4_dequantize", "lora_nf4_fwd", "lora_nf4_fwd_multi",
                    "lora_nf4_bwd", "lora_nf4_bwd_workspace_bytes", "lora_nf4_merge",
                    "lora_nf4_status_string", "lora_adamw_step", "lora_nf4_rslora_alpha",
                    "nf4_absmax_quantize", "nf4_absmax_dequantize", "lora_nf4_bwd_multi",
                    "lora_nf4_bwd_multi_workspace_bytes", "lora_nf4_fwd_workspace_bytes",
                    "lora_nf4_fwd_multi_workspace_bytes", "lora_nf4_bwd_noalloc",
                    "lora_nf4_set_weight_staging", "lora_nf4_mfma_probe", "lora_adamw8_step",
                    "lora_nf4_bwd_adamw", "lora_nf4_grad_ab", "lora_nf4_grad_ab_workspace_bytes")

_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "nf4_quantize": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _p, _p, _p]),
    "nf4_dequantize": (ctypes.c_int, [_p, _p, _i64, _i64, ctypes.c_int, _p, _p]),
    "lora_nf4_fwd": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_float,
                                    _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "lora_nf4_fwd_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, ctypes.c_int32]),
    "lora_nf4_fwd_multi": (ctypes.c_int, [_i64, _i64, ctypes.c_int32, _p, ctypes.c_int32,
                                          ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "lora_nf4_fwd_multi_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, ctypes.c_int32, _p, ctypes.c_int32]),
    "lora_nf4_bwd": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_float,
                                    _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "lora_nf4_bwd_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, ctypes.c_int32]),
    "lora_nf4_grad_ab_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, ctypes.c_int32]),
    "lora_nf4_grad_ab": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_float,
                                        _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "lora_nf4_bwd_noalloc": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_float,
                                            _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "lora_nf4_merge": (ctypes.c_int, [_i64, _i64, ctypes.c_int32, ctypes.c_float, _p, _p, _p, _p,
                                      ctypes.c_int, _p, _p]),
    "lora_nf4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_adamw_step": (ctypes.c_int, [_i64, _p, _p, _p, _p, _p, ctypes.c_int32, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, _p]),
    "lora_adamw8_step": (ctypes.c_int, [_i64, _p, _p, _p, _p, _p, _p, _p, ctypes.c_int32, ctypes.c_float,
                                        ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, _p]),
    "lora_nf4_bwd_adamw": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int32, ctypes.c_float, _p, _p, _p, _p,
                                          _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_int32,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                          ctypes.c_float, _p, ctypes.c_size_t, _p]),
    "lora_nf4_rslora_alpha": (ctypes.c_float, [ctypes.c_float, ctypes.c_int32]),
    "lora_nf4_set_weight_staging": (ctypes.c_int, [ctypes.c_int32]),
    "lora_nf4_mfma_probe": (ctypes.c_int64, [ctypes.c_int32, _p, _p]),
    "lora_nf4_bwd_multi": (ctypes.c_int, [_i64, _i64, ctypes.c_int32, _p, ctypes.c_int32, ctypes.c_float,
                                          _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]),
    "lora_nf4_bwd_multi_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, ctypes.c_int32, _p, ctypes.c_int32]),
    "nf4_absmax_quantize": (ctypes.c_int, [_p, _i64, _p, _p, _p, _p]),
    "nf4_absmax_dequantize": (ctypes.c_int, [_p, _p, _p, _i64, _p, _p]),
}


class LoraNF4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


def library():
    """The loaded liblora_nf4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with `python -m qlora_linear_amd.build` "
                "(there is no non-HIP fallback)")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return library().lora_nf4_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != LN_OK:
        raise LoraNF4Error(fn, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    return t


def nf4_quantize(w: torch.Tensor):
    """NF4-quantize a [rows, cols] float32 or bf16 matrix (cols % 64 == 0).

    Returns (codes uint8 [rows, cols/2], absmax float32 [rows, cols/64]).
    """
    _dev(w, "w", ndim=2)
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    rows, cols = w.shape
    codes = torch.empty((rows, max(cols // 2, 1)), dtype=torch.uint8, device=w.device)
    absmax = torch.empty((rows, max(cols // 64, 1)), dtype=torch.float32, device=w.device)
    dt = LN_BF16 if w.dtype == torch.bfloat16 else LN_F32
    _check("nf4_quantize", library().nf4_quantize(w.data_ptr(), dt, rows, cols, codes.data_ptr(),
                                                  absmax.data_ptr(), _stream(w)))
    return codes, absmax


def nf4_dequantize(codes: torch.Tensor, absmax: torch.Tensor, dtype=torch.float32):
    """Dequantize NF4 codes/absmax back to a [rows, cols] float32 or bf16 matrix."""
    _dev(codes, "codes", torch.uint8, 2)
    _dev(absmax, "absmax", torch.float32, 2)
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be float32 or bfloat16")
    rows, cols = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((rows, cols), dtype=dtype, device=codes.device)
    dt = LN_BF16 if dtype == torch.bfloat16 else LN_F32
    _check("nf4_dequantize", library().nf4_dequantize(codes.data_ptr(), absmax.data_ptr(), rows,
                                                      cols, dt, out.data_ptr(), _stream(codes)))
    return out


def _lora_shapes(x, codes, A, B):
    T, K = x.shape
    N = codes.shape[0]
    r = A.shape[1]
    if codes.shape[1] * 2 != K or A.shape[0] != K or B.shape != (r, N):
        raise ValueError(f"inconsistent shapes: x {tuple(x.shape)}, codes {tuple(codes.shape)}, "
                         f"A {tuple(A.shape)}, B {tuple(B.shape)}")
    return T, K, N, r


def lora_nf4_fwd_workspace_bytes(T: int, K: int, N: int, r: int) -> int:
    return int(library().lora_nf4_fwd_workspace_bytes(T, K, N, r))


def _workspace(nbytes: int, workspace, device):
    """The caller's workspace tensor, or a new one when the entry point needs one."""
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None
    return _dev(workspace, "workspace", torch.uint8)


def lora_nf4_fwd(x, codes, absmax, A, B, lora_alpha: float, save_u: bool = True, out=None,
                 workspace: torch.Tensor | None = None):
    """y = x deq(W)^T + (lora_alpha / r) (x A) B; returns (y, u) with u = bf16(x A) or None.
    Few-token shapes need a workspace (lora_nf4_fwd_workspace_bytes); one is allocated
    when none is given."""
    bf = torch.bfloat16
    _dev(x, "x", bf, 2), _dev(codes, "codes", torch.uint8, 2), _dev(absmax, "absmax", torch.float32, 2)
    _dev(A, "A", bf, 2), _dev(B, "B", bf, 2)
    T, K, N, r = _lora_shapes(x, codes, A, B)
    y = torch.empty((T, N), dtype=bf, device=x.device) if out is None else _dev(out, "out", bf, 2)
    u = torch.empty((T, r), dtype=bf, device=x.device) if save_u else None
    ws = _workspace(lora_nf4_fwd_workspace_bytes(T, K, N, r), workspace, x.device)
    _check("lora_nf4_fwd", library().lora_nf4_fwd(T, K, N, r, float(lora_alpha), x.data_ptr(),
                                                  codes.data_ptr(), absmax.data_ptr(), A.data_ptr(),
                                                  B.data_ptr(), y.data_ptr(), _ptr(u), _ptr(ws),
                                                  0 if ws is None else ws.numel(), _stream(x)))
    return y, u


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def lora_nf4_fwd_multi_workspace_bytes(T: int, K: int, d_outs, r: int) -> int:
    n = len(d_outs)
    arr = (ctypes.c_int64 * n)(*d_outs)
    return int(library().lora_nf4_fwd_multi_workspace_bytes(T, K, n, ctypes.cast(arr, ctypes.c_void_p), r))


def lora_nf4_fwd_multi(x, codes, absmax, A, B, lora_alpha: float, save_u: bool = True,
                       workspace: torch.Tensor | None = None):
    """Forward of several projections that share x (lists, one entry per projection):
    returns ([y_g], [u_g] or None), the same values as one lora_nf4_fwd per projection."""
    bf = torch.bfloat16
    _dev(x, "x", bf, 2)
    n = len(codes)
    if not (len(absmax) == len(A) == len(B) == n) or n < 1:
        raise ValueError("codes, absmax, A and B must be lists of the same non-zero length")
    shapes = []
    for g in range(n):
        _dev(codes[g], f"codes[{g}]", torch.uint8, 2), _dev(absmax[g], f"absmax[{g}]", torch.float32, 2)
        _dev(A[g], f"A[{g}]", bf, 2), _dev(B[g], f"B[{g}]", bf, 2)
        shapes.append(_lora_shapes(x, codes[g], A[g], B[g]))
    T, K, _, r = shapes[0]
    if any(sh[3] != r for sh in shapes):
        raise ValueError("all projections must share the rank r")
    ys = [torch.empty((T, sh[2]), dtype=bf, device=x.device) for sh in shapes]
    us = [torch.empty((T, r), dtype=bf, device=x.device) for _ in shapes] if save_u else None
    d_out = (ctypes.c_int64 * n)(*[sh[2] for sh in shapes])
    keep = [_ptr_array([t.data_ptr() for t in lst]) for lst in (codes, absmax, A, B, ys)]
    u_arr = _ptr_array([t.data_ptr() for t in us]) if save_u else (None, None)
    ws = _workspace(lora_nf4_fwd_multi_workspace_bytes(T, K, [sh[2] for sh in shapes], r), workspace,
                    x.device)
    _check("lora_nf4_fwd_multi", library().lora_nf4_fwd_multi(
        T, K, n, ctypes.cast(d_out, ctypes.c_void_p), r, float(lora_alpha), x.data_ptr(),
        keep[0][1], keep[1][1], keep[2][1], keep[3][1], keep[4][1], u_arr[1], _ptr(ws),
        0 if ws is None else ws.numel(), _stream(x)))
    return ys, us


def lora_nf4_bwd_workspace_bytes(T: int, K: int, N: int, r: int) -> int:
    return int(library().lora_nf4_bwd_workspace_bytes(T, K, N, r))


def lora_nf4_bwd(x, dy, codes, absmax, A, B, lora_alpha: float, u_saved=None, need_dx: bool = True,
                 workspace: torch.Tensor | None = None):
    """Gradients (dx or None, dA, dB) of the forward for upstream gradient dy."""
    bf = torch.bfloat16
    _dev(x, "x", bf, 2), _dev(dy, "dy", bf, 2), _dev(codes, "codes", torch.uint8, 2)
    _dev(absmax, "absmax", torch.float32, 2), _dev(A, "A", bf, 2), _dev(B, "B", bf, 2)
    T, K, N, r = _lora_shapes(x, codes, A, B)
    if dy.shape != (T, N):
        raise ValueError("dy must be [T, d_out]")
    if u_saved is not None:
        _dev(u_saved, "u_saved", bf, 2)
    dev = x.device
    dx = torch.empty((T, K), dtype=bf, device=dev) if need_dx else None
    dA = torch.empty((K, r), dtype=bf, device=dev)
    dB = torch.empty((r, N), dtype=bf, device=dev)
    nbytes = lora_nf4_bwd_workspace_bytes(T, K, N, r)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    _check("lora_nf4_bwd", library().lora_nf4_bwd(
        T, K, N, r, float(lora_alpha), x.data_ptr(), dy.data_ptr(), codes.data_ptr(),
        absmax.data_ptr(), A.data_ptr(), B.data_ptr(), _ptr(u_saved), _ptr(dx), dA.data_ptr(),
        dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(x)))
    return dx, dA, dB


def lora_nf4_grad_ab_workspace_bytes(T: int, K: int, N: int, r: int) -> int:
    return int(library().lora_nf4_grad_ab_workspace_bytes(T, K, N, r))


def lora_nf4_grad_ab(x, g, dy, u, lora_alpha: float, workspace: torch.Tensor | None = None):
    """(dA, dB) = (x^T g, s u^T dy) from the backward's intermediates g = bf16(s dy B^T)
    and u = bf16(x A), each [T, r]."""
    bf = torch.bfloat16
    _dev(x, "x", bf, 2), _dev(g, "g", bf, 2), _dev(dy, "dy", bf, 2), _dev(u, "u", bf, 2)
    T, K = x.shape
    N, r = dy.shape[1], g.shape[1]
    if dy.shape[0] != T or g.shape[0] != T or u.shape != (T, r):
        raise ValueError("x [T, d_in], g [T, r], dy [T, d_out] and u [T, r] must agree")
    dev = x.device
    dA = torch.empty((K, r), dtype=bf, device=dev)
    dB = torch.empty((r, N), dtype=bf, device=dev)
    nbytes = lora_nf4_grad_ab_workspace_bytes(T, K, N, r)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    _check("lora_nf4_grad_ab", library().lora_nf4_grad_ab(
        T, K, N, r, float(lora_alpha), x.data_ptr(), g.data_ptr(), dy.data_ptr(), u.data_ptr(), dA.data_ptr(),
        dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(x)))
    return dA, dB


def lora_nf4_bwd_noalloc(x, dy, codes, absmax, A, B, lora_alpha: float, u_saved=None, need_dx: bool = True):
    """lora_nf4_bwd without a workspace argument: the library's own device scratch
    serves as its workspace (calls overlapping on one GPU race)."""
    bf = torch.bfloat16
    _dev(x, "x", bf, 2), _dev(dy, "dy", bf, 2), _dev(codes, "codes", torch.uint8, 2)
    _dev(absmax, "absmax", torch.float32, 2), _dev(A, "A", bf, 2), _dev(B, "B", bf, 2)
    T, K, N, r = _lora_shapes(x, codes, A, B)
    if dy.shape != (T, N):
        raise ValueError("dy must be [T, d_out]")
    if u_saved is not None:
        _dev(u_saved, "u_saved", bf, 2)
    dev = x.device
    dx = torch.empty((T, K), dtype=bf, device=dev) if need_dx else None
    dA = torch.empty((K, r), dtype=bf, device=dev)
    dB = torch.empty((r, N), dtype=bf, device=dev)
    _check("lora_nf4_bwd_noalloc", library().lora_nf4_bwd_noalloc(
        T, K, N, r, float(lora_alpha), x.data_ptr(), dy.data_ptr(), codes.data_ptr(),
        absmax.data_ptr(), A.data_ptr(), B.data_ptr(), _ptr(u_saved), _ptr(dx), dA.data_ptr(),
        dB.data_ptr(), _stream(x)))
    return dx, dA, dB


def lora_nf4_bwd_multi_workspace_bytes(T: int, K: int, d_outs, r: int) -> int:
    n = len(d_outs)
    arr = (ctypes.c_int64 * n)(*d_outs)
    return int(library().lora_nf4_bwd_multi_workspace_bytes(T, K, n, ctypes.cast(arr, ctypes.c_void_p), r))


def lora_nf4_bwd_multi(x, dy, codes, absmax, A, B, lora_alpha: float, u_saved=None, need_dx: bool = True,
                       workspace: torch.Tensor | None = None):
    """Backward of projections sharing x: (dx summed over them or None, [dA_g], [dB_g])."""
    bf = torch.bfloat16
    _dev(x, "x", bf, 2)
    n = len(codes)
    if not (len(dy) == len(absmax) == len(A) == len(B) == n) or (u_saved is not None and len(u_saved) != n):
        raise ValueError("dy, codes, absmax, A, B (and u_saved) need one entry per projection")
    shapes = []
    for g in range(n):
        _dev(dy[g], f"dy[{g}]", bf, 2), _dev(codes[g], f"codes[{g}]", torch.uint8, 2)
        _dev(absmax[g], f"absmax[{g}]", torch.float32, 2), _dev(A[g], f"A[{g}]", bf, 2), _dev(B[g], f"B[{g}]", bf, 2)
        if u_saved is not None and u_saved[g] is not None:
            _dev(u_saved[g], f"u_saved[{g}]", bf, 2)
        sh = _lora_shapes(x, codes[g], A[g], B[g])
        if dy[g].shape != (sh[0], sh[2]):
            raise ValueError(f"dy[{g}] must be [T, d_out]")
        shapes.append(sh)
    T, K, _, r = shapes[0]
    if any(sh[3] != r for sh in shapes):
        raise ValueError("all projections must share the rank r")
    dev = x.device
    dx = torch.empty((T, K), dtype=bf, device=dev) if need_dx else None
    dAs = [torch.empty((K, r), dtype=bf, device=dev) for _ in range(n)]
    dBs = [torch.empty((r, sh[2]), dtype=bf, device=dev) for sh in shapes]
    d_out = [sh[2] for sh in shapes]
    nbytes = lora_nf4_bwd_multi_workspace_bytes(T, K, d_out, r)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    d_arr = (ctypes.c_int64 * n)(*d_out)
    keep = [_ptr_array([t.data_ptr() for t in lst]) for lst in (dy, codes, absmax, A, B, dAs, dBs)]
    u_arr = _ptr_array([0 if t is None else t.data_ptr() for t in u_saved]) if u_saved is not None else (None, None)
    _check("lora_nf4_bwd_multi", library().lora_nf4_bwd_multi(
        T, K, n, ctypes.cast(d_arr, ctypes.c_void_p), r, float(lora_alpha), x.data_ptr(), keep[0][1], keep[1][1],
        keep[2][1], keep[3][1], keep[4][1], u_arr[1], _ptr(dx), keep[5][1], keep[6][1], workspace.data_ptr(),
        workspace.numel(), _stream(x)))
    return dx, dAs, dBs


def lora_nf4_merge(codes, absmax, A, B, lora_alpha: float, dtype=torch.bfloat16):
    """Merged base weight W' = deq(W) + (lora_alpha / r) (A B)^T, [d_out, d_in], bf16 or float32."""
    _dev(codes, "codes", torch.uint8, 2), _dev(absmax, "absmax", torch.float32, 2)
    _dev(A, "A", torch.bfloat16, 2), _dev(B, "B", torch.bfloat16, 2)
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be float32 or bfloat16")
    N, K, r = codes.shape[0], codes.shape[1] * 2, A.shape[1]
    if A.shape[0] != K or B.shape != (r, N):
        raise ValueError(f"inconsistent shapes: codes {tuple(codes.shape)}, A {tuple(A.shape)}, "
                         f"B {tuple(B.shape)}")
    out = torch.empty((N, K), dtype=dtype, device=codes.device)
    dt = LN_BF16 if dtype == torch.bfloat16 else LN_F32
    _check("lora_nf4_merge", library().lora_nf4_merge(K, N, r, float(lora_alpha), codes.data_ptr(),
                                                      absmax.data_ptr(), A.data_ptr(), B.data_ptr(), dt,
                                                      out.data_ptr(), _stream(codes)))
    return out


def lora_adamw_step(p_master, p_bf16, grad, m, v, step: int, lr: float, betas=(0.9, 0.999),
                    eps: float = 1e-8, weight_decay: float = 0.0):
    """One AdamW step in place: p_master (float32), p_bf16 = bf16(p_master), moments m, v (float32)."""
    bf, f32 = torch.bfloat16, torch.float32
    _dev(p_master, "p_master", f32), _dev(p_bf16, "p_bf16", bf), _dev(grad, "grad", bf)
    _dev(m, "m", f32), _dev(v, "v", f32)
    n = p_master.numel()
    for t, name in ((p_bf16, "p_bf16"), (grad, "grad"), (m, "m"), (v, "v")):
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements, p_master {n}")
    _check("lora_adamw_step", library().lora_adamw_step(
        n, p_master.data_ptr(), p_bf16.data_ptr(), grad.data_ptr(), m.data_ptr(), v.data_ptr(), int(step),
        float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay), _stream(p_master)))


def adamw8_state(n: int, device="cuda"):
    """Zero 8-bit AdamW state for n elements: (m codes, m scales, v codes, v scales)."""
    nb = (n + 255) // 256
    return (torch.zeros(n, dtype=torch.uint8, device=device), torch.zeros(nb, dtype=torch.float32, device=device),
            torch.zeros(n, dtype=torch.uint8, device=device), torch.zeros(nb, dtype=torch.float32, device=device))


def lora_adamw8_step(p_master, p_bf16, grad, state, step: int, lr: float, betas=(0.9, 0.999),
                     eps: float = 1e-8, weight_decay: float = 0.0):
    """One AdamW step with 8-bit blockwise moments, in place; state from adamw8_state."""
    bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
    mq, ms, vq, vs = state
    _dev(p_master, "p_master", f32), _dev(p_bf16, "p_bf16", bf), _dev(grad, "grad", bf)
    _dev(mq, "m codes", u8), _dev(ms, "m scales", f32), _dev(vq, "v codes", u8), _dev(vs, "v scales", f32)
    n = p_master.numel()
    nb = (n + 255) // 256
    for t, name, want in ((p_bf16, "p_bf16", n), (grad, "grad", n), (mq, "m codes", n), (vq, "v codes", n),
                          (ms, "m scales", nb), (vs, "v scales", nb)):
        if t.numel() != want:
            raise ValueError(f"{name} has {t.numel()} elements, expected {want}")
    _check("lora_adamw8_step", library().lora_adamw8_step(
        n, p_master.data_ptr(), p_bf16.data_ptr(), grad.data_ptr(), mq.data_ptr(), ms.data_ptr(), vq.data_ptr(),
        vs.data_ptr(), int(step), float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay),
        _stream(p_master)))


def lora_nf4_bwd_adamw(x, dy, codes, absmax, A, B, lora_alpha: float, state, step: int, lr: float,
                       betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.0, u_saved=None,
                       need_dx: bool = True, workspace: torch.Tensor | None = None):
    """The backward with the AdamW step of A and B applied in its rank-r reduction:
    A and B (bf16) are updated in place, state = (A master, A m, A v, B master, B m, B v)
    float32 tensors shaped like A and B. Returns dx (or None)."""
    bf, f32 = torch.bfloat16, torch.float32
    _dev(x, "x", bf, 2), _dev(dy, "dy", bf, 2), _dev(codes, "codes", torch.uint8, 2)
    _dev(absmax, "absmax", f32, 2), _dev(A, "A", bf, 2), _dev(B, "B", bf, 2)
    T, K, N, r = _lora_shapes(x, codes, A, B)
    if dy.shape != (T, N):
        raise ValueError("dy must be [T, d_out]")
    if u_saved is not None:
        _dev(u_saved, "u_saved", bf, 2)
    names = ("A master", "A m", "A v", "B master", "B m", "B v")
    for t, name, shape in zip(state, names, (A.shape,) * 3 + (B.shape,) * 3):
        _dev(t, name, f32)
        if t.shape != shape:
            raise ValueError(f"{name} must have shape {tuple(shape)}")
    dev = x.device
    dx = torch.empty((T, K), dtype=bf, device=dev) if need_dx else None
    nbytes = lora_nf4_bwd_workspace_bytes(T, K, N, r)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    _check("lora_nf4_bwd_adamw", library().lora_nf4_bwd_adamw(
        T, K, N, r, float(lora_alpha), x.data_ptr(), dy.data_ptr(), codes.data_ptr(), absmax.data_ptr(),
        A.data_ptr(), B.data_ptr(), _ptr(u_saved), _ptr(dx), *(t.data_ptr() for t in state), int(step),
        float(lr), float(betas[0]), float(betas[1]), float(eps), float(weight_decay), workspace.data_ptr(),
        workspace.numel(), _stream(x)))
    return dx


def rslora_alpha(lora_alpha: float, r: int) -> float:
    """The lora_alpha whose library scale lora_alpha / r equals f32(lora_alpha / sqrt(r))."""
    a = library().lora_nf4_rslora_alpha(float(lora_alpha), int(r))
    if a != a:
        raise ValueError(f"no rank-stabilized alpha for lora_alpha={lora_alpha}, r={r}")
    return a


def set_weight_staging(enabled: bool) -> bool:
    """lora_nf4_set_weight_staging: True makes the large-token forward and dX read a
    bf16 copy of the weight dequantized into their workspace; False (the default)
    keeps the dequantization inside every kernel's main loop. Returns the previous
    setting."""
    return bool(library().lora_nf4_set_weight_staging(1 if enabled else 0))


class weight_staging:
    """Context manager: `with weight_staging(True): ...` runs the block with weight
    staging set as given and restores the previous setting on exit."""

    def __init__(self, enabled: bool):
        self.enabled = bool(enabled)
        self.prev = None

    def __enter__(self):
        self.prev = set_weight_staging(self.enabled)
        return self

    def __exit__(self, *exc):
        set_weight_staging(self.prev)
        return False


def nf4_absmax_quantize(absmax):
    """Double quantization of NF4 block scales: (codes uint8 [n], scale, offset float32 [ceil(n/256)])."""
    _dev(absmax, "absmax", torch.float32)
    n = absmax.numel()
    nb = (n + 255) // 256
    dev = absmax.device
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    sc = torch.empty(nb, dtype=torch.float32, device=dev)
    off = torch.empty(nb, dtype=torch.float32, device=dev)
    _check("nf4_absmax_quantize", library().nf4_absmax_quantize(absmax.data_ptr(), n, q.data_ptr(),
                                                                sc.data_ptr(), off.data_ptr(), _stream(absmax)))
    return q, sc, off


def nf4_absmax_dequantize(q, scale, offset):
    """float32 [n] block scales from their double-quantized form (use .view_as(absmax))."""
    _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32), _dev(offset, "offset", torch.float32)
    n = q.numel()
    nb = (n + 255) // 256
    if scale.numel() != nb or offset.numel() != nb:
        raise ValueError(f"scale and offset need {nb} entries for {n} codes")
    out = torch.empty(n, dtype=torch.float32, device=q.device)
    _check("nf4_absmax_dequantize", library().nf4_absmax_dequantize(
        q.data_ptr(), scale.data_ptr(), offset.data_ptr(), n, out.data_ptr(), _stream(q)))
    return out
