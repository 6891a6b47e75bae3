"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call."""
import contextlib
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_nf4.h")

LN_OK, LN_EINVAL, LN_ESHAPE, LN_EALIGN, LN_ERANK, LN_EWORKSPACE, LN_EALIAS = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def lib():
    import qlora_linear_amd as q
    if not os.path.exists(q.library_path):
        from qlora_linear_amd import build
        build.build()
    return q.library()


@contextlib.contextmanager
def staging(lib, on):
    """Weight staging (lora_nf4_set_weight_staging) set for the block, then restored."""
    prev = lib.lora_nf4_set_weight_staging(1 if on else 0)
    assert prev in (0, 1)
    try:
        yield
    finally:
        lib.lora_nf4_set_weight_staging(prev)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["nf4_quantize", "nf4_dequantize", "lora_nf4_fwd", "lora_nf4_fwd_multi",
                            "lora_nf4_bwd", "lora_nf4_bwd_workspace_bytes", "lora_nf4_merge",
                            "lora_nf4_status_string", "lora_adamw_step", "lora_nf4_rslora_alpha",
                            "nf4_absmax_quantize", "nf4_absmax_dequantize", "lora_nf4_bwd_multi",
                            "lora_nf4_bwd_multi_workspace_bytes", "lora_nf4_fwd_workspace_bytes",
                            "lora_nf4_fwd_multi_workspace_bytes", "lora_nf4_bwd_noalloc",
                            "lora_nf4_set_weight_staging", "lora_nf4_mfma_probe", "lora_adamw8_step",
                            "lora_nf4_bwd_adamw", "lora_nf4_grad_ab", "lora_nf4_grad_ab_workspace_bytes"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    import qlora_linear_amd as q
    assert sorted(q.EXPORTED_SYMBOLS) == declared_functions()


def test_status_strings(lib):
    for st in range(0, -8, -1):
        s = lib.lora_nf4_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.lora_nf4_status_string(-99).decode() == "unknown status"


# Plausible device-like addresses (never dereferenced: every call below fails validation).
P = 1 << 40


def _fwd(lib, T=8, K=64, N=64, r=8, alpha=16.0, x=P, c=P + (1 << 30), a=P + (2 << 30), A=P + (3 << 30),
         B=P + (4 << 30), y=P + (5 << 30), u=None, ws=P + (6 << 30), ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.lora_nf4_fwd_workspace_bytes(max(T, 0), K, N, r)
    return lib.lora_nf4_fwd(T, K, N, r, alpha, x, c, a, A, B, y, u, ws, ctypes.c_size_t(ws_bytes), None)


def test_fwd_validation(lib):
    assert _fwd(lib, x=None) == LN_EINVAL
    assert _fwd(lib, T=-1) == LN_EINVAL
    # T = 0 is an empty batch: accepted, nothing enqueued, token operands may be NULL
    assert _fwd(lib, T=0) == LN_OK
    assert _fwd(lib, T=0, x=None, y=None) == LN_OK
    assert _fwd(lib, T=0, A=None) == LN_EINVAL
    assert _fwd(lib, alpha=float("nan")) == LN_EINVAL
    assert _fwd(lib, r=0) == LN_ERANK
    assert _fwd(lib, r=257) == LN_ERANK
    assert _fwd(lib, K=100) == LN_ESHAPE
    # the shape rules of the linear: 1 <= r <= 256 and any d_out >= 1 (checked with
    # an empty batch, which validates every size and then enqueues nothing)
    for r in (1, 129, 200, 256):
        assert _fwd(lib, T=0, r=r) == LN_OK
    for n in (1, 7, 12, 13):
        assert _fwd(lib, T=0, N=n) == LN_OK
    assert _fwd(lib, T=0, N=0) == LN_EINVAL
    assert _fwd(lib, x=P + 8) == LN_EALIGN
    assert _fwd(lib, y=P) == LN_EALIAS                      # output on top of x
    assert _fwd(lib, u=P + (5 << 30) + 64) == LN_EALIAS     # u_save inside y


def test_fwd_workspace(lib):
    """Up to 128 tokens the reduction over d_in is split across workgroups, with a
    workspace (except a few tokens on d_out <= 4096: one streaming launch); the
    tiled path takes none below 1024 tokens (NULL accepted) and the dequantized
    weight from 1024 tokens on; the generic path takes none."""
    need = lib.lora_nf4_fwd_workspace_bytes(64, 64, 64, 8)
    assert need > 0 and need % 256 == 0
    assert lib.lora_nf4_fwd_workspace_bytes(128, 4096, 4096, 16) > 0
    assert lib.lora_nf4_fwd_workspace_bytes(8, 4096, 8192, 16) > 0       # few tokens, wide d_out
    assert lib.lora_nf4_fwd_workspace_bytes(8, 4096, 4096, 16) == 0      # few tokens: streaming
    assert lib.lora_nf4_fwd_workspace_bytes(1000, 4096, 4096, 16) == 0   # tiled
    # from 4096 tokens on 256 x 256 tiles (d_in % 256 == 0) the weight stays packed:
    # at rank 16 the kernel computes U itself (no workspace); at other ranks the
    # workspace holds A^T and bf16(s U) of the U pass
    assert lib.lora_nf4_fwd_workspace_bytes(8192, 4096, 4096, 16) == 0
    assert lib.lora_nf4_fwd_workspace_bytes(8192, 4096, 4096, 32) == 32 * 4096 * 2 + 8192 * 32 * 2
    # by default no path stages a bf16 copy of the weight
    assert lib.lora_nf4_fwd_workspace_bytes(2048, 4096, 4096, 16) == 0
    assert lib.lora_nf4_fwd_workspace_bytes(1024, 320, 200, 16) == 0
    with staging(lib, True):
        # staged: from 1024 tokens on 128 x 128 tiles the weight is dequantized once
        # into it (bf16), and from 4096 on 256 x 256 tiles
        assert lib.lora_nf4_fwd_workspace_bytes(2048, 4096, 4096, 16) >= 4096 * 4096 * 2
        assert lib.lora_nf4_fwd_workspace_bytes(1024, 320, 200, 16) == (320 * 200 * 2 + 255) // 256 * 256
        assert lib.lora_nf4_fwd_workspace_bytes(8192, 4096, 4096, 16) >= 4096 * 4096 * 2
    assert lib.lora_nf4_fwd_workspace_bytes(64, 64, 64, 12) == 0         # r % 8 != 0: generic kernels
    assert lib.lora_nf4_fwd_workspace_bytes(0, 64, 64, 8) == 0
    assert lib.lora_nf4_fwd_workspace_bytes(64, 65, 64, 8) == 0          # invalid sizes
    assert _fwd(lib, T=64, ws=None) == LN_EWORKSPACE
    assert _fwd(lib, T=64, ws_bytes=need - 1) == LN_EWORKSPACE
    assert _fwd(lib, T=64, ws=P + (6 << 30) + 16) == LN_EALIGN
    assert _fwd(lib, T=64, ws=P + (5 << 30)) == LN_EALIAS            # workspace on top of y
    assert _fwd(lib, T=64, ws=P + (3 << 30)) == LN_EALIAS            # workspace on top of A
    assert _fwd(lib, T=0, ws=None, ws_bytes=0) == LN_OK
    # multi: the largest per-projection need when the projections run one by one
    vp = ctypes.c_void_p
    d_out = (ctypes.c_int64 * 3)(64, 16, 16)
    assert lib.lora_nf4_fwd_multi_workspace_bytes(64, 64, 3, ctypes.cast(d_out, vp), 8) == need
    big = (ctypes.c_int64 * 3)(4096, 1024, 1024)
    # one launch of 256 x 256 register-dequantizing tiles: at rank 16 U is computed in
    # the kernel (none); at rank 32 one U pass per projection (A^T and bf16(s U) each)
    assert lib.lora_nf4_fwd_multi_workspace_bytes(8192, 4096, 3, ctypes.cast(big, vp), 16) == 0
    assert lib.lora_nf4_fwd_multi_workspace_bytes(8192, 4096, 3, ctypes.cast(big, vp), 32) == 3 * (32 * 4096 * 2 + 8192 * 32 * 2)
    assert lib.lora_nf4_fwd_multi_workspace_bytes(64, 64, 0, ctypes.cast(d_out, vp), 8) == 0


def _fwd_multi(lib, n=3, T=8, K=64, N=(64, 16, 16), r=8, alpha=16.0, x=P, ptrs=None, u=None, null=None,
               ws=P + (7 << 30), ws_bytes=None):
    # projection g's tensors sit at P + ((8 g + i) << 30), i = codes, absmax, A, B, y
    vp = ctypes.c_void_p
    base = {name: [P + ((8 * (g + 1) + i) << 30) for g in range(n)]
            for i, name in enumerate(("codes", "absmax", "A", "B", "y"))}
    if ptrs:
        for name, (g, v) in ptrs.items():
            base[name][g] = v
    arrs = {name: (vp * n)(*vals) for name, vals in base.items()}
    if null:
        arrs[null] = None
    d_out = (ctypes.c_int64 * n)(*list(N)[:n])
    u_arr = None if u is None else (vp * n)(*u)
    if ws_bytes is None:
        ws_bytes = lib.lora_nf4_fwd_multi_workspace_bytes(max(T, 0), K, n, ctypes.cast(d_out, vp), r)
    return lib.lora_nf4_fwd_multi(T, K, n, ctypes.cast(d_out, vp), r, alpha, x,
                                  *(ctypes.cast(arrs[k], vp) if arrs[k] is not None else None
                                    for k in ("codes", "absmax", "A", "B", "y")),
                                  ctypes.cast(u_arr, vp) if u_arr is not None else None, ws,
                                  ctypes.c_size_t(ws_bytes), None)


def test_fwd_multi_validation(lib):
    assert _fwd_multi(lib, n=0) == LN_EINVAL
    assert _fwd_multi(lib, T=0, x=None) == LN_OK
    assert _fwd_multi(lib, n=9, N=(64,) * 9) == LN_EINVAL
    assert _fwd_multi(lib, null="A") == LN_EINVAL
    assert _fwd_multi(lib, x=None) == LN_EINVAL
    assert _fwd_multi(lib, ptrs={"B": (1, None)}) == LN_EINVAL
    assert _fwd_multi(lib, T=0, N=(64, 12, 16)) == LN_OK   # empty batch: validated, nothing enqueued
    assert _fwd_multi(lib, N=(64, 0, 16)) == LN_EINVAL
    assert _fwd_multi(lib, K=100) == LN_ESHAPE
    assert _fwd_multi(lib, r=0) == LN_ERANK
    assert _fwd_multi(lib, alpha=float("inf")) == LN_EINVAL
    assert _fwd_multi(lib, x=P + 8) == LN_EALIGN
    assert _fwd_multi(lib, ptrs={"codes": (2, P + (3 << 30) + 4)}) == LN_EALIGN
    y0 = P + ((8 * 1 + 4) << 30)
    assert _fwd_multi(lib, ptrs={"y": (2, y0 + 256)}) == LN_EALIAS     # y[2] inside y[0]
    assert _fwd_multi(lib, ptrs={"y": (1, P)}) == LN_EALIAS            # y[1] on top of x
    assert _fwd_multi(lib, u=[None, y0, None]) == LN_EALIAS           # u[1] on top of y[0]
    assert _fwd_multi(lib, T=64, ws=None) == LN_EWORKSPACE
    assert _fwd_multi(lib, T=64, ws=y0) == LN_EALIAS                  # workspace on top of y[0]


def test_bwd_workspace_holds_the_dequantized_weight_at_large_token_counts(lib):
    """With weight staging on, dX runs on a bf16 copy of the weight from 1024 tokens
    on 128 x 128 tiles and from 4096 on 256 x 256 tiles (q_proj 4096 x 4096 takes
    128 tiles at 1024 tokens and 256 at 4095 and 4096): the workspace grows by at
    least 2 d_in d_out bytes across each threshold. By default there is no such
    copy; at rank 16 the 256 x 256 dX tiles dequantize in registers from the packed
    weight transposed into the workspace: d_in d_out / 2 bytes of codes plus
    d_in d_out / 16 of absmax."""
    K = N = 4096
    w = 2 * K * N
    packed_t = K * N // 2 + (K // 64) * N * 4
    with staging(lib, True):
        for r in (16, 64):
            assert lib.lora_nf4_bwd_workspace_bytes(1023, K, N, r) < w
            assert lib.lora_nf4_bwd_workspace_bytes(1024, K, N, r) - lib.lora_nf4_bwd_workspace_bytes(1023, K, N, r) >= w
            assert lib.lora_nf4_bwd_workspace_bytes(4095, K, N, r) < w
            assert lib.lora_nf4_bwd_workspace_bytes(4096, K, N, r) - lib.lora_nf4_bwd_workspace_bytes(4095, K, N, r) >= w
            assert lib.lora_nf4_bwd_workspace_bytes(8192, K, N, r) >= w
    for r in (16, 64):
        for T in (1024, 2048, 4096, 8192):
            assert lib.lora_nf4_bwd_workspace_bytes(T, K, N, r) < w
        assert lib.lora_nf4_bwd_workspace_bytes(8192, K, 4160, r) < 2 * K * 4160
    r = 16
    grow = lib.lora_nf4_bwd_workspace_bytes(4096, K, N, r) - lib.lora_nf4_bwd_workspace_bytes(4095, K, N, r)
    assert packed_t <= grow < w


def test_weight_staging_mode(lib):
    assert lib.lora_nf4_set_weight_staging(-1) == 0  # the default: in-loop dequantization
    assert lib.lora_nf4_set_weight_staging(2) == LN_EINVAL
    assert lib.lora_nf4_set_weight_staging(-2) == LN_EINVAL
    assert lib.lora_nf4_set_weight_staging(1) == 0
    assert lib.lora_nf4_set_weight_staging(-1) == 1
    assert lib.lora_nf4_set_weight_staging(0) == 1
    assert lib.lora_nf4_set_weight_staging(-1) == 0


def test_bwd_validation_and_workspace(lib):
    T, K, N, r = 8, 64, 64, 8
    need = lib.lora_nf4_bwd_workspace_bytes(T, K, N, r)
    assert need > 0
    assert lib.lora_nf4_bwd_workspace_bytes(0, K, N, r) == 0
    assert lib.lora_nf4_bwd_workspace_bytes(T, 65, N, r) == 0
    assert lib.lora_nf4_bwd_workspace_bytes(T, K, N, 0) == 0
    ptrs = [P + (i << 30) for i in range(12)]
    x, dy, c, a, A, B, u, dx, dA, dB, ws = ptrs[:11]

    def call(ws_ptr=ws, ws_bytes=need, **kw):
        args = dict(x=x, dy=dy, c=c, a=a, A=A, B=B, u=u, dx=dx, dA=dA, dB=dB)
        args.update(kw)
        return lib.lora_nf4_bwd(T, K, N, r, 16.0, args["x"], args["dy"], args["c"], args["a"], args["A"],
                                args["B"], args["u"], args["dx"], args["dA"], args["dB"], ws_ptr,
                                ctypes.c_size_t(ws_bytes), None)

    assert call(dA=None) == LN_EINVAL
    assert call(ws_ptr=None) == LN_EWORKSPACE
    assert call(ws_bytes=need - 1) == LN_EWORKSPACE
    assert call(ws_ptr=ws + 16) == LN_EALIGN                # workspace must be 256-byte aligned
    assert call(dx=x) == LN_EALIAS
    assert call(dB=dA) == LN_EALIAS


def test_grad_ab_validation_and_workspace(lib):
    """The rank-r gradients alone: the workspace query (0 for invalid sizes or T = 0)
    and every argument check ahead of any HIP call."""
    T, K, N, r = 300, 128, 72, 16
    need = lib.lora_nf4_grad_ab_workspace_bytes(T, K, N, r)
    assert need >= 2 * 256  # dA and dB partial sums
    assert lib.lora_nf4_grad_ab_workspace_bytes(0, K, N, r) == 0
    assert lib.lora_nf4_grad_ab_workspace_bytes(T, 65, N, r) == 0
    assert lib.lora_nf4_grad_ab_workspace_bytes(T, K, N, 257) == 0
    assert lib.lora_nf4_grad_ab_workspace_bytes(T, K, N, 12) > 0   # generic rank tiles
    ptrs = [P + (i << 30) for i in range(8)]
    x, g, dy, u, dA, dB, ws = ptrs[:7]

    def call(ws_ptr=ws, ws_bytes=need, rank=r, t=T, **kw):
        a = dict(x=x, g=g, dy=dy, u=u, dA=dA, dB=dB)
        a.update(kw)
        return lib.lora_nf4_grad_ab(t, K, N, rank, 16.0, a["x"], a["g"], a["dy"], a["u"], a["dA"], a["dB"],
                                    ws_ptr, ctypes.c_size_t(ws_bytes), None)

    assert call(dA=None) == LN_EINVAL
    assert call(g=None) == LN_EINVAL
    assert call(rank=0) == LN_ERANK
    assert call(ws_ptr=None) == LN_EWORKSPACE
    assert call(ws_bytes=need - 1) == LN_EWORKSPACE
    assert call(ws_ptr=ws + 16) == LN_EALIGN
    assert call(u=u + 2) == LN_EALIGN
    assert call(dA=x) == LN_EALIAS
    assert call(dB=dA) == LN_EALIAS
    assert call(ws_ptr=g) == LN_EALIAS
    assert call(t=0, dA=dA, dB=dA) == LN_EALIAS  # the empty batch still checks its outputs


def test_bwd_accepts_rank_256_and_any_d_out(lib):
    """1 <= r <= 256 and any d_out >= 1 are valid sizes (the generic kernels take r >
    64 and d_out % 8 != 0): the workspace query, which returns 0 for invalid sizes,
    sizes them, with the rank-r partial sums at the rank's 16-column tiles. No call
    here reaches a launch."""
    for T, K, N, r in ((8, 64, 64, 256), (300, 128, 1, 16), (70, 192, 7, 24), (5, 64, 13, 200)):
        assert lib.lora_nf4_bwd_workspace_bytes(T, K, N, r) > 0, (T, K, N, r)
    assert lib.lora_nf4_bwd_workspace_bytes(8, 64, 64, 257) == 0
    assert lib.lora_nf4_bwd_workspace_bytes(8, 64, 0, 16) == 0
    ptrs = [P + (i << 30) for i in range(12)]
    x, dy, c, a, A, B, u, dx, dA, dB, ws = ptrs[:11]
    assert lib.lora_nf4_bwd(8, 64, 64, 257, 16.0, x, dy, c, a, A, B, u, dx, dA, dB, ws, ctypes.c_size_t(1 << 30),
                            None) == LN_ERANK
    # the partial sums of dA cover 16 rank-tile columns at r = 256: splits x d_in x 256 x 4 bytes
    assert lib.lora_nf4_bwd_workspace_bytes(64, 64, 64, 256) >= 64 * 256 * 4


def test_bwd_noalloc_validation(lib):
    """The no-allocation backward checks its arguments like lora_nf4_bwd and rejects
    shapes whose workspace exceeds its scratch, all before any HIP call."""
    ptrs = [P + (i << 30) for i in range(12)]
    x, dy, c, a, A, B, u, dx, dA, dB = ptrs[:10]

    def call(T=8, K=64, N=64, r=8, **kw):
        args = dict(x=x, dy=dy, c=c, a=a, A=A, B=B, u=u, dx=dx, dA=dA, dB=dB)
        args.update(kw)
        return lib.lora_nf4_bwd_noalloc(T, K, N, r, 16.0, args["x"], args["dy"], args["c"], args["a"], args["A"],
                                        args["B"], args["u"], args["dx"], args["dA"], args["dB"], None)

    assert call(dA=None) == LN_EINVAL
    assert call(r=257) == LN_ERANK
    assert call(K=96) == LN_ESHAPE
    assert call(dx=x + 8) == LN_EALIGN
    # G and U alone of 2^20 tokens at rank 256 are 1 GiB: past the 64 MiB scratch
    assert call(T=1 << 20, K=8192, N=28672, r=256) == LN_EWORKSPACE


def test_merge_validation(lib):
    c, a, A, B, o = (P + (i << 30) for i in range(5))

    def call(K=64, N=16, r=8, alpha=16.0, dt=1, **kw):
        p = dict(c=c, a=a, A=A, B=B, o=o)
        p.update(kw)
        return lib.lora_nf4_merge(K, N, r, alpha, p["c"], p["a"], p["A"], p["B"], dt, p["o"], None)

    assert call(o=None) == LN_EINVAL
    assert call(dt=5) == LN_EINVAL
    assert call(N=0) == LN_EINVAL
    assert call(alpha=float("nan")) == LN_EINVAL
    assert call(r=0) == LN_ERANK
    assert call(r=257) == LN_ERANK
    assert call(K=96) == LN_ESHAPE
    assert call(A=A + 2) == LN_EALIGN
    assert call(o=c + 64) == LN_EALIAS


def test_quantize_validation(lib):
    assert lib.nf4_quantize(None, 0, 4, 64, P, P + (1 << 30), None) == LN_EINVAL
    assert lib.nf4_quantize(P, 2, 4, 64, P + (1 << 30), P + (2 << 30), None) == LN_EINVAL
    assert lib.nf4_quantize(P, 0, 4, 96, P + (1 << 30), P + (2 << 30), None) == LN_ESHAPE
    assert lib.nf4_quantize(P + 4, 0, 4, 64, P + (1 << 30), P + (2 << 30), None) == LN_EALIGN
    assert lib.nf4_quantize(P, 0, 4, 64, P + 64, P + (2 << 30), None) == LN_EALIAS
    assert lib.nf4_dequantize(P, P + (1 << 30), 4, 64, 3, P + (2 << 30), None) == LN_EINVAL
    assert lib.nf4_dequantize(P, P + (1 << 30), 4, 64, 0, P + 16, None) == LN_EALIAS


def test_bwd_multi_validation(lib):
    import ctypes
    n = 3
    base = [P + (i << 30) for i in range(40)]
    arr = lambda vals: (ctypes.c_void_p * len(vals))(*vals)
    d_out = (ctypes.c_int64 * n)(64, 64, 128)

    def call(T=64, K=128, r=16, alpha=16.0, nproj=n, ws_bytes=1 << 30, **kw):
        a = dict(x=base[0], dy=arr(base[1:4]), c=arr(base[4:7]), s=arr(base[7:10]), A=arr(base[10:13]),
                 B=arr(base[13:16]), u=None, dx=base[16], dA=arr(base[17:20]), dB=arr(base[20:23]), ws=base[23],
                 d=d_out)
        a.update(kw)
        return lib.lora_nf4_bwd_multi(T, K, nproj, a["d"], r, alpha, a["x"], a["dy"], a["c"], a["s"], a["A"],
                                      a["B"], a["u"], a["dx"], a["dA"], a["dB"], a["ws"], ws_bytes, None)

    assert call(nproj=0) == LN_EINVAL
    assert call(nproj=9) == LN_EINVAL
    assert call(dy=None) == LN_EINVAL
    assert call(dA=arr([base[17], None, base[19]])) == LN_EINVAL
    assert call(r=0) == LN_ERANK
    assert call(K=96) == LN_ESHAPE
    assert call(d=(ctypes.c_int64 * n)(64, 0, 128)) == LN_EINVAL
    assert call(r=257) == LN_ERANK
    # any d_out >= 1 and r up to 256 are valid (the query returns their workspace)
    assert lib.lora_nf4_bwd_multi_workspace_bytes(64, 128, n, (ctypes.c_int64 * n)(64, 60, 128), 16) > 0
    assert lib.lora_nf4_bwd_multi_workspace_bytes(64, 128, n, d_out, 256) > 0
    assert call(dx=base[16] + 8) == LN_EALIGN
    assert call(ws=None) == LN_EWORKSPACE
    assert call(ws_bytes=16) == LN_EWORKSPACE
    assert call(ws=base[23] + 16) == LN_EALIGN
    assert call(dB=arr([base[20], base[1], base[22]])) == LN_EALIAS  # a dB on top of a dy
    assert call(dx=base[10]) == LN_EALIAS  # dx on top of A[0]
    need = lib.lora_nf4_bwd_multi_workspace_bytes(64, 128, n, d_out, 16)
    assert need > 0
    assert lib.lora_nf4_bwd_multi_workspace_bytes(0, 128, n, d_out, 16) == 0
    assert lib.lora_nf4_bwd_multi_workspace_bytes(64, 96, n, d_out, 16) == 0


def test_adamw_validation(lib):
    p, pb, g, m, v = (P + (i << 30) for i in range(5))

    def call(n=64, step=1, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8, wd=0.0, **kw):
        a = dict(p=p, pb=pb, g=g, m=m, v=v)
        a.update(kw)
        return lib.lora_adamw_step(n, a["p"], a["pb"], a["g"], a["m"], a["v"], step, lr, b1, b2, eps, wd, None)

    assert call(n=0, p=None) == LN_OK  # empty: nothing to do
    assert call(n=-1) == LN_EINVAL
    assert call(step=0) == LN_EINVAL
    assert call(eps=0.0) == LN_EINVAL
    assert call(b1=1.0) == LN_EINVAL
    assert call(b2=-0.1) == LN_EINVAL
    assert call(lr=float("inf")) == LN_EINVAL
    assert call(m=None) == LN_EINVAL
    assert call(v=v + 8) == LN_EALIGN
    assert call(m=g + 64) == LN_EALIAS  # a moment overlapping the gradient
    assert call(pb=p + 128) == LN_EALIAS


def test_adamw8_validation(lib):
    p, pb, g, mq, ms, vq, vs = (P + (i << 30) for i in range(7))

    def call(n=300, step=1, **kw):
        a = dict(p=p, pb=pb, g=g, mq=mq, ms=ms, vq=vq, vs=vs)
        a.update(kw)
        return lib.lora_adamw8_step(n, a["p"], a["pb"], a["g"], a["mq"], a["ms"], a["vq"], a["vs"], step,
                                    1e-3, 0.9, 0.999, 1e-8, 0.0, None)

    assert call(n=0, p=None) == LN_OK
    assert call(step=0) == LN_EINVAL
    assert call(ms=None) == LN_EINVAL
    assert call(vs=vs + 4) == LN_EALIGN
    assert call(ms=mq + 256) == LN_EALIAS   # the scales inside the 300 codes
    assert call(vq=g + 512) == LN_EALIAS    # codes on top of the gradient


def test_bwd_adamw_validation(lib):
    T, K, N, r = 8, 64, 64, 8
    ptrs = [P + (i << 30) for i in range(16)]
    x, dy, c, a, A, B, dx, am, amm, av, bm, bmm, bv, ws = ptrs[:14]
    need = lib.lora_nf4_bwd_workspace_bytes(T, K, N, r)

    def call(T=T, K=K, N=N, r=r, step=1, u=None, ws_bytes=need, **kw):
        d = dict(x=x, dy=dy, c=c, a=a, A=A, B=B, dx=dx, am=am, amm=amm, av=av, bm=bm, bmm=bmm, bv=bv, ws=ws)
        d.update(kw)
        return lib.lora_nf4_bwd_adamw(T, K, N, r, 16.0, d["x"], d["dy"], d["c"], d["a"], d["A"], d["B"], u,
                                      d["dx"], d["am"], d["amm"], d["av"], d["bm"], d["bmm"], d["bv"], step,
                                      1e-3, 0.9, 0.999, 1e-8, 0.0, d["ws"], ctypes.c_size_t(ws_bytes), None)

    assert call(T=0) == LN_EINVAL          # nothing to learn from
    assert call(step=0) == LN_EINVAL
    assert call(bv=None) == LN_EINVAL
    assert call(r=12) == LN_ERANK           # the fused reduction needs r % 8 == 0, r <= 64
    assert call(r=72) == LN_ERANK
    assert call(N=60) == LN_ESHAPE          # ... and d_out % 8 == 0
    assert call(ws=None) == LN_EWORKSPACE
    assert call(ws_bytes=need - 1) == LN_EWORKSPACE
    assert call(amm=am + 8) == LN_EALIGN
    assert call(amm=am + 16) == LN_EALIAS   # A's moments overlapping its master copy
    assert call(A=x) == LN_EALIAS           # the factor on top of x
    assert call(bm=B) == LN_EALIAS


def test_absmax_dq_validation(lib):
    a, q, s, o = (P + (i << 30) for i in range(4))
    assert lib.nf4_absmax_quantize(a, 0, None, None, None, None) == LN_OK
    assert lib.nf4_absmax_quantize(a, -5, q, s, o, None) == LN_EINVAL
    assert lib.nf4_absmax_quantize(None, 300, q, s, o, None) == LN_EINVAL
    assert lib.nf4_absmax_quantize(a, 300, q + 1, s, o, None) == LN_EALIGN
    assert lib.nf4_absmax_quantize(a, 300, q, s, a + 16, None) == LN_EALIAS
    assert lib.nf4_absmax_quantize(a, 300, q, s, s, None) == LN_EALIAS  # scale and offset the same array
    assert lib.nf4_absmax_dequantize(q, s, o, 300, None, None) == LN_EINVAL
    assert lib.nf4_absmax_dequantize(q, s, o, 300, q + 64, None) == LN_EALIAS


def test_rslora_alpha_gives_the_rank_stabilized_scale_exactly(lib):
    import numpy as np
    from oracle import optim
    for alpha in (1.0, 16.0, 32.0, 7.5, 0.3):
        for r in (1, 2, 3, 5, 8, 12, 16, 24, 32, 48, 64, 100, 128, 200, 256):
            a = lib.lora_nf4_rslora_alpha(alpha, r)
            got = np.float32(a) / np.float32(r)  # the library's own s = lora_alpha / r in float32
            want = np.float32(optim.rslora_scale(float(np.float32(alpha)), r))  # alpha crosses as float32
            if r & (r - 1) == 0:
                assert got == want, (alpha, r)
            else:
                assert abs(float(got) - float(want)) <= float(np.spacing(want)), (alpha, r)
    assert lib.lora_nf4_rslora_alpha(32.0, 16) == 128.0  # s = 32 / sqrt(16) = 8
    assert lib.lora_nf4_rslora_alpha(16.0, 0) != lib.lora_nf4_rslora_alpha(16.0, 0)  # NaN
    assert lib.lora_nf4_rslora_alpha(float("inf"), 4) != lib.lora_nf4_rslora_alpha(float("inf"), 4)


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import qlora_linear_amd as q
    with pytest.raises(ValueError):
        q.nf4_quantize(torch.zeros(4, 64))


def test_mfma_probe_validation(lib):
    # rejected before any launch
    assert lib.lora_nf4_mfma_probe(0, P, None) == LN_EINVAL
    assert lib.lora_nf4_mfma_probe(1 << 21, P, None) == LN_EINVAL
    assert lib.lora_nf4_mfma_probe(16, None, None) == LN_EINVAL
    assert lib.lora_nf4_mfma_probe(16, P + 4, None) == LN_EALIGN
