"""Host logic of bench.py: turning per-dispatch counter rows into the forward's
traffic (no GPU). From 1024 tokens a forward call is the weight's dequantization
followed by the tile kernel; the backward's input gradient pairs the same
dequantization with the dX tile kernel and must not be counted as forward."""
import bench


def _rows():
    # (dispatch id, kernel name, KiB): copy, then two steps of fwd (dequant + tile),
    # bwd (dequant + dX tile kernel, rank-r kernels)
    out = [(1, "void at::native::MulFunctor<float>", 512.0)]
    did = 2
    for _ in range(2):
        for name, v in (("void lnf4::nf4_dequantize_kernel<true>(unsigned int const*)", 40.0),
                        ("void lnf4::lora_fwd_kernel<256, 16, 16, true>(int)", 100.0),
                        ("void lnf4::nf4_dequantize_kernel<true>(unsigned int const*)", 45.0),
                        ("void lnf4::lora_dx_kernel<256, 16, 16, false, true>(int)", 110.0),
                        ("void lnf4::skinny_partial_kernel<32>(int)", 30.0),
                        ("lnf4::skinny_reduce2_kernel(float const*)", 2.0)):
            out.append((did, name, v))
            did += 1
    return out


def test_forward_traffic_pairs_dequantization_with_its_tile_kernel():
    fwd, other = bench.forward_kib(_rows())
    assert fwd == 140.0                                  # 40 + 100, not the dX tile kernel
    assert other["lora_dx (nf4_dequantize_kernel + lora_dx_kernel)"] == 155.0
    assert other["skinny_partial_kernel"] == 30.0 and other["skinny_reduce2_kernel"] == 2.0
    assert other["MulFunctor"] == 512.0


def test_forward_traffic_single_launch_below_1024_tokens():
    rows = [(1, "MulFunctor", 4.0), (2, "void lnf4::lora_fwd_kernel<128, 16, 16, false>(int)", 70.0),
            (3, "void lnf4::lora_dx_kernel<128, 16, 16, false>(int)", 60.0),
            (4, "void lnf4::lora_fwd_kernel<128, 16, 16, false>(int)", 72.0)]
    fwd, other = bench.forward_kib(rows)
    assert fwd == 71.0 and other["lora_dx_kernel"] == 60.0


def test_register_path_pairs_the_transposition_with_dx():
    """Default mode: the forward is one register-dequantizing launch; dX is the packed
    weight's transposition followed by the register-dequantizing dX kernel."""
    rows = [(1, "MulFunctor", 8.0)]
    did = 2
    for _ in range(3):
        for name, v in (("void lnf4::lora_fwd_rw_kernel<16, true>(int)", 90.0),
                        ("lnf4::nf4_transpose_kernel(unsigned int const*)", 12.0),
                        ("lnf4::lora_dx_rw_kernel(int)", 95.0),
                        ("void lnf4::skinny_partial_kernel<32>(int)", 30.0)):
            rows.append((did, name, v))
            did += 1
    fwd, other = bench.forward_kib(rows)
    assert fwd == 90.0
    assert other["lora_dx (nf4_transpose_kernel + lora_dx_rw_kernel)"] == 107.0
    assert "lora_dx_rw_kernel" not in other and other["skinny_partial_kernel"] == 30.0
