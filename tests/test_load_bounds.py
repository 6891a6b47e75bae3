"""Host-side model of the tiled kernels' buffer-load addressing.

Every load of the tiled kernels goes through a raw buffer descriptor (a base and a
byte count) with a per-lane offset (voffset) and a uniform scalar offset (soffset).
Whether the hardware adds soffset before the range check is not something the
kernels may depend on, so each load must satisfy, for every lane, one of:

* voffset >= range: the lane reads zeros, with or without soffset;
* voffset + soffset + size <= range: the lane reads real bytes inside the range.

and every descriptor must end inside its operand. The functions below restate the
index arithmetic of each kernel's loads (including the run-ahead loads past the
last K-step, whose step index the kernels clamp) and check both conditions over
every lane, load and step, on ragged shapes and on boundary tiles. They mirror the
device code in qlora_linear_amd/csrc (lora_fwd, lora_rw, lora_dx, lora_skinny,
lora_upass); a change to one of those load streams changes its model here.
"""
import numpy as np
import pytest

OOR = 0x7FFFFFF0  # the kernels' out-of-range lane offset
LIM = 0x7FFFFF00  # operands a descriptor covers stay below this many bytes


class Checker:
    def __init__(self):
        self.loads = 0

    def __call__(self, what, operand_bytes, base, rng, voff, soff, size):
        voff = np.asarray(voff, dtype=np.int64).ravel()
        assert base >= 0 and rng >= 0, (what, base, rng)
        assert base + rng <= operand_bytes, f"{what}: descriptor ends past the operand"
        assert rng < LIM and operand_bytes < LIM + 256, what
        assert np.all(voff >= 0) and np.all(voff < 2**32), what
        ok = (voff >= rng) | (voff + soff + size <= rng)
        assert ok.all(), f"{what}: lane offsets {voff[~ok][:4]} + {soff} straddle the range {rng}"
        # a zero-reading lane stays out of range even if soffset is added (no wrap)
        assert np.all((voff < rng) | (voff + soff < 2**32)), what
        self.loads += voff.size


def boundary(n):
    """Tile indices worth checking: first, second, second last, last."""
    return sorted({0, min(1, n - 1), max(n - 2, 0), n - 1})


def lanes(threads):
    tid = np.arange(threads)
    return tid, tid & 63, tid >> 6


# ---- forward tile kernel (lora_fwd.hip), BT x BT tiles, K-steps of 64 -------------
def check_fwd_tiled(chk, T, K, N, r, BT, steps_per, dq):
    kthreads = 2 * BT
    RU = 0 if r == 0 else (16 if r <= 16 else (r + 31) // 32 * 32)
    tid, lane, wave = lanes(kthreads)
    KB, K2 = K // 64, K // 2
    mt, nt = -(-T // BT), -(-N // BT)
    splits = -(-KB // steps_per)
    rows_x_l = [(wave * 4 + q) * 8 + (lane >> 3) for q in range(4)]
    xvoff = np.concatenate([row * K * 2 + (((lane & 7) ^ ((row >> 1) & 7)) * 16) for row in rows_x_l])
    crow, chalf = tid >> 1, tid & 1
    cvoff = crow * K2 + chalf * 16
    svoff = crow * KB * 4
    kaper = (64 * RU // 8 + kthreads - 1) // kthreads
    for tm in boundary(mt):
        for tn in boundary(nt):
            for sp in boundary(splits):
                m0, n0 = tm * BT, tn * BT
                kbeg = sp * steps_per
                nsteps = min(KB - kbeg, steps_per)
                assert nsteps >= 1
                rows_x, rows_w = min(T - m0, BT), min(N - n0, BT)
                for kt in range(nsteps + 2):  # run-ahead: one and two steps past the end
                    k = min(kt, nsteps - 1)
                    chk("fwd x", T * K * 2, (m0 * K + kbeg * 64) * 2, rows_x * K * 2 - kbeg * 128,
                        xvoff, k * 128, 16)
                    if dq:
                        chk("fwd wdq", N * K * 2, (n0 * K + kbeg * 64) * 2, rows_w * K * 2 - kbeg * 128,
                            xvoff, k * 128, 16)
                    else:
                        chk("fwd codes", N * K2, n0 * K2 + kbeg * 32, rows_w * K2 - kbeg * 32, cvoff, k * 32, 16)
                        chk("fwd absmax", N * KB * 4, (n0 * KB + kbeg) * 4, (rows_w * KB - kbeg) * 4,
                            svoff, k * 4, 4)
                    for i in range(kaper):
                        ch = tid + kthreads * i
                        avoff = np.where(ch < 8 * r, ch * 16, OOR)
                        chk("fwd A", K * r * 2, kbeg * 64 * r * 2, (K - kbeg * 64) * r * 2, avoff,
                            k * 64 * r * 2, 16)


# ---- register-dequantizing tile (lora_rw.hip): 256 x 256, 8 waves ---------------------
def check_rw(chk, T, L, ncols, dx, lu):
    kthreads, BT = 512, 256
    tid, lane, wave = lanes(kthreads)
    l32, hh = lane & 31, lane >> 5
    L2, LB = L // 2, L // 64
    last = LB - 1
    xvoff = np.concatenate([(32 * wave + 8 * q + (lane >> 3)) * L * 2
                            + (((lane & 7) ^ (((32 * wave + 8 * q + (lane >> 3)) >> 1) & 7)) << 4)
                            for q in range(4)])
    wrow = 32 * wave + l32
    cvoff = wrow * L2 + 16 * hh
    svoff = wrow * LB * 4
    if dx:
        j = 2 * wave + (lane >> 5)
        pd = lane & 31
        lvoff = j * L * 2 + ((((pd >> 2) ^ (j & 7)) << 4) | ((pd & 3) << 2))
    else:
        lvoff = 256 * wave + 4 * lane
    avoff = ((wave >> 1) * L + lane) * 4
    mt, ct = -(-T // BT), -(-ncols // BT)
    for tm in boundary(mt):
        for tc in boundary(ct):
            m0, c0 = tm * BT, tc * BT
            rows_x, rows_w = min(T - m0, BT), min(ncols - c0, BT)
            for kt in range(LB + 3):
                k = min(kt, last)
                chk("rw x", T * L * 2, m0 * L * 2, rows_x * L * 2, xvoff, k * 128, 16)
                chk("rw codes", ncols * L2, c0 * L2, rows_w * L2, cvoff, k * 32, 16)
                if lu:
                    chk("rw rank slice", L * 32, 0, L * 32, lvoff, k * 128 if dx else k * 2048, 4)
                if dx:
                    chk("rw dX absmax", (ncols // 64) * L * 4, (c0 // 64) * L * 4, 4 * L * 4, avoff,
                        min(kt + 1, last) * 256, 4)
                else:
                    chk("rw absmax", ncols * LB * 4, c0 * LB * 4, rows_w * LB * 4, svoff, k * 4, 4)


# ---- dX tile kernel (lora_dx.hip): per-step descriptors, several projections ---------
def check_dx_tiled(chk, T, K, Ns, r, BT, dq, steps_per=None):
    kthreads = 512 if BT == 256 else 256
    RU = 16 if r <= 16 else (r + 31) // 32 * 32
    tid, lane, wave = lanes(kthreads)
    KB, K2 = K // 64, K // 2
    steps = [-(-n // 64) for n in Ns]
    step_end = np.cumsum(steps).tolist()
    NS_all = step_end[-1]
    if steps_per is None:
        steps_per = NS_all
    assert len(Ns) == 1 or steps_per == NS_all
    splits = -(-NS_all // steps_per)
    e = ((wave[:, None] * 4 + np.arange(4)[None, :]) * 512 + lane[:, None] * 8).ravel()
    n_w, pp = e // BT, (e % BT) // 8
    run = (tid & 3) | (((tid >> 4) & 1) << 2) if BT == 256 else (tid & 3)
    if BT == 256:
        nl = 4 * (((tid >> 2) & 3) | (((tid >> 5) & 3) << 2)) + ((tid >> 7) & 3)
    else:
        nl = 4 * (((tid >> 2) & 3) | (((tid >> 4) & 3) << 2)) + ((tid >> 6) & 3)
    assert nl.max() < 64 and run.max() < BT // 32
    kbper = (RU * 8 + kthreads - 1) // kthreads
    bj, bch = tid >> 3, tid & 7
    mt, kt_tiles = -(-T // BT), -(-K // BT)

    def proj_of(st):
        g = 0
        while st >= step_end[g] and g + 1 < len(Ns):
            g += 1
        return g, (step_end[g - 1] if g else 0), step_end[g]

    for tm in boundary(mt):
        for tk in boundary(kt_tiles):
            for sp in boundary(splits):
                m0, k0 = tm * BT, tk * BT
                rows_t = min(T - m0, BT)
                sbeg = sp * steps_per
                NS = min(NS_all, sbeg + steps_per)
                for st in range(sbeg, NS + 2):
                    g, beg, end = proj_of(st)
                    N = Ns[g]
                    ls = min(st, end - 1) - beg
                    assert 0 <= ls < steps[g]
                    rows = [(wave * 4 + q) * 8 + (lane >> 3) for q in range(4)]
                    yvoff = np.concatenate([row * N * 2 + (((lane & 7) ^ ((row >> 1) & 7)) * 16) for row in rows])
                    chk("dx dY", T * N * 2, (m0 * N + ls * 64) * 2, rows_t * N * 2 - ls * 128, yvoff, 0, 16)
                    if dq:
                        wvoff = n_w * K * 2 + ((pp ^ (4 * (n_w & 3))) * 16)
                        chk("dx wdq", N * K * 2, (k0 + ls * 64 * K) * 2, (N * K - k0 - ls * 64 * K) * 2,
                            wvoff, 0, 16)
                    else:
                        cstep, sstep = ls * 64 * K2, ls * 64 * KB
                        chk("dx codes", N * K2, k0 // 2 + cstep, N * K2 - k0 // 2 - cstep, nl * K2 + run * 16, 0, 16)
                        chk("dx absmax", N * KB * 4, (k0 // 64 + sstep) * 4, (N * KB - k0 // 64 - sstep) * 4,
                            (nl * KB + (run >> 1)) * 4, 0, 4)
                    for i in range(kbper):
                        bvoff = bj * N * 2 + bch * 16 + i * (kthreads // 8) * N * 2
                        chk("dx B", r * N * 2, ls * 128, r * N * 2 - ls * 128, bvoff, 0, 16)


# ---- small-token weight-gradient kernel (lora_skinny.hip) ----------------------------
def check_skinny(chk, T, C, r, vstr, splits):
    TT, BC = 64, 256
    RU = next(ru for ru in (32, 64, 128, 192) if r <= ru)
    tid, lane, wave = lanes(256)
    per = -(-T // splits)
    per = -(-per // TT) * TT
    kvpw = RU // 32
    v_pieces = r // 8
    for cb in boundary(-(-C // BC)):
        c0 = cb * BC
        mvoff = []
        for q in range(8):
            t = wave * 16 + q * 2 + (lane >> 5)
            piece = lane & 31
            lunit = (piece >> 1) ^ (2 * (t & 3))
            mvoff.append(t * C * 2 + (c0 + lunit * 16 + (piece & 1) * 8) * 2)
        mvoff = np.concatenate(mvoff)
        vvoff = []
        for p in range(kvpw):
            piece = wave * kvpw + p
            e = piece * 512 + lane * 8
            vvoff.append(np.where(piece < v_pieces, ((e // r) * vstr + e % r) * 2, OOR))
        vvoff = np.concatenate(vvoff)
        for split in range(splits):
            t_begin = split * per
            t_end = min(T, t_begin + per)
            nrows = t_end - t_begin
            for st in range(max(0, -(-nrows // TT))):
                left = nrows - st * TT
                row0 = t_begin + st * TT
                chk("skinny M", T * C * 2, row0 * C * 2, left * C * 2, mvoff, 0, 16)
                chk("skinny V", ((T - 1) * vstr + r) * 2, row0 * vstr * 2, ((left - 1) * vstr + r) * 2, vvoff, 0, 16)


# ---- U pass (lora_upass.hip): 32 token rows, stages of SC columns ------------------
def check_upass(chk, T, K, R, AR, NS, SC):
    tid, lane, wave = lanes(256)
    nst = K // SC
    rpl, cpr = 1024 // (2 * SC), SC // 8
    kxl, kal, kaw = 32 // rpl // 4, AR // rpl // 4, AR // 4
    assert kxl >= 1 and kal >= 1

    def voff(row):
        return row * K * 2 + (((lane % cpr) ^ (row & 15)) << 4)
    xvo = np.concatenate([voff(rpl * (kxl * wave + q) + lane // cpr) for q in range(kxl)])
    avo = np.concatenate([voff(kaw * wave + rpl * q + lane // cpr) for q in range(kal)])
    for tm in boundary(-(-T // 32)):
        m0 = tm * 32
        rows = min(T - m0, 32)
        rot = (tm % (K // 256)) * (256 // SC)  # workgroup tm starts at 256-column block tm % (K / 256)
        for i in range(nst + NS - 1):  # the ring's run-ahead issues up to step nst + NS - 2
            soff = ((min(i, nst - 1) + rot) % nst) * SC * 2
            chk("upass x", T * K * 2, m0 * K * 2, rows * K * 2, xvo, soff, 16)
            chk("upass A^T", R * K * 2, 0, R * K * 2, avo, soff, 16)


@pytest.mark.parametrize("BT", [128, 256])
@pytest.mark.parametrize("T,K,N,r", [(1000, 4096, 264, 16), (257, 192, 8, 8), (8192, 4160, 4096, 64),
                                     (300, 128, 1032, 32), (65, 64, 520, 48)])
def test_fwd_tiled_loads(BT, T, K, N, r):
    chk = Checker()
    KB = K // 64
    for steps_per in sorted({KB, max(1, -(-KB // 3))}):
        for dq in (False, True):
            check_fwd_tiled(chk, T, K, N, r, BT, steps_per, dq)
    assert chk.loads > 0


@pytest.mark.parametrize("T,L,ncols", [(4096, 4096, 4096), (4100, 256, 264), (5000, 512, 14336)])
def test_rw_forward_loads(T, L, ncols):
    chk = Checker()
    for lu in (False, True):
        check_rw(chk, T, L, ncols, dx=False, lu=lu)
    assert chk.loads > 0


@pytest.mark.parametrize("T,N,K", [(4096, 4096, 4096), (4100, 256, 512), (4353, 1024, 768)])
def test_rw_dx_loads(T, N, K):
    chk = Checker()
    check_rw(chk, T, N, K, dx=True, lu=True)
    assert chk.loads > 0


@pytest.mark.parametrize("BT", [128, 256])
@pytest.mark.parametrize("T,K,Ns,r", [(1000, 4096, [264], 16), (257, 192, [8], 8), (300, 256, [1032], 64),
                                      (513, 640, [4096, 1024, 1024], 16), (129, 128, [72, 8, 200], 48)])
def test_dx_tiled_loads(BT, T, K, Ns, r):
    chk = Checker()
    NS_all = sum(-(-n // 64) for n in Ns)
    for dq in (False, True):
        check_dx_tiled(chk, T, K, Ns, r, BT, dq)
        if len(Ns) == 1 and NS_all > 2:
            check_dx_tiled(chk, T, K, Ns, r, BT, dq, steps_per=-(-NS_all // 3))
    assert chk.loads > 0


@pytest.mark.parametrize("T,C,r,vstr,splits", [(1, 4096, 16, 16, 1), (100, 4104, 16, 48, 2),
                                               (1000, 520, 64, 64, 7), (64, 256, 8, 24, 1), (4000, 4096, 32, 96, 16),
                                               (8200, 4096, 192, 192, 13), (300, 768, 96, 96, 3)])
def test_skinny_loads(T, C, r, vstr, splits):
    chk = Checker()
    check_skinny(chk, T, C, r, vstr, splits)
    assert chk.loads > 0


@pytest.mark.parametrize("T,K,R,AR,NS,SC", [(1000, 4096, 48, 64, 3, 256), (33, 256, 16, 16, 4, 256),
                                             (8192, 512, 64, 64, 3, 256), (70, 768, 24, 32, 4, 256),
                                             (1000, 4096, 192, 192, 2, 128), (33, 256, 96, 128, 2, 128),
                                             (4100, 1024, 256, 256, 2, 128), (70, 768, 144, 192, 2, 128)])
def test_upass_loads(T, K, R, AR, NS, SC):
    chk = Checker()
    check_upass(chk, T, K, R, AR, NS, SC)
    assert chk.loads > 0


def test_checker_catches_soffset_dependence():
    """The check fails for the pattern it guards against: rows past the end held in
    the scalar offset (a lane offset in range plus a step that leaves it)."""
    chk = Checker()
    with pytest.raises(AssertionError):
        chk("planted", 4096, 0, 4096, np.array([4000]), 128, 16)
    chk("fine", 4096, 0, 4096, np.array([4096, 3968]), 112, 16)
