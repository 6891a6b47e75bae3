#!/usr/bin/env python3
"""Benchmark of the fused NF4-LoRA linear, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--fuse] [--no-cpu-baseline]

One step = lora_nf4_fwd + lora_nf4_bwd (dX, dA, dB; U reused from the forward)
over every projection of the workload, on seeded synthetic bf16 inputs already
resident in HBM (the NF4 weights are quantized once, before timing, as at model
load). Default workload: the Llama-3-8B q_proj projection, T = 8192 tokens
(batch 4 x seq 2048), d_in = d_out = 4096, r = 16, alpha = 16.

Prints ONE JSON line. `value` is algorithmic TFLOP/s of the whole step:
4 T d_in d_out + 6 T r (d_in + d_out) per projection (no dequantization, no
padding, no redundant in-tile work counted). `roofline` describes the forward
kernel (one launch per lora_nf4_fwd call, timed with HIP events on the stream it
runs on); `cpu_baseline` times the CPU fp64 oracle on a bounded token sample of
the same projection; `small_tokens` times forward and backward of the largest
projection at a few tokens (the weight-streaming kernels), where the bound is
reading the packed weight from HBM; `medium_tokens` does the same at a few hundred
tokens (tiled kernels on a grid of 128 x 128 tiles); `merge` times lora_nf4_merge of that
projection (the 16-bit export, also HBM-bound); `train_step` times the AdamW step of A and B and the
absmax double quantization; `multi_projection` times Llama-3-8B q/k/v (r = 64, one x) as one
lora_nf4_fwd_multi + lora_nf4_bwd_multi against separate calls. With --fuse, projections that read the same
activations in a transformer layer (q/k/v, gate/up) share one x, run their
forward as one lora_nf4_fwd_multi launch and their backward as one
lora_nf4_bwd_multi call (dX summed over the group); the FLOPs counted are unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "fused NF4-LoRA linear fwd+bwd TFLOP/s & tokens/s, % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 FLOP/clk x 2.4 GHz (published: 2.5 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_lora_fwd_kernel_llama3-8b-q_proj.json")
FWD_SOURCES = ("qlora_linear_amd/csrc/lora_fwd.hip", "qlora_linear_amd/csrc/nf4_quant.hip",
               "qlora_linear_amd/csrc/device_common.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3-8b-q_proj",
                    help="one of: " + ", ".join(w.name for w in synth.WORKLOADS))
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the q/k/v multi-projection leg (fused against separate calls)")
    ap.add_argument("--fuse", action="store_true",
                    help="q/k/v and gate/up share x and run one multi-projection forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--small-tokens", type=int, default=16,
                    help="token count of the weight-bound measurement (0: skip)")
    ap.add_argument("--medium-tokens", type=int, default=512,
                    help="token count of the medium-size measurement (0: skip)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run under rocprofv3 --pmc: one plain copy of COPY_BYTES (calibration), "
                         "then --steps fwd+bwd steps; prints nothing else")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output dirs (FETCH_SIZE, WRITE_SIZE runs of "
                         "--counter-pass) into the traffic record used by the roofline")
    return ap.parse_args()


COPY_BYTES = 256 << 20  # calibration copy: reads and writes exactly this many bytes


def fwd_source_sha() -> str:
    h = hashlib.sha256()
    for rel in FWD_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 counter runs, or
    None when they were taken on a different version of the forward kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != fwd_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def counter_dispatches(d: str, counter: str) -> list:
    """(dispatch id, kernel name, value summed over XCDs) of `counter` from a rocprofv3 csv run,
    in dispatch order."""
    import csv
    import glob
    import collections
    per = collections.defaultdict(float)
    names = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                did = int(r["Dispatch_Id"])
                per[did] += float(r["Counter_Value"])
                names[did] = r["Kernel_Name"]
    return [(did, names[did], per[did]) for did in sorted(per)]


def forward_kib(disp: list) -> tuple:
    """Mean counter value (KiB) per forward call and per other kernel. From 1024 tokens a
    forward call is two launches, the weight's dequantization and the tile kernel
    (lora_fwd_kernel); the backward's input gradient likewise pairs it with the dX tile
    kernel (lora_dx_kernel)."""
    import collections
    fwd, other = [], collections.defaultdict(list)
    prev = None
    for _, name, v in disp:
        after_dq = prev is not None and "nf4_dequantize_kernel" in prev[0]
        if "lora_fwd_kernel" in name:
            fwd.append(prev[1] + v if after_dq else v)
        elif "lora_dx_kernel" in name and after_dq:
            other["lora_dx (nf4_dequantize_kernel + lora_dx_kernel)"].append(prev[1] + v)
        elif "nf4_dequantize" not in name:
            for key in ("lora_dx_kernel", "skinny_partial_kernel", "skinny_reduce2_kernel", "MulFunctor"):
                if key in name:
                    other[key].append(v)
        prev = (name, v)
    if not fwd:
        raise SystemExit("no dispatch of lora_fwd_kernel in the counter data")
    return sum(fwd) / len(fwd), {k: sum(v) / len(v) for k, v in other.items()}


def ingest_counters(fetch_dir: str, write_dir: str):
    fetch_fwd, fetch_other = forward_kib(counter_dispatches(fetch_dir, "FETCH_SIZE"))
    write_fwd, write_other = forward_kib(counter_dispatches(write_dir, "WRITE_SIZE"))
    copy_key = "MulFunctor"  # the calibration copy: torch.mul(src, 1.0, out=dst)
    if copy_key not in fetch_other or copy_key not in write_other:
        raise SystemExit("no dispatch of the calibration copy in the counter data")
    cal_f = (COPY_BYTES / 1024) / fetch_other[copy_key]
    cal_w = (COPY_BYTES / 1024) / write_other[copy_key]
    rec = {"kernel": "lora_fwd (nf4_dequantize_kernel + lora_fwd_kernel at large token counts)",
           "workload": "llama3-8b-q_proj",
           "commands": ["rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR -o run --output-format csv -- "
                        "python3 bench.py --counter-pass --steps 2",
                        "rocprofv3 --pmc WRITE_SIZE -d WRITE_DIR -o run --output-format csv -- "
                        "python3 bench.py --counter-pass --steps 2",
                        "python3 bench.py --ingest-counters FETCH_DIR WRITE_DIR"],
           "source_sha": fwd_source_sha(),
           "fetch_kib_raw": fetch_fwd, "write_kib_raw": write_fwd,
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": cal_f, "write_factor": cal_w}}
    rec["hbm_bytes_per_launch"] = round(1024 * (rec["fetch_kib_raw"] * cal_f + rec["write_kib_raw"] * cal_w))
    rec["other_kernels_hbm_bytes_per_launch"] = {
        k: round(1024 * (fetch_other[k] * cal_f + write_other.get(k, 0.0) * cal_w))
        for k in fetch_other if k != copy_key}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(w: synth.Workload, target_s: float):
    """The oracle as it stands, fwd + bwd of the workload's first projection on a
    token sample sized to take about target_s seconds on this host."""
    from oracle import lora as olora
    from oracle import nf4 as onf4
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    p = w.projections[0]
    inp = synth.projection_inputs(w, 0)
    codes, absmax = onf4.quantize(synth.bf16_bits_to_f32(inp["W"]))   # one-time, not timed
    x_all, dy_all = olora.bf16_to_f64(inp["x"]), olora.bf16_to_f64(inp["dY"])
    A, B = olora.bf16_to_f64(inp["A"]), olora.bf16_to_f64(inp["B"])

    def step(tok):
        D = onf4.dequantize_exact(codes, absmax)
        olora.forward(x_all[:tok], D, A, B, w.alpha, w.r)
        olora.backward(x_all[:tok], dy_all[:tok], D, A, B, w.alpha, w.r)

    tok = min(256, w.tokens)
    t0 = time.perf_counter()
    step(tok)
    dt = time.perf_counter() - t0
    tok = int(min(w.tokens, max(64, tok * target_s / max(dt, 1e-3))))
    tok = max(64, (tok // 64) * 64)
    # the whole workload may take well under target_s on a fast host: repeat it
    reps = max(1, min(20, int(target_s / max(dt * tok / min(256, w.tokens), 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        step(tok)
    dt = (time.perf_counter() - t0) / reps
    fl = synth.flops(tok, p.d_in, p.d_out, w.r)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds_per_pass": round(dt, 3), "passes": reps,
            "tokens_per_s": round(tok / dt, 1),
            "sample": f"{p.name} {p.d_in}->{p.d_out} r={w.r}, {tok} of {w.tokens} tokens"
                      f"{f' x {reps} passes' if reps > 1 else ''}, "
                      f"fp64 NumPy fwd+bwd incl. dequantization"}


def time_fwd_bwd(lib, q, torch, d, w, tokens, sp, reps):
    """Forward and backward of one projection on the first `tokens` rows of the
    resident x and dY, back to back through the C ABI with preallocated buffers;
    HIP events on the stream bracket `reps` calls of each. Returns (T, K, N, r,
    forward us, backward us)."""
    p = d["p"]
    T, K, N, r = min(tokens, w.tokens), p.d_in, p.d_out, w.r
    x, dy = d["x"][:T], d["dY"][:T]
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((T, r), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((K, r), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((r, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(q.lora_nf4_bwd_workspace_bytes(T, K, N, r), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(q.lora_nf4_fwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")

    def fwd():
        st = lib.lora_nf4_fwd(T, K, N, r, w.alpha, x.data_ptr(), d["codes"].data_ptr(),
                              d["absmax"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(),
                              y.data_ptr(), u.data_ptr(), fws.data_ptr(), fws.numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_fwd", st)

    def bwd():
        st = lib.lora_nf4_bwd(T, K, N, r, w.alpha, x.data_ptr(), dy.data_ptr(), d["codes"].data_ptr(),
                              d["absmax"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(), u.data_ptr(),
                              dx.data_ptr(), dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_bwd", st)

    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1000.0 / reps
    return T, K, N, r, res["fwd"], res["bwd"]


def small_token_run(lib, q, torch, d, w, tokens, sp, reps=50):
    """A few tokens: the weight-streaming kernels, bound by reading the packed weight."""
    T, K, N, r, f_us, b_us = time_fwd_bwd(lib, q, torch, d, w, tokens, sp, reps)
    res = {"fwd": f_us, "bwd": b_us}
    wbytes = N * K // 2 + N * (K // 64) * 4  # packed codes + fp32 absmax, read once per call
    return {"tokens": T, "projection": f"{d['p'].name} {K}->{N}", "r": r,
            "fwd_us": round(res["fwd"], 2), "bwd_us": round(res["bwd"], 2),
            "weight_bytes": wbytes, "bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "fwd_weight_GBps": round(wbytes / res["fwd"] / 1e3, 1),
            "fwd_frac": round(wbytes / res["fwd"] / 1e3 / PEAK_HBM_GBS, 4),
            "bwd_weight_GBps": round(wbytes / res["bwd"] / 1e3, 1)}


def medium_token_run(lib, q, torch, d, w, tokens, sp, reps=50):
    """Hundreds of tokens: the tiled kernels on a grid too small for 256 x 256 tiles
    to fill the GPU (the launcher then takes 128 x 128 tiles). Algorithmic TFLOP/s
    of forward and backward (same per-token FLOPs as the step)."""
    T, K, N, r, f_us, b_us = time_fwd_bwd(lib, q, torch, d, w, tokens, sp, reps)
    f_fl = 2 * T * K * N + 2 * T * r * (K + N)
    b_fl = 2 * T * K * N + 4 * T * r * (K + N)
    return {"tokens": T, "projection": f"{d['p'].name} {K}->{N}", "r": r,
            "fwd_us": round(f_us, 2), "bwd_us": round(b_us, 2), "bound": "mfma",
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "fwd_TFLOPs": round(f_fl / f_us / 1e6, 1), "bwd_TFLOPs": round(b_fl / b_us / 1e6, 1)}


def merge_run(lib, q, torch, d, w, sp, reps=20):
    """lora_nf4_merge of one projection into a preallocated bf16 [d_out, d_in], HIP
    events around `reps` back-to-back C-ABI calls; bytes = packed weight in + bf16 out."""
    p = d["p"]
    K, N, r = p.d_in, p.d_out, w.r
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")

    def call():
        st = lib.lora_nf4_merge(K, N, r, w.alpha, d["codes"].data_ptr(), d["absmax"].data_ptr(),
                                d["A"].data_ptr(), d["B"].data_ptr(), 1, out.data_ptr(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_merge", st)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    nbytes = N * K // 2 + N * (K // 64) * 4 + N * K * 2
    del out
    return {"projection": f"{p.name} {K}->{N}", "r": r, "us": round(us, 2), "bytes": nbytes,
            "bound": "hbm", "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}


def train_step_run(lib, q, torch, d, w, sp, reps=50):
    """The training-step companions on one projection, HIP events around `reps`
    back-to-back C-ABI calls each:
      adamw      lora_adamw_step over A and B (float32 master, bf16 copy, bf16
                 gradient and moments); bytes = 4 + 2 + 2 + 2*2 + 2*2 read/written
                 per element = 16 (master in and out, copy out, gradient in, m, v in
                 and out);
      absmax_dq  nf4_absmax_quantize of the projection's block scales; bytes = 4 in
                 + 1 out per scale (+ 8 per 256)."""
    p = d["p"]
    K, N, r = p.d_in, p.d_out, w.r
    n = K * r + r * N
    master = torch.zeros(n, dtype=torch.float32, device="cuda")
    copy = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    grad = torch.full((n,), 1e-3, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    na = d["absmax"].numel()
    dq_q = torch.empty(na, dtype=torch.uint8, device="cuda")
    dq_s = torch.empty((na + 255) // 256, dtype=torch.float32, device="cuda")
    dq_o = torch.empty_like(dq_s)

    def adamw(step):
        st = lib.lora_adamw_step(n, master.data_ptr(), copy.data_ptr(), grad.data_ptr(), m.data_ptr(),
                                 v.data_ptr(), step, 1e-4, 0.9, 0.999, 1e-8, 0.01, sp)
        if st != 0:
            raise q.LoraNF4Error("lora_adamw_step", st)

    def dq(step):
        st = lib.nf4_absmax_quantize(d["absmax"].data_ptr(), na, dq_q.data_ptr(), dq_s.data_ptr(),
                                     dq_o.data_ptr(), sp)
        if st != 0:
            raise q.LoraNF4Error("nf4_absmax_quantize", st)

    out = {}
    stream = torch.cuda.current_stream()
    for name, fn, nbytes in (("adamw", adamw, 16 * n), ("absmax_dq", dq, 5 * na + 8 * dq_s.numel())):
        for i in range(3):
            fn(i + 1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i + 4)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / reps
        out[name] = {"elements": n if name == "adamw" else na, "us": round(us, 2), "bytes": nbytes,
                     "bound": "hbm", "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
    out["projection"] = f"{p.name} {K}->{N}"
    del master, copy, grad, m, v, dq_q, dq_s, dq_o
    return out


def multi_projection_run(lib, q, torch, sp, reps=10):
    """Llama-3-8B q/k/v (4096 -> 4096, 1024, 1024) at 8192 tokens, r = 64, sharing one
    x: one fwd + bwd of the three projections as lora_nf4_fwd_multi + lora_nf4_bwd_multi
    (dX summed over them) against three lora_nf4_fwd + three lora_nf4_bwd calls (three
    separate dX, not summed). HIP events around `reps` back-to-back steps each."""
    w = next(x for x in synth.WORKLOADS if x.name == "llama3-8b-attn-r64")
    T, r = w.tokens, w.r
    ins = [synth.projection_inputs(w, g, tensors=("W", "A", "B", "dY") if g else ("x", "W", "A", "B", "dY"))
           for g in range(3)]
    x = to_dev_bf16(ins[0]["x"])
    K = w.projections[0].d_in
    Ns = [w.projections[g].d_out for g in range(3)]
    codes, absmax, A, B, dy = [], [], [], [], []
    for inp in ins:
        c, a = q.nf4_quantize(to_dev_bf16(inp["W"]))
        codes.append(c), absmax.append(a)
        A.append(to_dev_bf16(inp["A"])), B.append(to_dev_bf16(inp["B"])), dy.append(to_dev_bf16(inp["dY"]))
    ys, us = q.lora_nf4_fwd_multi(x, codes, absmax, A, B, w.alpha)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dxs = [torch.empty((T, K), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    dAs = [torch.empty((K, r), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    dBs = [torch.empty((r, N), dtype=torch.bfloat16, device="cuda") for N in Ns]
    wsm = torch.empty(max(q.lora_nf4_bwd_multi_workspace_bytes(T, K, Ns, r), 256), dtype=torch.uint8, device="cuda")
    wss = [torch.empty(max(q.lora_nf4_bwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")
           for N in Ns]
    fwsm = torch.empty(max(q.lora_nf4_fwd_multi_workspace_bytes(T, K, Ns, r), 256), dtype=torch.uint8,
                       device="cuda")
    fwss = [torch.empty(max(q.lora_nf4_fwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")
            for N in Ns]
    import ctypes
    arr = lambda ts: (ctypes.c_void_p * 3)(*[t.data_ptr() for t in ts])
    cv = lambda a: ctypes.cast(a, ctypes.c_void_p)
    d_out = (ctypes.c_int64 * 3)(*Ns)
    keep = dict(c=arr(codes), a=arr(absmax), A=arr(A), B=arr(B), y=arr(ys), u=arr(us), dy=arr(dy), dA=arr(dAs),
                dB=arr(dBs))

    def fused():
        st = lib.lora_nf4_fwd_multi(T, K, 3, cv(d_out), r, w.alpha, x.data_ptr(), cv(keep["c"]), cv(keep["a"]),
                                    cv(keep["A"]), cv(keep["B"]), cv(keep["y"]), cv(keep["u"]), fwsm.data_ptr(),
                                    fwsm.numel(), sp)
        st = st or lib.lora_nf4_bwd_multi(T, K, 3, cv(d_out), r, w.alpha, x.data_ptr(), cv(keep["dy"]),
                                          cv(keep["c"]), cv(keep["a"]), cv(keep["A"]), cv(keep["B"]),
                                          cv(keep["u"]), dx.data_ptr(), cv(keep["dA"]), cv(keep["dB"]),
                                          wsm.data_ptr(), wsm.numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_fwd_multi / lora_nf4_bwd_multi", st)

    def separate():
        for g in range(3):
            st = lib.lora_nf4_fwd(T, K, Ns[g], r, w.alpha, x.data_ptr(), codes[g].data_ptr(), absmax[g].data_ptr(),
                                  A[g].data_ptr(), B[g].data_ptr(), ys[g].data_ptr(), us[g].data_ptr(),
                                  fwss[g].data_ptr(), fwss[g].numel(), sp)
            st = st or lib.lora_nf4_bwd(T, K, Ns[g], r, w.alpha, x.data_ptr(), dy[g].data_ptr(),
                                        codes[g].data_ptr(), absmax[g].data_ptr(), A[g].data_ptr(),
                                        B[g].data_ptr(), us[g].data_ptr(), dxs[g].data_ptr(), dAs[g].data_ptr(),
                                        dBs[g].data_ptr(), wss[g].data_ptr(), wss[g].numel(), sp)
            if st != 0:
                raise q.LoraNF4Error("lora_nf4_fwd / lora_nf4_bwd", st)

    out = {"workload": "llama3-8b-attn-r64 q_proj + k_proj + v_proj (one x)", "tokens": T, "r": r}
    stream = torch.cuda.current_stream()
    flops = sum(synth.flops(T, K, N, r) for N in Ns)
    for name, fn in (("fused", fused), ("separate", separate)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{name}_ms"] = round(ms, 4)
        out[f"{name}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
    out["note"] = "separate leaves three dX arrays unsummed; fused returns their sum"
    del x, codes, absmax, A, B, dy, ys, us, dx, dxs, dAs, dBs, wsm, wss
    return out


def to_dev_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus N with N > 1 is not supported "
              "(the path shards over tokens with one all-reduce of dA/dB, which is not built here).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import qlora_linear_amd as q

    w = next((x for x in synth.WORKLOADS if x.name == args.workload), None)
    if w is None:
        sys.exit(f"unknown workload {args.workload}")
    q.library()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    # resident inputs, NF4 weights quantized once (model load), workspaces preallocated
    projs = []
    for pi, p in enumerate(w.projections):
        inp = synth.projection_inputs(w, pi)
        x, W, A, B, dY = (to_dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
        codes, absmax = q.nf4_quantize(W)
        del W
        T, K, N, r = w.tokens, p.d_in, p.d_out, w.r
        ws = torch.empty(q.lora_nf4_bwd_workspace_bytes(T, K, N, r), dtype=torch.uint8, device="cuda")
        fws = torch.empty(max(q.lora_nf4_fwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")
        projs.append(dict(p=p, x=x, A=A, B=B, dY=dY, codes=codes, absmax=absmax, ws=ws, fws=fws,
                          y=torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
                          u=torch.empty((T, r), dtype=torch.bfloat16, device="cuda"),
                          dx=torch.empty((T, K), dtype=torch.bfloat16, device="cuda"),
                          dA=torch.empty((K, r), dtype=torch.bfloat16, device="cuda"),
                          dB=torch.empty((r, N), dtype=torch.bfloat16, device="cuda")))
    lib = q.library()
    sp = stream.cuda_stream

    # forward units: one projection each, or (--fuse) the groups that share x
    units, seen = [], {}
    for j, d in enumerate(projs):
        key = {"q_proj": "qkv", "k_proj": "qkv", "v_proj": "qkv", "gate_proj": "gu",
               "up_proj": "gu"}.get(d["p"].name) if args.fuse else None
        if key is not None and key in seen:
            units[seen[key]].append(j)
            d["x"] = projs[units[seen[key]][0]]["x"]  # the group reads one x
        else:
            if key is not None:
                seen[key] = len(units)
            units.append([j])
    import ctypes
    multi_args = {}
    for ui, un in enumerate(units):
        if len(un) > 1:
            arr = lambda key: (ctypes.c_void_p * len(un))(*[projs[j][key].data_ptr() for j in un])
            d_out = [projs[j]["p"].d_out for j in un]
            nb = q.lora_nf4_bwd_multi_workspace_bytes(w.tokens, projs[un[0]]["p"].d_in, d_out, w.r)
            nf = q.lora_nf4_fwd_multi_workspace_bytes(w.tokens, projs[un[0]]["p"].d_in, d_out, w.r)
            multi_args[ui] = dict(d_out=(ctypes.c_int64 * len(un))(*d_out),
                                  codes=arr("codes"), absmax=arr("absmax"), A=arr("A"), B=arr("B"),
                                  y=arr("y"), u=arr("u"), dy=arr("dY"), dA=arr("dA"), dB=arr("dB"),
                                  ws=torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda"),
                                  fws=torch.empty(max(nf, 256), dtype=torch.uint8, device="cuda"))
            for j in un:  # the group's per-projection backward workspaces are not used
                projs[j]["ws"] = torch.empty(0, dtype=torch.uint8, device="cuda")
    torch.cuda.empty_cache()

    def fwd(d):
        p = d["p"]
        st = lib.lora_nf4_fwd(w.tokens, p.d_in, p.d_out, w.r, w.alpha, d["x"].data_ptr(),
                              d["codes"].data_ptr(), d["absmax"].data_ptr(), d["A"].data_ptr(),
                              d["B"].data_ptr(), d["y"].data_ptr(), d["u"].data_ptr(), d["fws"].data_ptr(),
                              d["fws"].numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_fwd", st)

    def bwd(d):
        p = d["p"]
        st = lib.lora_nf4_bwd(w.tokens, p.d_in, p.d_out, w.r, w.alpha, d["x"].data_ptr(),
                              d["dY"].data_ptr(), d["codes"].data_ptr(), d["absmax"].data_ptr(),
                              d["A"].data_ptr(), d["B"].data_ptr(), d["u"].data_ptr(),
                              d["dx"].data_ptr(), d["dA"].data_ptr(), d["dB"].data_ptr(),
                              d["ws"].data_ptr(), d["ws"].numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_bwd", st)

    def fwd_unit(ui):
        un = units[ui]
        if len(un) == 1:
            return fwd(projs[un[0]])
        m, d0 = multi_args[ui], projs[un[0]]
        cv = lambda a: ctypes.cast(a, ctypes.c_void_p)
        st = lib.lora_nf4_fwd_multi(w.tokens, d0["p"].d_in, len(un), cv(m["d_out"]), w.r, w.alpha,
                                    d0["x"].data_ptr(), cv(m["codes"]), cv(m["absmax"]), cv(m["A"]),
                                    cv(m["B"]), cv(m["y"]), cv(m["u"]), m["fws"].data_ptr(), m["fws"].numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_fwd_multi", st)

    def bwd_unit(ui):
        un = units[ui]
        if len(un) == 1:
            return bwd(projs[un[0]])
        m, d0 = multi_args[ui], projs[un[0]]
        cv = lambda a: ctypes.cast(a, ctypes.c_void_p)
        st = lib.lora_nf4_bwd_multi(w.tokens, d0["p"].d_in, len(un), cv(m["d_out"]), w.r, w.alpha,
                                    d0["x"].data_ptr(), cv(m["dy"]), cv(m["codes"]), cv(m["absmax"]),
                                    cv(m["A"]), cv(m["B"]), cv(m["u"]), d0["dx"].data_ptr(), cv(m["dA"]),
                                    cv(m["dB"]), m["ws"].data_ptr(), m["ws"].numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_bwd_multi", st)

    def step_all():
        for ui, un in enumerate(units):
            fwd_unit(ui)
            bwd_unit(ui)

    if args.counter_pass:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # plain copy of known size: calibrates the counters
        torch.cuda.synchronize()
        for _ in range(args.steps):
            step_all()
        torch.cuda.synchronize()
        return

    for _ in range(args.warmup):
        step_all()
    torch.cuda.synchronize()

    # events around every forward launch (one kernel each; one per unit) and the
    # backward calls of the unit's projections
    nev = args.steps * len(units)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nev)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    i = 0
    for _ in range(args.steps):
        for ui, un in enumerate(units):
            ev[i][0].record(stream)
            fwd_unit(ui)
            ev[i][1].record(stream)
            bwd_unit(ui)
            ev[i][2].record(stream)
            i += 1
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    flops_step = sum(synth.flops(w.tokens, d["p"].d_in, d["p"].d_out, w.r) for d in projs)
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    tokens_s = w.tokens / (ms_step * 1e-3)

    # forward launch of the unit holding the largest projection: average duration
    big = max(range(len(projs)), key=lambda j: projs[j]["p"].d_in * projs[j]["p"].d_out)
    bu = next(ui for ui, un in enumerate(units) if big in un)
    fwd_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(nev) if k % len(units) == bu]
    bwd_ms = [ev[k][1].elapsed_time(ev[k][2]) for k in range(nev) if k % len(units) == bu]
    pb = projs[big]["p"]
    T, K, N, r = w.tokens, pb.d_in, pb.d_out, w.r
    fwd_flops = sum(2 * T * projs[j]["p"].d_in * projs[j]["p"].d_out
                    + 2 * T * r * (projs[j]["p"].d_in + projs[j]["p"].d_out) for j in units[bu])
    unit_label = " + ".join(f"{projs[j]['p'].name} {projs[j]['p'].d_in}->{projs[j]['p'].d_out}"
                            for j in units[bu])
    fwd_avg = float(np.mean(fwd_ms))
    achieved = fwd_flops / (fwd_avg * 1e-3) / 1e12
    traffic = measured_traffic()

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq,
                   "r": w.r, "alpha": w.alpha,
                   "projections": [f"{d['p'].name} {d['p'].d_in}->{d['p'].d_out}" for d in projs],
                   "weights": "NF4 blocksize 64, fp32 absmax", "parallelism": "single GPU",
                   "fused_forward": [[projs[j]["p"].name for j in un] for un in units if len(un) > 1],
                   "fused_backward": [[projs[j]["p"].name for j in un] for un in units if len(un) > 1]},
        "tokens_per_s": round(tokens_s, 1),
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_avg, 4),
        "bwd_ms": round(float(np.mean(bwd_ms)), 4),
        "host_wall_s": round(wall, 4),
        "roofline": {"kernel": ("lora_fwd (nf4_dequantize_kernel + lora_fwd_kernel)"
                                if q.lora_nf4_fwd_workspace_bytes(T, K, N, r) >= K * N * 2
                                else "lora_fwd_kernel"), "projection": unit_label,
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if args.small_tokens > 0:
        out["small_tokens"] = small_token_run(lib, q, torch, projs[big], w, args.small_tokens, sp)
    if args.medium_tokens > 0:
        out["medium_tokens"] = medium_token_run(lib, q, torch, projs[big], w, args.medium_tokens, sp)
    out["merge"] = merge_run(lib, q, torch, projs[big], w, sp)
    out["train_step"] = train_step_run(lib, q, torch, projs[big], w, sp)
    if not args.no_multi:
        out["multi_projection"] = multi_projection_run(lib, q, torch, sp)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
