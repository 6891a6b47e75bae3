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
the same projection; `small_tokens` times forward and backward of the Llama-3-70B
gate projection (8192 -> 28672, 132 MB of packed weight) at 1 and 16 tokens (the
weight-streaming kernels, bound by reading the packed weight), back to back and
cold (after a 1 GiB read), and `small_tokens_headline_projection` the headline
projection at a few tokens; `medium_tokens` does the same at a few hundred
tokens (tiled kernels on a grid of 128 x 128 tiles); `merge` times lora_nf4_merge of that
projection (the 16-bit export, also HBM-bound); `rank_r_gradients` times the backward's
rank-r step alone (lora_nf4_grad_ab, bound by reading x and dY); `train_step` times the AdamW step of A and B and the
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_lora_fwd_rw_kernel_llama3-8b-q_proj.json")
# (build.py holds the compile flags, among them the tile file's scheduling strategy)
FWD_SOURCES = ("qlora_linear_amd/csrc/lora_rw.hip", "qlora_linear_amd/csrc/lora_fwd.hip",
               "qlora_linear_amd/csrc/nf4_quant.hip", "qlora_linear_amd/csrc/device_common.h",
               "qlora_linear_amd/build.py")
# tile kernels of the forward and of dX, and the launches that may precede them in
# the same call (the weight dequantized to bf16 with staging on; the packed weight
# transposed for the register-dequantizing dX)
FWD_KERNELS = ("lora_fwd_rw_kernel", "lora_fwd_kernel")
DX_KERNELS = ("lora_dx_rw_kernel", "lora_dx_kernel")
PRE_KERNELS = ("nf4_dequantize_kernel", "nf4_transpose_kernel")


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
    ap.add_argument("--staged", action="store_true",
                    help="time the headline with weight staging on (lora_nf4_set_weight_staging(1))")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the staging, cold-cache and per-config legs")
    ap.add_argument("--sustain-s", type=float, default=2.0,
                    help="seconds of back-to-back headline steps with the clock sampled (0: skip)")
    ap.add_argument("--leg-steps", type=int, default=10,
                    help="timed steps of each per-config leg")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run under rocprofv3 --pmc: one plain copy of COPY_BYTES (calibration), "
                         "then --steps fwd+bwd steps; prints nothing else")
    ap.add_argument("--small-token-pass", action="store_true",
                    help="run under rocprofv3 --pmc: the calibration copy, then two fwd+bwd of the "
                         "Llama-3-70B gate projection at 1 and at 16 tokens; prints nothing else")
    ap.add_argument("--ingest-small-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="per-kernel HBM bytes of two --small-token-pass counter runs, as markdown")
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
    """Mean counter value (KiB) per forward call and per other kernel. A forward call
    is the tile kernel (lora_fwd_rw_kernel, or lora_fwd_kernel), preceded with weight
    staging on by the weight's dequantization (counted with it); the backward's input
    gradient pairs its tile kernel with the launch before it the same way (the
    dequantization, or the transposition of the packed weight)."""
    import collections
    fwd, other = [], collections.defaultdict(list)
    prev = None
    short = lambda name, keys: next((k for k in keys if k in name), None)
    for _, name, v in disp:
        pre = short(prev[0], PRE_KERNELS) if prev is not None else None
        fk, dk = short(name, FWD_KERNELS), short(name, DX_KERNELS)
        if fk is not None:
            fwd.append(prev[1] + v if pre == "nf4_dequantize_kernel" else v)
        elif dk is not None and pre is not None:
            other[f"lora_dx ({pre} + {dk})"].append(prev[1] + v)
        elif short(name, PRE_KERNELS) is None:
            for key in DX_KERNELS + ("skinny_partial_kernel", "skinny_reduce2_kernel", "MulFunctor"):
                if key in name:
                    other[key].append(v)
                    break
        prev = (name, v)
    if not fwd:
        raise SystemExit("no dispatch of a forward tile kernel in the counter data")
    return sum(fwd) / len(fwd), {k: sum(v) / len(v) for k, v in other.items()}


def ingest_counters(fetch_dir: str, write_dir: str):
    fetch_fwd, fetch_other = forward_kib(counter_dispatches(fetch_dir, "FETCH_SIZE"))
    write_fwd, write_other = forward_kib(counter_dispatches(write_dir, "WRITE_SIZE"))
    copy_key = "MulFunctor"  # the calibration copy: torch.mul(src, 1.0, out=dst)
    if copy_key not in fetch_other or copy_key not in write_other:
        raise SystemExit("no dispatch of the calibration copy in the counter data")
    cal_f = (COPY_BYTES / 1024) / fetch_other[copy_key]
    cal_w = (COPY_BYTES / 1024) / write_other[copy_key]
    rec = {"kernel": "lora_fwd_rw_kernel (the forward call at 8192 tokens: one launch)",
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


SMALL_TOKENS = (1, 16)  # token counts of the weight-bound measurement (70B gate projection)


def gate_projection(q, torch):
    """The Llama-3-70B gate projection's draws (x and dY at 16 tokens), NF4 weight
    quantized on the device."""
    w = next(x for x in synth.WORKLOADS if x.name == "llama3-70b-layer")
    pi = next(i for i, p in enumerate(w.projections) if p.name == "gate_proj")
    inp = synth.projection_inputs(w, pi, tokens=max(SMALL_TOKENS))
    d = {"p": w.projections[pi]}
    for k in ("x", "A", "B", "dY"):
        d[k] = to_dev_bf16(inp[k])
    d["codes"], d["absmax"] = q.nf4_quantize(to_dev_bf16(inp["W"]))
    return w, d


def ingest_small_counters(fetch_dir: str, write_dir: str):
    """Mean FETCH_SIZE / WRITE_SIZE per dispatch of each kernel of the small-token
    pass (first half of the dispatches after the calibration copy: 1 token, second
    half: 16 tokens), scaled by the calibration copy, as a markdown table."""
    import collections
    out = []
    cal = {}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = counter_dispatches(d, counter)
        i = next(j for j, (_, n, _) in enumerate(disp) if "MulFunctor" in n)
        cal[counter] = (COPY_BYTES / 1024) / disp[i][2]
        rest = [x for x in disp[i + 1:] if "lnf4" in x[1]]
        half = len(rest) // 2
        for ti, chunk in enumerate((rest[:half], rest[half:])):
            acc = collections.defaultdict(list)
            for _, name, v in chunk:
                key = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("lnf4::", "")
                key = key.split("(")[0]
                acc[key].append(v * cal[counter] * 1024)
            for k, v in acc.items():
                per.setdefault((SMALL_TOKENS[ti], k), {})[counter] = sum(v) / len(v)
    out.append("| tokens | kernel | read MB / dispatch | written MB / dispatch |")
    out.append("|---|---|---|---|")
    for (t, k), v in sorted(per.items()):
        out.append(f"| {t} | `{k}` | {v.get('FETCH_SIZE', 0) / 1e6:.2f} | {v.get('WRITE_SIZE', 0) / 1e6:.2f} |")
    out.append("")
    out.append(f"calibration: FETCH_SIZE x {cal['FETCH_SIZE']:.3f}, WRITE_SIZE x {cal['WRITE_SIZE']:.3f} "
               f"(a {COPY_BYTES >> 20} MiB copy)")
    print("\n".join(out))


def cpu_baseline(w: synth.Workload, target_s: float):
    """The oracle as it stands, fwd + bwd of the workload's first projection on a
    token sample sized to take about target_s seconds on this host."""
    from oracle import lora as olora
    from oracle import nf4 as onf4
    host = host_facts()
    cores = host["blas_threads"] or host["nproc"]
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
    # three passes over the sample (the median is reported); a pass is sized so the
    # three take about target_s together
    tok = int(min(w.tokens, max(64, tok * (target_s / 3) / max(dt, 1e-3))))
    tok = max(64, (tok // 64) * 64)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        step(tok)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    fl = synth.flops(tok, p.d_in, p.d_out, w.r)
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds_per_pass": round(dt, 3), "passes": 3, "statistic": "median",
            "tokens_per_s": round(tok / dt, 1), "host": host,
            "sample": f"{p.name} {p.d_in}->{p.d_out} r={w.r}, {tok} of {w.tokens} tokens x 3 passes, "
                      f"fp64 NumPy fwd+bwd incl. dequantization"}


def host_facts() -> dict:
    """The host the CPU baseline runs on: logical CPUs, CPU model, the BLAS library
    NumPy calls and its thread count."""
    facts = {"nproc": os.cpu_count(), "cpu_model": None, "blas": None, "blas_threads": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    facts["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        facts["sched_affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            facts["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            facts["blas_threads"] = int(blas[0].get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return facts


def time_fwd_bwd(lib, q, torch, d, w, tokens, sp, reps, warm=5):
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
        for _ in range(warm):
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


def small_token_cold(lib, q, torch, d, w, tokens, sp, reps=15):
    """The same calls one at a time after a 1 GiB read (four times the memory-side
    cache, read rather than written so that no dirty lines are written back during
    the call), HIP events around each call; medians."""
    T = min(tokens, w.tokens)
    p = d["p"]
    K, N, r = p.d_in, p.d_out, w.r
    x, dy = d["x"][:T], d["dY"][:T]
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((T, r), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((K, r), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((r, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(q.lora_nf4_bwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(q.lora_nf4_fwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")
    scrub = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fwd():
        return lib.lora_nf4_fwd(T, K, N, r, w.alpha, x.data_ptr(), d["codes"].data_ptr(), d["absmax"].data_ptr(),
                                d["A"].data_ptr(), d["B"].data_ptr(), y.data_ptr(), u.data_ptr(),
                                fws.data_ptr(), fws.numel(), sp)

    def bwd():
        return lib.lora_nf4_bwd(T, K, N, r, w.alpha, x.data_ptr(), dy.data_ptr(), d["codes"].data_ptr(),
                                d["absmax"].data_ptr(), d["A"].data_ptr(), d["B"].data_ptr(), u.data_ptr(),
                                dx.data_ptr(), dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), ws.numel(), sp)
    res = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        ts = []
        for _ in range(reps):
            scrub.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if st != 0:
                raise q.LoraNF4Error("lora_nf4_" + name, st)
            ts.append(e0.elapsed_time(e1) * 1000.0)
        res[name] = pct(ts, 50)
    del scrub
    return res["fwd"], res["bwd"]


def weight_bound_legs(lib, q, torch, d, w, sp, tokens=(1, 16)):
    """The Llama-3-70B gate projection (8192 -> 28672, 132 MB of packed weight) at a
    few tokens: forward and backward back to back (warm: the weight may stay in the
    256 MB memory-side cache) and one call at a time after a cache scrub (cold),
    as weight GB/s against the 8 TB/s HBM peak."""
    out = []
    for T in tokens:
        leg = small_token_run(lib, q, torch, d, w, T, sp)
        f_c, b_c = small_token_cold(lib, q, torch, d, w, T, sp)
        wb = leg["weight_bytes"]
        leg.update({"cold_fwd_us": round(f_c, 2), "cold_bwd_us": round(b_c, 2),
                    "cold_fwd_weight_GBps": round(wb / f_c / 1e3, 1),
                    "cold_fwd_frac": round(wb / f_c / 1e3 / PEAK_HBM_GBS, 4),
                    "cold_bwd_weight_GBps": round(wb / b_c / 1e3, 1)})
        out.append(leg)
    return out


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


def rank_r_run(lib, q, torch, d, w, sp, reps=50):
    """The backward's rank-r step alone (lora_nf4_grad_ab: dA = x^T G, dB = s U^T dY)
    on the whole projection, HIP events around `reps` back-to-back C-ABI calls; G and
    U (bf16 [T, r]) made once with float32 torch products. Bytes = x and dY in (the
    bound: 2 T (d_in + d_out)) + G and U in + dA and dB out."""
    p = d["p"]
    K, N, r, T = p.d_in, p.d_out, w.r, w.tokens
    s = w.alpha / r
    x, dy = d["x"], d["dY"]
    g = (dy.float() @ d["B"].float().t() * s).bfloat16().contiguous()
    u = (x.float() @ d["A"].float()).bfloat16().contiguous()
    dA = torch.empty((K, r), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((r, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(q.lora_nf4_grad_ab_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")

    def call():
        st = lib.lora_nf4_grad_ab(T, K, N, r, w.alpha, x.data_ptr(), g.data_ptr(), dy.data_ptr(), u.data_ptr(),
                                  dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_grad_ab", st)

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
    nbytes = 2 * T * (K + N) + 2 * 2 * T * r + 2 * r * (K + N)
    del g, u, dA, dB, ws
    return {"projection": f"{p.name} {K}->{N}", "tokens": T, "r": r, "us": round(us, 2), "bytes": nbytes,
            "bound": "hbm", "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}


def train_step_run(lib, q, torch, d, w, sp, reps=50):
    """The training-step companions on one projection, HIP events around `reps`
    back-to-back C-ABI calls each:
      adamw      lora_adamw_step over A and B (float32 master, bf16 copy, bf16
                 gradient, float32 moments); bytes per element: master in and out 8,
                 copy out 2, gradient in 2, each moment in and out 8 = 28;
      adamw8     lora_adamw8_step (8-bit blockwise moments): 8 + 2 + 2 + 2 x 2 = 16
                 per element (+ 16 per 256 for the scales);
      absmax_dq  nf4_absmax_quantize of the projection's block scales; bytes = 4 in
                 + 1 out per scale (+ 8 per 256).
    And the optimizer fused into the backward: lora_nf4_bwd_adamw against
    lora_nf4_bwd + two lora_adamw_step calls on the same state, at the
    workload's token count."""
    p = d["p"]
    K, N, r = p.d_in, p.d_out, w.r
    n = K * r + r * N
    master = torch.zeros(n, dtype=torch.float32, device="cuda")
    copy = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    grad = torch.full((n,), 1e-3, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    st8 = q.adamw8_state(n)
    na = d["absmax"].numel()
    dq_q = torch.empty(na, dtype=torch.uint8, device="cuda")
    dq_s = torch.empty((na + 255) // 256, dtype=torch.float32, device="cuda")
    dq_o = torch.empty_like(dq_s)

    def adamw(step):
        st = lib.lora_adamw_step(n, master.data_ptr(), copy.data_ptr(), grad.data_ptr(), m.data_ptr(),
                                 v.data_ptr(), step, 1e-4, 0.9, 0.999, 1e-8, 0.01, sp)
        if st != 0:
            raise q.LoraNF4Error("lora_adamw_step", st)

    def adamw8(step):
        st = lib.lora_adamw8_step(n, master.data_ptr(), copy.data_ptr(), grad.data_ptr(), st8[0].data_ptr(),
                                  st8[1].data_ptr(), st8[2].data_ptr(), st8[3].data_ptr(), step, 1e-4, 0.9,
                                  0.999, 1e-8, 0.01, sp)
        if st != 0:
            raise q.LoraNF4Error("lora_adamw8_step", st)

    def dq(step):
        st = lib.nf4_absmax_quantize(d["absmax"].data_ptr(), na, dq_q.data_ptr(), dq_s.data_ptr(),
                                     dq_o.data_ptr(), sp)
        if st != 0:
            raise q.LoraNF4Error("nf4_absmax_quantize", st)

    out = {}
    stream = torch.cuda.current_stream()

    def time_calls(fn, count):
        for i in range(3):
            fn(i + 1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(count):
            fn(i + 4)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / count

    for name, fn, nbytes, elems in (("adamw", adamw, 28 * n, n), ("adamw8", adamw8, 16 * n + n // 16, n),
                                    ("absmax_dq", dq, 5 * na + 8 * dq_s.numel(), na)):
        us = time_calls(fn, reps)
        out[name] = {"elements": elems, "us": round(us, 2), "bytes": nbytes,
                     "bound": "hbm", "achieved": round(nbytes / us / 1e3, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}
    # fused optimizer: backward + AdamW of A and B in one call, against backward + two steps
    T = w.tokens
    A2, B2 = d["A"].clone(), d["B"].clone()
    sa = [torch.zeros(K * r, dtype=torch.float32, device="cuda") for _ in range(3)]
    sb = [torch.zeros(r * N, dtype=torch.float32, device="cuda") for _ in range(3)]
    sa[0].copy_(A2.float().view(-1)), sb[0].copy_(B2.float().view(-1))
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((K, r), dtype=torch.bfloat16, device="cuda")
    dB = torch.empty((r, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(q.lora_nf4_bwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8, device="cuda")

    def fused(step):
        st = lib.lora_nf4_bwd_adamw(T, K, N, r, w.alpha, d["x"].data_ptr(), d["dY"].data_ptr(),
                                    d["codes"].data_ptr(), d["absmax"].data_ptr(), A2.data_ptr(), B2.data_ptr(),
                                    d["u"].data_ptr(), dx.data_ptr(), *(t.data_ptr() for t in sa),
                                    *(t.data_ptr() for t in sb), step, 1e-4, 0.9, 0.999, 1e-8, 0.01,
                                    ws.data_ptr(), ws.numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_bwd_adamw", st)

    def unfused(step):
        st = lib.lora_nf4_bwd(T, K, N, r, w.alpha, d["x"].data_ptr(), d["dY"].data_ptr(), d["codes"].data_ptr(),
                              d["absmax"].data_ptr(), A2.data_ptr(), B2.data_ptr(), d["u"].data_ptr(),
                              dx.data_ptr(), dA.data_ptr(), dB.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        st = st or lib.lora_adamw_step(K * r, sa[0].data_ptr(), A2.data_ptr(), dA.data_ptr(), sa[1].data_ptr(),
                                       sa[2].data_ptr(), step, 1e-4, 0.9, 0.999, 1e-8, 0.01, sp)
        st = st or lib.lora_adamw_step(r * N, sb[0].data_ptr(), B2.data_ptr(), dB.data_ptr(), sb[1].data_ptr(),
                                       sb[2].data_ptr(), step, 1e-4, 0.9, 0.999, 1e-8, 0.01, sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_bwd + lora_adamw_step", st)

    if lora_bwd_adamw_available(q, r, N):
        # interleaved rounds (the clock drifts over a run), median of each
        tf, tu = [], []
        for _ in range(5):
            tf.append(time_calls(fused, 10))
            tu.append(time_calls(unfused, 10))
        t_f, t_u = float(np.median(tf)), float(np.median(tu))
        out["bwd_with_optimizer"] = {"tokens": T, "fused_us": round(t_f, 2), "separate_us": round(t_u, 2),
                                     "what": "lora_nf4_bwd_adamw (AdamW of A and B in the rank-r reduction) "
                                             "against lora_nf4_bwd + two lora_adamw_step launches"}
    out["projection"] = f"{p.name} {K}->{N}"
    del master, copy, grad, m, v, st8, dq_q, dq_s, dq_o, A2, B2, sa, sb, dx, dA, dB, ws
    return out


def lora_bwd_adamw_available(q, r, N):
    return r % 8 == 0 and r <= 64 and N % 8 == 0


def multi_projection_run(lib, q, torch, sp, reps=10, rounds=5):
    """Llama-3-8B q/k/v (4096 -> 4096, 1024, 1024) at 8192 tokens, r = 64, sharing one
    x: one fwd + bwd of the three projections as lora_nf4_fwd_multi + lora_nf4_bwd_multi
    (dX summed over them) against three lora_nf4_fwd + three lora_nf4_bwd calls (three
    separate dX, not summed). HIP events around blocks of `reps` back-to-back steps,
    `rounds` blocks per side, alternating."""
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
    for fn in (fused, separate):
        for _ in range(2):
            fn()
    torch.cuda.synchronize()
    # alternating blocks of `reps` back-to-back steps, so that a change of clock
    # during the leg reaches both sides; medians over the blocks
    per = {"fused": [], "separate": []}
    for _ in range(rounds):
        for name, fn in (("fused", fused), ("separate", separate)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            per[name].append(e0.elapsed_time(e1) / reps)
    for name, v in per.items():
        ms = pct(v, 50)
        out[f"{name}_ms"] = round(ms, 4)
        out[f"{name}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
    out["fused_faster_by"] = round(1.0 - out["fused_ms"] / out["separate_ms"], 4)
    out["blocks"] = f"{rounds} alternating blocks of {reps} steps each side, medians"
    out["note"] = "separate leaves three dX arrays unsummed; fused returns their sum"
    del x, codes, absmax, A, B, dy, ys, us, dx, dxs, dAs, dBs, wsm, wss
    return out


def to_dev_bf16(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


class Runner:
    """One workload resident on the GPU: inputs drawn from synth (seeded), NF4
    weights quantized once (model load), every output and workspace allocated up
    front. step() enqueues one forward + backward of every projection (or of every
    fused group, see --fuse) through the C ABI on the current stream."""

    def __init__(self, lib, q, torch, w, fuse):
        import ctypes
        self.lib, self.q, self.w = lib, q, w
        self.sp = torch.cuda.current_stream().cuda_stream
        projs = []
        for pi, p in enumerate(w.projections):
            inp = synth.projection_inputs(w, pi)
            x, W, A, B, dY = (to_dev_bf16(inp[k]) for k in ("x", "W", "A", "B", "dY"))
            del inp
            codes, absmax = q.nf4_quantize(W)
            del W
            T, K, N, r = w.tokens, p.d_in, p.d_out, w.r
            projs.append(dict(p=p, x=x, A=A, B=B, dY=dY, codes=codes, absmax=absmax,
                              y=torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
                              u=torch.empty((T, r), dtype=torch.bfloat16, device="cuda"),
                              dx=torch.empty((T, K), dtype=torch.bfloat16, device="cuda"),
                              dA=torch.empty((K, r), dtype=torch.bfloat16, device="cuda"),
                              dB=torch.empty((r, N), dtype=torch.bfloat16, device="cuda")))
        # forward units: one projection each, or (fuse) the groups that share x
        units, seen = [], {}
        for j, d in enumerate(projs):
            key = {"q_proj": "qkv", "k_proj": "qkv", "v_proj": "qkv", "gate_proj": "gu",
                   "up_proj": "gu"}.get(d["p"].name) if fuse else None
            if key is not None and key in seen:
                units[seen[key]].append(j)
                d["x"] = projs[units[seen[key]][0]]["x"]  # the group reads one x
            else:
                if key is not None:
                    seen[key] = len(units)
                units.append([j])
        self.projs, self.units = projs, units
        self.multi = {}
        for ui, un in enumerate(units):
            if len(un) > 1:
                arr = lambda key: (ctypes.c_void_p * len(un))(*[projs[j][key].data_ptr() for j in un])
                self.multi[ui] = dict(d_out=(ctypes.c_int64 * len(un))(*[projs[j]["p"].d_out for j in un]),
                                      codes=arr("codes"), absmax=arr("absmax"), A=arr("A"), B=arr("B"),
                                      y=arr("y"), u=arr("u"), dy=arr("dY"), dA=arr("dA"), dB=arr("dB"))
        self.size_workspaces(torch)

    def size_workspaces(self, torch):
        """(Re)allocate the workspaces for the current weight-staging mode."""
        q, w = self.q, self.w
        for d in self.projs:
            T, K, N, r = w.tokens, d["p"].d_in, d["p"].d_out, w.r
            d["ws"] = torch.empty(max(q.lora_nf4_bwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8,
                                  device="cuda")
            d["fws"] = torch.empty(max(q.lora_nf4_fwd_workspace_bytes(T, K, N, r), 256), dtype=torch.uint8,
                                   device="cuda")
        for ui, m in self.multi.items():
            un = self.units[ui]
            d_out = [self.projs[j]["p"].d_out for j in un]
            K = self.projs[un[0]]["p"].d_in
            m["ws"] = torch.empty(max(q.lora_nf4_bwd_multi_workspace_bytes(w.tokens, K, d_out, w.r), 256),
                                  dtype=torch.uint8, device="cuda")
            m["fws"] = torch.empty(max(q.lora_nf4_fwd_multi_workspace_bytes(w.tokens, K, d_out, w.r), 256),
                                   dtype=torch.uint8, device="cuda")
            for j in un:  # the group's per-projection workspaces are not used
                self.projs[j]["ws"] = self.projs[j]["fws"] = None
        torch.cuda.empty_cache()

    def fwd_unit(self, ui):
        import ctypes
        lib, q, w, sp = self.lib, self.q, self.w, self.sp
        un = self.units[ui]
        if len(un) == 1:
            d = self.projs[un[0]]
            p = d["p"]
            st = lib.lora_nf4_fwd(w.tokens, p.d_in, p.d_out, w.r, w.alpha, d["x"].data_ptr(),
                                  d["codes"].data_ptr(), d["absmax"].data_ptr(), d["A"].data_ptr(),
                                  d["B"].data_ptr(), d["y"].data_ptr(), d["u"].data_ptr(), d["fws"].data_ptr(),
                                  d["fws"].numel(), sp)
            if st != 0:
                raise q.LoraNF4Error("lora_nf4_fwd", st)
            return
        m, d0 = self.multi[ui], self.projs[un[0]]
        cv = lambda a: ctypes.cast(a, ctypes.c_void_p)
        st = lib.lora_nf4_fwd_multi(w.tokens, d0["p"].d_in, len(un), cv(m["d_out"]), w.r, w.alpha,
                                    d0["x"].data_ptr(), cv(m["codes"]), cv(m["absmax"]), cv(m["A"]),
                                    cv(m["B"]), cv(m["y"]), cv(m["u"]), m["fws"].data_ptr(), m["fws"].numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_fwd_multi", st)

    def bwd_unit(self, ui):
        import ctypes
        lib, q, w, sp = self.lib, self.q, self.w, self.sp
        un = self.units[ui]
        if len(un) == 1:
            d = self.projs[un[0]]
            p = d["p"]
            st = lib.lora_nf4_bwd(w.tokens, p.d_in, p.d_out, w.r, w.alpha, d["x"].data_ptr(),
                                  d["dY"].data_ptr(), d["codes"].data_ptr(), d["absmax"].data_ptr(),
                                  d["A"].data_ptr(), d["B"].data_ptr(), d["u"].data_ptr(),
                                  d["dx"].data_ptr(), d["dA"].data_ptr(), d["dB"].data_ptr(),
                                  d["ws"].data_ptr(), d["ws"].numel(), sp)
            if st != 0:
                raise q.LoraNF4Error("lora_nf4_bwd", st)
            return
        m, d0 = self.multi[ui], self.projs[un[0]]
        cv = lambda a: ctypes.cast(a, ctypes.c_void_p)
        st = lib.lora_nf4_bwd_multi(w.tokens, d0["p"].d_in, len(un), cv(m["d_out"]), w.r, w.alpha,
                                    d0["x"].data_ptr(), cv(m["dy"]), cv(m["codes"]), cv(m["absmax"]),
                                    cv(m["A"]), cv(m["B"]), cv(m["u"]), d0["dx"].data_ptr(), cv(m["dA"]),
                                    cv(m["dB"]), m["ws"].data_ptr(), m["ws"].numel(), sp)
        if st != 0:
            raise q.LoraNF4Error("lora_nf4_bwd_multi", st)

    def step(self):
        for ui in range(len(self.units)):
            self.fwd_unit(ui)
            self.bwd_unit(ui)

    def flops(self):
        w = self.w
        return sum(synth.flops(w.tokens, d["p"].d_in, d["p"].d_out, w.r) for d in self.projs)

    def big_unit(self):
        """(unit index, its projections' forward FLOPs, label) of the unit holding the largest projection."""
        projs, w = self.projs, self.w
        big = max(range(len(projs)), key=lambda j: projs[j]["p"].d_in * projs[j]["p"].d_out)
        bu = next(ui for ui, un in enumerate(self.units) if big in un)
        fl = sum(2 * w.tokens * projs[j]["p"].d_in * projs[j]["p"].d_out
                 + 2 * w.tokens * w.r * (projs[j]["p"].d_in + projs[j]["p"].d_out) for j in self.units[bu])
        label = " + ".join(f"{projs[j]['p'].name} {projs[j]['p'].d_in}->{projs[j]['p'].d_out}"
                           for j in self.units[bu])
        return bu, fl, label


def timed_region(torch, run, steps, warmup):
    """`warmup` untimed steps, then `steps` steps between two HIP events and no
    others (nothing enqueued between the steps' kernels). Returns ms."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        run.step()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def timed_steps(torch, run, steps, warmup, scrub=None):
    """`warmup` untimed steps, then `steps` timed ones. HIP events on the stream
    bracket the whole region, every step, and the forward / backward calls of the
    largest projection's unit. scrub: a callable enqueued before every timed step
    (outside its events), e.g. a cache flush. Returns total ms and the per-step ms
    lists of the whole step, of that unit's forward and of its backward."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    bu, _, _ = run.big_unit()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    t0, t1 = ev(), ev()
    st = [(ev(), ev(), ev(), ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        if scrub is not None:
            scrub()
        s0, f0, f1, b1, s1 = st[i]
        s0.record(stream)
        for ui in range(len(run.units)):
            if ui == bu:
                f0.record(stream)
            run.fwd_unit(ui)
            if ui == bu:
                f1.record(stream)
            run.bwd_unit(ui)
            if ui == bu:
                b1.record(stream)
        s1.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    per_step = [e[0].elapsed_time(e[4]) for e in st]
    fwd = [e[1].elapsed_time(e[2]) for e in st]
    bwd = [e[2].elapsed_time(e[3]) for e in st]
    return t0.elapsed_time(t1), per_step, fwd, bwd


def progress(msg):
    """One line on stderr per finished part (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def pct(xs, p):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), p))


class ClockSampler:
    """Shader clock (MHz) of GPU 0, polled with amd-smi in a background thread while a
    timed region runs. None where amd-smi gives no reading."""

    def __init__(self, period_s=0.05):
        import threading
        self.period, self.samples, self.stop = period_s, [], threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def read():
        import re
        import subprocess
        try:
            out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True,
                                 text=True, timeout=5).stdout
            starts = [i for i in (out.find("{"), out.find("[")) if i >= 0]
            data = json.loads(out[min(starts):])
        except Exception:
            return None
        vals = []

        # {"gpu_data": [{"clock": {"gfx_0": {"clk": {"value": 2100, "unit": "MHz"}, ...}, ...}}]}:
        # the current clock of every graphics partition (not min_clk / max_clk)
        def walk(o, path):
            if isinstance(o, dict):
                for k, v in o.items():
                    walk(v, path + [str(k).lower()])
            elif isinstance(o, list):
                for v in o:
                    walk(v, path)
            elif (len(path) >= 3 and path[-3].startswith("gfx") and path[-2] == "clk"
                  and path[-1] == "value"):
                try:
                    vals.append(float(re.sub(r"[^0-9.]", "", str(o))))
                except ValueError:
                    pass
        walk(data, [])
        vals = [v for v in vals if v > 0]
        return sum(vals) / len(vals) if vals else None  # mean over the XCDs' graphics clocks

    def _run(self):
        while not self.stop.is_set():
            v = self.read()
            if v is not None:
                self.samples.append(v)
            self.stop.wait(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join(timeout=10)
        return False

    def summary(self):
        if not self.samples:
            return None
        top = max(self.samples)
        busy = [v for v in self.samples if v >= 0.5 * top]  # idle readings at the window's edges dropped
        return {"median_mhz": round(pct(busy, 50), 1), "min_mhz": round(min(busy), 1),
                "max_mhz": round(top, 1), "samples": len(busy), "dropped_idle": len(self.samples) - len(busy),
                "source": "amd-smi metric -g 0 -c (mean of the XCDs' gfx clocks), polled every 50 ms"}


def sustained_run(torch, run, seconds):
    """The headline step repeated back to back for about `seconds` (well past the
    timed region's few tens of ms), the shader clock polled with amd-smi meanwhile:
    the clock the GPU holds under this load, and the median step time at it."""
    if seconds <= 0:
        return None
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    per = []
    with ClockSampler() as clock:
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            batch = [(ev(), ev()) for _ in range(50)]
            for a, b in batch:
                a.record(stream)
                run.step()
                b.record(stream)
            torch.cuda.synchronize()
            per.extend(a.elapsed_time(b) for a, b in batch)
    return {"seconds": seconds, "steps": len(per), "step_ms": step_stats(per), "sclk": clock.summary()}


def step_stats(per_step):
    return {"p10": round(pct(per_step, 10), 4), "p50": round(pct(per_step, 50), 4),
            "p90": round(pct(per_step, 90), 4)}


def config_leg(lib, q, torch, name, steps, warmup, extra=None):
    """fwd + bwd of every projection of one workload (fused where the projections
    share x), per-step HIP events; median step time, TFLOP/s and tokens/s. `extra`
    (run) -> dict runs further measurements on the resident workload."""
    w = next(x for x in synth.WORKLOADS if x.name == name)
    run = Runner(lib, q, torch, w, fuse=True)
    total, per_step, fwd, bwd = timed_steps(torch, run, steps, warmup)
    more = extra(run) if extra is not None else {}
    med = pct(per_step, 50)
    out = {"tokens": w.tokens, "r": w.r, "fwd_ms_p50_largest_unit": round(pct(fwd, 50), 4),
           "bwd_ms_p50_largest_unit": round(pct(bwd, 50), 4),
           "projections": [f"{d['p'].name} {d['p'].d_in}->{d['p'].d_out}" for d in run.projs],
           "fused": [[run.projs[j]["p"].name for j in un] for un in run.units if len(un) > 1],
           "steps": steps, "step_ms": step_stats(per_step), "ms_per_step_mean": round(total / steps, 4),
           "tflops_median_step": round(run.flops() / (med * 1e-3) / 1e12, 2),
           "tokens_per_s_median_step": round(w.tokens / (med * 1e-3), 1),
           "pct_of_bf16_peak": round(100.0 * run.flops() / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    out.update(more)
    del run
    torch.cuda.empty_cache()
    return out


def mfma_probe(lib, torch, sp):
    """The library's MFMA-only probe (lora_nf4_mfma_probe): back-to-back
    v_mfma_f32_32x32x16_bf16 on register operands, two waves per SIMD on every CU;
    HIP events around one launch after a warm-up launch. None if the probe is absent."""
    if not hasattr(lib, "lora_nf4_mfma_probe"):
        return None
    sink = torch.zeros(1024, dtype=torch.float32, device="cuda")
    iters = 4096
    flops = lib.lora_nf4_mfma_probe(iters, sink.data_ptr(), sp)  # warm-up; returns the launch's FLOPs
    if flops <= 0:
        return None
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        lib.lora_nf4_mfma_probe(iters, sink.data_ptr(), sp)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "launch_ms": round(ms, 4),
            "frac_of_spec": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "what": "v_mfma_f32_32x32x16_bf16 back to back on registers, 8 independent accumulators per "
                    "wave, 8 waves per CU, no memory traffic"}


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.ingest_small_counters:
        ingest_small_counters(*args.ingest_small_counters)
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
    lib = q.library()
    torch.cuda.set_device(0)
    q.set_weight_staging(bool(args.staged))
    if args.small_token_pass:
        gw, gd = gate_projection(q, torch)
        sp = torch.cuda.current_stream().cuda_stream
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # plain copy of known size: calibrates the counters
        torch.cuda.synchronize()
        for T in SMALL_TOKENS:
            time_fwd_bwd(lib, q, torch, gd, gw, T, sp, 2, warm=0)
        torch.cuda.synchronize()
        return
    run = Runner(lib, q, torch, w, args.fuse)
    sp = run.sp

    if args.counter_pass:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # plain copy of known size: calibrates the counters
        torch.cuda.synchronize()
        for _ in range(args.steps):
            run.step()
        torch.cuda.synchronize()
        return

    # the timed region (value, ms_per_step): K steps between two events; then K more
    # steps with events around every step and the largest unit's forward and
    # backward (their distributions and the roofline's forward time)
    wall0 = time.perf_counter()
    total_ms = timed_region(torch, run, args.steps, args.warmup)
    wall = time.perf_counter() - wall0
    _, per_step, fwd_ms, bwd_ms = timed_steps(torch, run, args.steps, 2)
    ms_step = total_ms / args.steps
    progress(f"{w.name}: {args.steps} steps, {ms_step:.4f} ms/step")
    flops_step = run.flops()
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    tokens_s = w.tokens / (ms_step * 1e-3)
    bu, fwd_flops, unit_label = run.big_unit()
    pb = run.projs[run.units[bu][0]]["p"]
    T, K, N, r = w.tokens, pb.d_in, pb.d_out, w.r
    fwd_avg = float(np.mean(fwd_ms))
    achieved = fwd_flops / (fwd_avg * 1e-3) / 1e12
    traffic = None if args.staged else measured_traffic()  # the record covers the default mode's kernel
    staged = q.lora_nf4_fwd_workspace_bytes(T, K, N, r) >= K * N * 2
    kernel = ("lora_fwd (nf4_dequantize_kernel + lora_fwd_kernel on the staged bf16 weight)" if staged else
              "lora_fwd_rw_kernel (NF4 dequantized into MFMA fragments in the K loop)")

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
                   "projections": [f"{d['p'].name} {d['p'].d_in}->{d['p'].d_out}" for d in run.projs],
                   "weights": "NF4 blocksize 64, fp32 absmax", "parallelism": "single GPU",
                   "weight_staging": bool(args.staged),
                   "fused_forward": [[run.projs[j]["p"].name for j in un] for un in run.units if len(un) > 1],
                   "fused_backward": [[run.projs[j]["p"].name for j in un] for un in run.units if len(un) > 1]},
        "tokens_per_s": round(tokens_s, 1),
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_ms": step_stats(per_step),
        "step_ms_note": "p10/p50/p90 from a second pass of K steps with HIP events around every step and "
                        "around the forward and backward (events add a few us per step)",
        "fwd_ms": round(fwd_avg, 4),
        "fwd_ms_p50": round(pct(fwd_ms, 50), 4),
        "bwd_ms": round(float(np.mean(bwd_ms)), 4),
        "bwd_ms_p50": round(pct(bwd_ms, 50), 4),
        "host_wall_s": round(wall, 4),
        "sustained": sustained_run(torch, run, args.sustain_s),
        "roofline": {"kernel": kernel, "projection": unit_label,
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    out["mfma_probe"] = mfma_probe(lib, torch, sp)
    if out["mfma_probe"] is not None:
        out["roofline"]["frac_of_measured_mfma_peak"] = round(achieved / out["mfma_probe"]["tflops"], 4)
    if not args.no_legs:
        # the same step with the weight dequantized to bf16 into the workspace first
        prev = q.set_weight_staging(not args.staged)
        run.size_workspaces(torch)
        total2, per2, fwd2, bwd2 = timed_steps(torch, run, args.steps, args.warmup)
        q.set_weight_staging(prev)
        run.size_workspaces(torch)
        med2 = pct(per2, 50)
        progress(f"weight staging {'off' if args.staged else 'on'}: median step {med2:.4f} ms")
        out["weight_staging_" + ("off" if args.staged else "on")] = {
            "step_ms": step_stats(per2), "fwd_ms_p50": round(pct(fwd2, 50), 4),
            "bwd_ms_p50": round(pct(bwd2, 50), 4),
            "tflops_median_step": round(flops_step / (med2 * 1e-3) / 1e12, 2),
            "note": "lora_nf4_set_weight_staging(1): the forward and dX read a bf16 copy of the weight "
                    "dequantized into their workspace (2 B/weight) instead of dequantizing in the K loop"}
        # cold caches: a 512 MiB write (twice the 256 MB memory-side cache) before every step
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        _, per3, fwd3, bwd3 = timed_steps(torch, run, max(10, args.steps // 5), 2, scrub=lambda: flush.fill_(1))
        del flush
        progress(f"cold cache: median step {pct(per3, 50):.4f} ms")
        out["cold_cache"] = {"step_ms": step_stats(per3), "fwd_ms_p50": round(pct(fwd3, 50), 4),
                             "bwd_ms_p50": round(pct(bwd3, 50), 4),
                             "steps": len(per3),
                             "scrub": "512 MiB device fill before every step (outside its events)"}
    progress("mfma probe: " + (f"{out['mfma_probe']['tflops']} TFLOP/s" if out["mfma_probe"] else "absent"))
    if args.small_tokens > 0:
        out["small_tokens_headline_projection"] = small_token_run(lib, q, torch, run.projs[run.units[bu][0]], w,
                                                                  args.small_tokens, sp)
    if args.medium_tokens > 0:
        out["medium_tokens"] = medium_token_run(lib, q, torch, run.projs[run.units[bu][0]], w, args.medium_tokens, sp)
    out["merge"] = merge_run(lib, q, torch, run.projs[run.units[bu][0]], w, sp)
    out["rank_r_gradients"] = rank_r_run(lib, q, torch, run.projs[run.units[bu][0]], w, sp)
    out["train_step"] = train_step_run(lib, q, torch, run.projs[run.units[bu][0]], w, sp)
    progress("small / medium tokens, merge, training step done")
    del run
    torch.cuda.empty_cache()
    if not args.no_multi:
        out["multi_projection"] = multi_projection_run(lib, q, torch, sp)
        progress("multi-projection leg done")
    if not args.no_legs:
        out["configs"] = {}
        for name in ("llama3-8b-attn-r64", "qwen14b-attn", "llama3-70b-layer"):
            if name != w.name:
                extra = None
                if name == "llama3-70b-layer" and args.small_tokens > 0:
                    def extra(run):
                        gate = next(dd for dd in run.projs if dd["p"].name == "gate_proj")
                        return {"small_tokens_gate": weight_bound_legs(lib, q, torch, gate, run.w, sp)}
                out["configs"][name] = config_leg(lib, q, torch, name, args.leg_steps, 3, extra)
                progress(f"{name}: median step {out['configs'][name]['step_ms']['p50']} ms")
                if "small_tokens_gate" in out["configs"][name]:
                    out["small_tokens"] = out["configs"][name].pop("small_tokens_gate")
                    progress("small tokens (70B gate) done")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        progress("cpu baseline done")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
