#!/usr/bin/env python3
"""Benchmark of attn_fwd on one MI355X: attention forward TFLOP/s and the
fraction of the dense bf16 MFMA peak, on the long-context causal workload
B=2, H=32, N=8192, d=128 (bf16 in and out, fp32 arithmetic).

One step is one attn_fwd call over the whole batch (every stage of the path
runs inside it).  Inputs are seeded synthetic tensors already resident in HBM
when the timed region starts.  Prints ONE JSON line.

Counted work is 4*B*H*N^2*d, halved for causal.  Peak: MI355X dense bf16
MFMA, 256 CUs x 2.4 GHz x 4096 flop/clk/CU = 2516.6 TFLOP/s.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS
HBM_PEAK_GBPS = 8000.0
METRIC = "attn fwd TFLOP/s + % of bf16 MFMA peak, 1 GPU, N=8192 d=128 causal"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_long_causal_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_io_aware_27_amd", "csrc", f)
                  for f in ("attn_fwd_kernel.hip", "attn_common.h", "exp2_poly.h")]  # the forward kernel's own code


def code_only(text):
    """C++ source without its comments and blank lines, so that an edit to a
    comment does not count as a change of the kernel."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def compiler_id():
    """hipcc's version lines (HIP and clang): a compiler change changes the
    generated code.  Only those lines, so that the id is the same on every
    machine with the same compiler (hipcc may add warnings about the host's
    devices on stderr)."""
    import subprocess

    from exact_io_aware_27_amd import build
    try:
        text = subprocess.check_output([build.HIPCC, "--version"], text=True, stderr=subprocess.DEVNULL)
    except (OSError, subprocess.CalledProcessError):
        return "hipcc unavailable"
    return "\n".join(l for l in text.splitlines() if l.startswith(("HIP version", "AMD clang version")))


def device_clock_ghz():
    """The peak shader clock the HIP runtime reports for device 0, in GHz
    (hipDeviceAttributeClockRate, in kHz), or None.  The dense bf16 peak
    derived from it and the CU count (4096 flops per CU per clock: four
    matrix cores, each a 32x32x16 MFMA of 32768 flops every 32 clocks) is
    printed beside the published one."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch and libattn.so already hold
    except OSError:
        return None
    khz = ctypes.c_int(0)
    attr_clock_rate = 5  # hipDeviceAttributeClockRate, sixth entry of hipDeviceAttribute_t
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), attr_clock_rate, 0) != 0 or khz.value <= 0:
        return None
    return khz.value / 1e6


def device_info(props):
    ghz = device_clock_ghz()
    return {"name": props.name, "cus": props.multi_processor_count,
            "gcn_arch": getattr(props, "gcnArchName", None), "clock_ghz": ghz,
            "bf16_peak_from_device_tflops": (round(props.multi_processor_count * 4096 * ghz / 1e3, 1)
                                             if ghz else None)}


def kernel_hash():
    """Hash of what the forward kernel's machine code depends on: its source
    (comments excluded), the build flags and the compiler version."""
    from exact_io_aware_27_amd import build
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            h.update(code_only(f.read()).encode())
    # the flags, less the include directory's location (a checkout's path,
    # which differs between machines and does not change the code)
    flags, skip = [], False
    for f in build.FLAGS:
        if skip:
            skip = False
        elif f == "-I":
            skip = True
        else:
            flags.append(f)
    h.update(" ".join(flags).encode())
    h.update(compiler_id().encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def pmc_summary(fetch_csv, write_csv, copy_mib, out_json=TRAFFIC_FILE):
    """HBM bytes per attn_fwd launch from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, both in KiB per dispatch), each scaled by what the same
    counter reads for the plain device copy of copy_mib MiB that bench.py runs
    with --copy-calibration-mib (an elementwise kernel that reads and writes
    copy_mib MiB; the largest non-attention dispatch of each run).  Writes
    out_json and returns the summary."""
    import csv

    def per_dispatch(path, counter):
        attn, copy = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                if "attn_fwd_kernel" in name:
                    attn.append(float(r["Counter_Value"]))
                else:  # the fill and the copy of the calibration buffer
                    copy.append(float(r["Counter_Value"]))
        if not attn or not copy:
            raise SystemExit("%s: no %s rows for attn_fwd_kernel and the calibration copy" % (path, counter))
        return sum(attn) / len(attn), max(copy)

    known = copy_mib * 1024.0  # KiB moved each way by the copy
    fa, fc = per_dispatch(fetch_csv, "FETCH_SIZE")
    wa, wc = per_dispatch(write_csv, "WRITE_SIZE")
    f_fetch, f_write = known / fc, known / wc
    total = (fa * f_fetch + wa * f_write) * 1024.0
    summary = {"kernel_hash": kernel_hash(), "workload": "long_causal B=2 H=32 N=8192 d=128 causal",
               "fetch_kib_per_launch": fa, "write_kib_per_launch": wa,
               "copy_mib": copy_mib, "copy_fetch_kib": fc, "copy_write_kib": wc,
               "fetch_scale": f_fetch, "write_scale": f_write,
               "hbm_bytes_per_launch": total}
    with open(out_json, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    return summary


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, rows_per_head):
    """Time the fp64 oracle on a bounded, seeded row sample of the same workload;
    the same rows double as a parity check of the timed launch's output."""
    import numpy as np
    import torch

    import oracle
    from exact_io_aware_27_amd import inputs

    rows = inputs.row_subsets(w, R=rows_per_head)
    threads = oracle.oracle.default_threads()
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention(q, k, v, w.causal, w.scale, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    keys = (rows + 1).double() if w.causal else torch.full(rows.shape, float(w.N), dtype=torch.float64)
    flops = float(keys.sum()) * 4 * w.d
    # parity of the sampled rows
    flat_o = o_gpu.reshape(w.B * w.H, w.N, w.d)
    flat_l = lse_gpu.reshape(w.B * w.H, w.N)
    idx = rows.to(o_gpu.device)
    og = torch.gather(flat_o, 1, idx[:, :, None].expand(-1, -1, w.d)).double().cpu().numpy()
    lg = torch.gather(flat_l, 1, idx).double().cpu().numpy()
    do = np.abs(og - o_ref.reshape(og.shape))
    dl = np.abs(lg - lse_ref.reshape(lg.shape))
    ref = o_ref.reshape(og.shape)
    half_ulp = np.where(ref == 0, 0.0, np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), np.abs(og)))[1] - 9))
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": "%d seeded query rows per head (%d of %d rows, rows 0 and N-1 included), "
                  "every visible key of each row; %.3g counted flops in %.1f s"
                  % (rows_per_head, rows.numel(), w.B * w.H * w.N, flops, dt),
        # the whole workload at the sample's rate (rows weighted by their visible keys)
        "extrapolated_all_rows_s": round(w.flops / (flops / dt), 1),
    }, {"rows": int(rows.numel()), "max_abs_dO": float(do.max()), "mean_abs_dO": float(do.mean()),
        "max_abs_dLSE": float(dl.max()), "n_over_relaxed": int((do > 1e-2 + half_ulp).sum())}


def parity_ok(par, literal_max=True):
    """The stated bars on a parity summary: max|dO| <= 1e-2 (literal where the
    rounding floor allows, else 1e-2 + half a bf16 ulp of |O|), mean|dO| <=
    1e-3, |dLSE| <= 1e-3."""
    max_ok = par["max_abs_dO"] <= 1e-2 if literal_max else par.get("n_over_relaxed", 0) == 0
    return bool(max_ok and par["mean_abs_dO"] <= 1e-3 and par["max_abs_dLSE"] <= 1e-3)


def bench_parity(args):
    """One JSON line per workload of WORKLOADS: attn_fwd in the bench's launch
    configuration against the fp64 oracle (every row of the first three
    workloads; the seeded row subsets of the large-logit and very long ones,
    rows 0 and N-1 included), with the literal max/mean |dO| and max |dLSE|
    next to the oracle-only bf16 rounding floor (|bf16(O_ref) - O_ref|) and
    the outcome under both the literal max bar and the 1e-2 + half-ulp one."""
    import numpy as np
    import torch

    import oracle
    from exact_io_aware_27_amd import attn, inputs

    attn.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    names = args.parity.split(",") if args.parity != "all" else [w.name for w in inputs.WORKLOADS]
    ok_all = True
    for w in inputs.WORKLOADS:
        if w.name not in names:
            continue
        q, k, v = inputs.workload_qkv(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        od = torch.empty_like(qd)
        lsed = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        attn.attn_fwd(qd, kd, vd, od, lsed, w.B, w.H, w.N, w.d, w.causal, w.scale, stream)
        torch.cuda.synchronize()
        rows = inputs.row_subsets(w) if w.rows_checked else None
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(q, k, v, w.causal, w.scale, rows=rows,
                                          nthreads=oracle.oracle.default_threads())
        dt = time.perf_counter() - t0
        if rows is None:
            og, lg = od.cpu(), lsed.cpu()
        else:
            flat_o = od.reshape(w.B * w.H, w.N, w.d)
            idx = rows.to(dev)
            og = torch.gather(flat_o, 1, idx[:, :, None].expand(-1, -1, w.d)).cpu()
            lg = torch.gather(lsed.reshape(w.B * w.H, w.N), 1, idx).cpu()
        o = og.double().numpy().reshape(o_ref.shape)
        lse = lg.double().numpy().reshape(lse_ref.shape)
        d_o = np.abs(o - o_ref)
        half_ulp = np.where(o_ref == 0, 0.0, np.ldexp(1.0, np.frexp(np.maximum(np.abs(o_ref), np.abs(o)))[1] - 9))
        floor = np.abs(torch.from_numpy(o_ref).to(torch.bfloat16).double().numpy() - o_ref)
        par = {"max_abs_dO": float(d_o.max()), "mean_abs_dO": float(d_o.mean()),
               "max_abs_dLSE": float(np.abs(lse - lse_ref).max()),
               "floor_max_abs": float(floor.max()), "floor_mean_abs": float(floor.mean()),
               "n_over_literal": int((d_o > 1e-2).sum()),
               "n_over_relaxed": int((d_o > 1e-2 + half_ulp).sum())}
        literal = parity_ok(par, literal_max=True)
        relaxed = parity_ok(par, literal_max=False)
        # the bar each workload is held to: literal, except the large-logit
        # one, whose rounding floor alone passes 1e-2
        held = relaxed if w.name == "large_logits" else literal
        ok_all = ok_all and held
        out = {"metric": "attn fwd parity vs fp64 oracle", "workload": w.describe(), "seed": w.seed,
               "rows": "all %d" % (w.B * w.H * w.N) if rows is None else
               "%d seeded per head (%d), rows 0 and N-1 included" % (w.rows_checked, rows.numel()),
               **par, "pass_literal": literal, "pass_relaxed_max": relaxed, "pass": held,
               "bars": {"max_abs_dO": 1e-2, "mean_abs_dO": 1e-3, "max_abs_dLSE": 1e-3},
               "oracle_s": round(dt, 1)}
        print(json.dumps(out), flush=True)
    return 0 if ok_all else 3


def bench_splitkv(args):
    """One JSON line for a split-KV workload (attn_fwd_splitkv): decode is
    bounded by HBM (K and V read once), one long head by the MFMAs.  The same
    problem with one key range is timed beside it."""
    import torch
    import numpy as np

    import oracle
    from exact_io_aware_27_amd import attn, inputs

    attn.load()
    w = {x.name: x for x in inputs.SPLITKV_WORKLOADS}[args.splitkv]
    splits = args.splits or w.splits
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = inputs.make_q_kv(w.B, w.H, w.Nq, w.Nk, w.d, w.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    nbytes = attn.splitkv_workspace_bytes(w.B, w.H, w.Nq, w.d, splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def timed(S):
        nb = attn.splitkv_workspace_bytes(w.B, w.H, w.Nq, w.d, S)

        def step():
            attn.attn_fwd_splitkv(qd, kd, vd, od, lsed, w.B, w.H, w.Nq, w.Nk, w.d, w.causal, w.scale, S,
                                  ws, nb, stream)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms1 = timed(1)
    ms = timed(splits)  # last: od and lsed hold the split result
    hbm_bound = w.Nq * 4 < w.Nk // 64  # a handful of queries per key: memory-bound
    if hbm_bound:
        metric, unit = "split-KV decode K/V read GB/s, 1 GPU", "GB/s"
        value = w.kv_bytes / (ms * 1e-3) / 1e9
        one_range = w.kv_bytes / (ms1 * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBPS, 4), "traffic": None}
    else:
        metric, unit = "split-KV attn fwd TFLOP/s, 1 GPU", "TFLOP/s"
        value = w.flops / (ms * 1e-3) / 1e12
        one_range = w.flops / (ms1 * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(value, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4), "traffic": None}
    out = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.describe(splits), "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                      "causal": w.causal, "splits": splits, "seed": w.seed},
           "roofline": roof, "one_range": {"value": round(one_range, 2), "unit": unit, "ms_per_step": round(ms1, 5)}}
    if args.cpu_rows > 0:
        R = min(w.Nq, w.rows_checked or w.Nq, args.cpu_rows)
        rows = torch.stack([inputs.row_subset(w.Nq, R, w.seed, bh, (0, w.Nq - 1)) for bh in range(w.B * w.H)])
        threads = oracle.oracle.default_threads()
        t0 = time.perf_counter()
        o_ref, lse_ref = oracle.attention(q, k, v, w.causal, w.scale, rows=rows, nthreads=threads)
        dt = time.perf_counter() - t0
        off = w.Nk - w.Nq
        keys = (rows + off + 1).double() if w.causal else torch.full(rows.shape, float(w.Nk), dtype=torch.float64)
        flops = float(keys.sum()) * 4 * w.d
        og = torch.gather(od.reshape(w.B * w.H, w.Nq, w.d), 1,
                          rows.to(dev)[:, :, None].expand(-1, -1, w.d)).double().cpu().numpy()
        lg = torch.gather(lsed.reshape(w.B * w.H, w.Nq), 1, rows.to(dev)).double().cpu().numpy()
        out["cpu_baseline"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                               "sample": "%d query rows per head (%d rows), every visible key; %.3g counted flops "
                                         "in %.1f s" % (R, rows.numel(), flops, dt)}
        out["parity_sampled_rows"] = {"rows": int(rows.numel()),
                                      "max_abs_dO": float(np.abs(og - o_ref.reshape(og.shape)).max()),
                                      "max_abs_dLSE": float(np.abs(lg - lse_ref.reshape(lg.shape)).max())}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def bench_bwd(args):
    """One JSON line for the backward pass (attn_bwd: the dQ kernel, then the
    dK/dV kernel) on a workload of WORKLOADS.  One step is one attn_bwd call
    over the whole batch; O and LSE come from one attn_fwd call before the
    timed region.  Counted work is the five products of the gradient
    definition (S, dP, dV, dK, dQ: 10*B*H*N^2*d, halved when causal); the
    kernels recompute S and dP in both passes (seven products), which the
    count does not credit."""
    import numpy as np
    import torch

    import oracle
    from exact_io_aware_27_amd import attn, inputs

    attn.load()
    w = {x.name: x for x in inputs.WORKLOADS}[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = inputs.workload_qkv(w)
    g = inputs.make_grad_out(w.B, w.H, w.N, w.d, seed=w.seed + 104729)
    qd, kd, vd, gd = q.to(dev), k.to(dev), v.to(dev), g.to(dev)
    stream = torch.cuda.current_stream(dev)
    od, lsed = attn.attention(qd, kd, vd, causal=w.causal, scale=w.scale, stream=stream)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    nb = attn.bwd_workspace_bytes(w.B, w.H, w.N, w.d)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step():
        attn.attn_bwd(qd, kd, vd, od, lsed, gd, dq, dk, dv, w.B, w.H, w.N, w.d, w.causal, w.scale, ws, nb,
                      stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 2.5 * w.flops
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"metric": "attn bwd TFLOP/s (5-product count) + % of bf16 MFMA peak, 1 GPU", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.describe() + " backward", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                      "causal": w.causal, "scale": w.scale, "seed": w.seed},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                        "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                        "kernels": "attn_bwd_dq_kernel + attn_bwd_dkdv_kernel, back to back"}}
    if args.cpu_heads > 0:
        # the oracle on whole heads (dK and dV need every query of a head)
        heads = [(b, h) for b in range(w.B) for h in range(w.H)][:args.cpu_heads]
        threads = min(len(heads), oracle.oracle.default_threads())
        sel = torch.tensor([b * w.H + h for b, h in heads])

        def pick(x):
            return x.reshape(w.B * w.H, *x.shape[2:])[sel].unsqueeze(0).contiguous()

        t0 = time.perf_counter()
        rq, rk, rv, _ = oracle.attention_bwd(pick(q), pick(k), pick(v), pick(g), w.causal, w.scale,
                                             nthreads=threads)
        dt = time.perf_counter() - t0
        head_flops = 2.5 * w.flops / (w.B * w.H)
        out["cpu_baseline"] = {"value": head_flops * len(heads) / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "%d whole head(s) of the workload, every query and key; %.3g counted "
                                         "flops in %.1f s" % (len(heads), head_flops * len(heads), dt)}
        rel = {}
        for name, x, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            xs = pick(x.cpu()).double().numpy()
            rel[name + "_max_rel"] = float(np.abs(xs - ref).max() / max(np.abs(ref).max(), 1e-30))
        out["parity_sampled_heads"] = dict(heads=len(heads), **rel)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def bench_fp8(args):
    """One JSON line for the FP8 forward (attn_fwd_fp8) on a workload of
    WORKLOADS (head dim 128).  Q and K are rotated with seeded random signs
    and quantized, V quantized and transposed, once before the timed region;
    one step is one attn_fwd_fp8 call.  The three quantization launches are
    timed separately, and the whole path (quantize Q, K, V + attention) too."""
    import numpy as np
    import torch

    from oracle import fp8_oracle as f8
    from exact_io_aware_27_amd import attn, inputs

    attn.load()
    w = {x.name: x for x in inputs.WORKLOADS}[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = inputs.workload_qkv(w)
    signs = inputs.make_signs(w.d, seed=w.seed + 1).numpy()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    stream = torch.cuda.current_stream(dev)
    q8, qe = attn.fp8_quantize(qd, signs=signs, stream=stream, scale=w.scale)
    k8, ke = attn.fp8_quantize(kd, signs=signs, stream=stream)
    vt8, ve = attn.fp8_quantize(vd, transpose=True, stream=stream)
    od = torch.empty_like(qd)
    lsed = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    def attend():
        attn.attn_fwd_fp8(q8, k8, vt8, qe, ke, ve, od, lsed, w.B, w.H, w.N, w.d, w.causal, stream)

    def quantize():
        attn.fp8_quantize_status(qd, w.B, w.H, w.N, w.d, False, signs, q8, qe, stream, w.scale)
        attn.fp8_quantize_status(kd, w.B, w.H, w.N, w.d, False, signs, k8, ke, stream)
        attn.fp8_quantize_status(vd, w.B, w.H, w.N, w.d, True, None, vt8, ve, stream)

    def timed(fn, steps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    qms = timed(quantize, max(1, args.steps // 2))
    ms = timed(attend, args.steps)  # last: od and lsed hold the result
    tflops = w.flops / (ms * 1e-3) / 1e12
    out = {"metric": "attn fwd FP8 TFLOP/s + % of fp8 MFMA peak, 1 GPU", "value": round(tflops, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8-e4m3", "data": "synthetic",
           "config": {"workload": w.describe() + " fp8 (block 64, incoherent processing)", "B": w.B, "H": w.H,
                      "N": w.N, "d": w.d, "causal": w.causal, "scale": w.scale, "seed": w.seed},
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(PEAK_FP8_TFLOPS, 1),
                        "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4), "traffic": None},
           "quantize_ms": round(qms, 5),
           "with_quantize_TFLOPs": round(w.flops / ((ms + qms) * 1e-3) / 1e12, 2)}
    if args.cpu_rows > 0:
        # the oracle's FP8 method on a row sample of one head: quantize the head
        # (rotation, blocks), then exact attention of the dequantized operands
        R = min(args.cpu_rows, w.N)
        rows = inputs.row_subset(w.N, R, w.seed, 0, (0, w.N - 1)).numpy()
        t0 = time.perf_counter()
        prep = f8.prepare_fp8(q[:1, :1], k[:1, :1], v[:1, :1], signs=signs, scale=w.scale)
        o_ref, lse_ref, sig = [], [], []
        for r in rows:
            hi = r + 1 if w.causal else w.N
            a, b_, c = f8.attention_fp64(prep["q"][:, :, [r]], prep["k"][:, :, :hi], prep["v"][:, :, :hi], False,
                                         prep["qk_mul"], p_rounding=True)
            o_ref.append(a), lse_ref.append(b_), sig.append(c)
        dt = time.perf_counter() - t0
        o_ref, lse_ref, sig = (np.concatenate(x, axis=2) for x in (o_ref, lse_ref, sig))
        keys = (rows + 1).sum() if w.causal else len(rows) * w.N
        flops = float(keys) * 4 * w.d
        og = od[0, 0, rows].double().cpu().numpy()[None, None]
        z = (og - o_ref) / np.sqrt(sig ** 2 + 1e-10)
        out["cpu_baseline"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                               "sample": "head (0, 0): quantization of the whole head, then %d seeded query rows "
                                         "against every visible key; %.3g counted flops in %.1f s" % (R, flops, dt)}
        out["parity_sampled_rows"] = {"rows": int(R), "mean_z2": float(np.mean(z ** 2)),
                                      "max_abs_z": float(np.abs(z).max()),
                                      "max_abs_dLSE": float(np.abs(lsed[0, 0, rows].double().cpu().numpy()
                                                                   - lse_ref[0, 0]).max())}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def bench_micro(args):
    """One JSON line of gfx950 issue rates (exact_io_aware_27_amd/micro.py):
    cycles per VALU instruction by kind and waves per SIMD, dependent-chain
    latencies, cycles per 32x32x16 bf16 MFMA when k FMAs and e
    exponentials follow each one, LDS read throughput, and cycles per MFMA
    when its operand comes from LDS in the attention step's issue order --
    the per-unit cycle count the attention kernels are designed against,
    measured in shader cycles."""
    import torch

    from exact_io_aware_27_amd import micro

    micro.load()
    torch.cuda.set_device(0)
    rates = []
    for op in ("fma", "mul", "exp", "poly"):
        for w in (1, 2, 4):
            r = micro.rate(op, w)
            print("rate %-4s waves/SIMD %d: %.2f cycles/inst per SIMD  (%.2f GHz)"
                  % (op, w, r["cycles_per_inst"], r["clock_ghz"]), file=sys.stderr, flush=True)
            rates.append(r)
        r = micro.rate(op, 1, dependent=True)
        print("latency %-4s: %.2f cycles per dependent element" % (op, r["cycles_per_element"]),
              file=sys.stderr, flush=True)
        rates.append(r)
    mixes = []
    for k, e, poly in micro.MIXES:
        for w in (1, 2):
            m = micro.mix(k, e, poly, w)
            print("mix %d fma + %d %s per MFMA, waves/SIMD %d: %.2f cycles/MFMA, %.0f TFLOP/s (%.2f GHz)"
                  % (k, e, m["exp"], w, m["cycles_per_mfma"], m["tflops"], m["clock_ghz"]),
                  file=sys.stderr, flush=True)
            mixes.append(m)
    for k, e, shape in micro.SHAPED_MIXES:
        for w in (1, 2):
            m = micro.mix(k, e, False, w, shape=shape)
            print("mix %d fma + %d exp per MFMA (%s), waves/SIMD %d: %.2f cycles/MFMA, %.0f TFLOP/s (%.2f GHz)"
                  % (k, e, m["shape"], w, m["cycles_per_mfma"], m["tflops"], m["clock_ghz"]),
                  file=sys.stderr, flush=True)
            mixes.append(m)
    lds_rates = []
    for kind in (0, 1):
        for w in (1, 2, 4):
            r = micro.lds_rate(kind, w)
            print("lds %-18s waves/SIMD %d: %.1f bytes/cycle per CU  (%.2f GHz)"
                  % (r["read"], w, r["bytes_per_cycle_per_cu"], r["clock_ghz"]), file=sys.stderr, flush=True)
            lds_rates.append(r)
    lds_mixes = []
    for kind in (0, 1, 2):
        for w in (1, 2):
            m = micro.mix_lds(kind, w)
            print("MFMA with its operand from LDS (%s), waves/SIMD %d: %.2f cycles/MFMA, %.0f TFLOP/s (%.2f GHz)"
                  % (m["operand"], w, m["cycles_per_mfma"], m["tflops"], m["clock_ghz"]), file=sys.stderr,
                  flush=True)
            lds_mixes.append(m)
    hbm = []
    for blocked in (False, True):
        for wgs in (512, 1024, 2048, 4096, 8192):
            h = micro.hbm_read(4096, wgs, blocked)
            print("hbm read stream, 4 GiB, %d workgroups of 256, %s: %.0f GB/s"
                  % (wgs, "one slice per workgroup" if blocked else "grid-interleaved", h["GBps"]),
                  file=sys.stderr, flush=True)
            hbm.append(h)
    out = {"metric": "gfx950 issue rates (shader cycles), 1 GPU", "unit": "cycles", "rates": rates,
           "mixes": mixes, "lds_rates": lds_rates, "lds_mixes": lds_mixes, "hbm_read": hbm, "note": "rate: per SIMD over all its waves (independent chains) or per dependent "
                                  "instruction; mix: per 32x32x16 bf16 MFMA per SIMD (32 = matrix-core rate)"}
    print(json.dumps(out), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="long_causal",
                    help="name of a workload in exact_io_aware_27_amd.inputs.WORKLOADS")
    ap.add_argument("--cpu-rows", type=int, default=5120,
                    help="query rows per head in the oracle's CPU-baseline sample (0: skip)")
    ap.add_argument("--splitkv", default=None,
                    help="measure attn_fwd_splitkv on a workload of exact_io_aware_27_amd.inputs.SPLITKV_WORKLOADS")
    ap.add_argument("--splits", type=int, default=0, help="key ranges for --splitkv (0: the workload's)")
    ap.add_argument("--bwd", action="store_true", help="measure the backward pass (attn_bwd) on --workload")
    ap.add_argument("--fp8", action="store_true", help="measure the FP8 forward (attn_fwd_fp8) on --workload")
    ap.add_argument("--parity", default=None, metavar="WORKLOADS",
                    help="parity report against the fp64 oracle: 'all' or comma-separated workload names; "
                         "one JSON line per workload (exit 3 if one fails its bar)")
    ap.add_argument("--lib", default=None,
                    help="load this libattn.so instead of the in-tree one (A/B of build "
                         "options, see exact_io_aware_27_amd/build.py --out)")
    ap.add_argument("--micro", action="store_true",
                    help="gfx950 issue-rate microbenchmarks (VALU, exp, exp2_poly, MFMA mixes) in shader cycles")
    ap.add_argument("--cpu-heads", type=int, default=1,
                    help="--bwd: whole heads in the oracle's CPU-baseline sample (0: skip)")
    ap.add_argument("--per-launch", action="store_true",
                    help="add each timed launch's duration, in launch order, as ms_launches")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter CSVs (FETCH_SIZE run, WRITE_SIZE run, "
                         "both with --copy-calibration-mib) into HBM bytes per launch")
    args = ap.parse_args()

    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1],
                                     args.copy_calibration_mib or 1024)))
        return 0

    if args.lib:
        from exact_io_aware_27_amd import attn
        attn.LIB_PATH = os.path.abspath(args.lib)

    if args.gpus != 1:
        print("bench.py: the attention library runs on one GPU only; --gpus %d is not supported "
              "(the path has no multi-GPU mode)" % args.gpus, file=sys.stderr)
        return 2

    if args.splitkv:
        return bench_splitkv(args)
    if args.bwd:
        return bench_bwd(args)
    if args.fp8:
        return bench_fp8(args)
    if args.micro:
        return bench_micro(args)
    if args.parity:
        return bench_parity(args)

    import torch

    from exact_io_aware_27_amd import attn, inputs

    if not os.path.exists(attn.LIB_PATH):
        from exact_io_aware_27_amd import build
        build.build()
    attn.load()

    w = {x.name: x for x in inputs.WORKLOADS}[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = inputs.workload_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)  # an elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    # The binding's tensor checks once, then every step calls the C ABI with
    # the same marshalled arguments (and checks its status): the per-call
    # Python checks would otherwise show as gaps between the short launches
    # of the small workloads.
    shape = (w.B, w.H, w.N, w.d)
    for x, name in ((qd, "q"), (kd, "k"), (vd, "v"), (od, "o")):
        attn._check(x, name, shape, torch.bfloat16)
    attn._check(lsed, "lse", shape[:3], torch.float32)
    lib = attn.load()
    import ctypes
    raw = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), od.data_ptr(), lsed.data_ptr(), w.B, w.H, w.N, w.d,
           1 if w.causal else 0, ctypes.c_float(w.scale), ctypes.c_void_p(stream.cuda_stream))

    def step():
        st = lib.attn_fwd(*raw)
        if st:
            raise attn.AttnError(st, lib.attn_last_hip_error())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one event before the first timed launch and one after each: the first to
    # the last bracket exactly the timed steps (their mean is ms_per_step);
    # neighbours give each launch's own duration
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    events[0].record(stream)
    for i in range(args.steps):
        step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = events[0].elapsed_time(events[-1]) / args.steps  # one kernel per step: average launch duration
    in_order = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    per_launch = sorted(in_order)
    ms_median = per_launch[len(per_launch) // 2] if len(per_launch) % 2 else \
        0.5 * (per_launch[len(per_launch) // 2 - 1] + per_launch[len(per_launch) // 2])

    tflops = w.flops / (ms * 1e-3) / 1e12
    compulsory = w.B * w.H * (8 * w.N * w.d + 4 * w.N)  # Q,K,V read + O write (bf16) + LSE (fp32)
    traffic = measured_traffic() if not args.lib else None  # counters are of the in-tree build
    props = torch.cuda.get_device_properties(dev)
    out = {
        # the headline metric on its own workload; another workload names itself
        "metric": METRIC if w.name == "long_causal" else
        "attn fwd TFLOP/s + %% of bf16 MFMA peak, 1 GPU, %s" % w.describe(),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_median": round(ms_median, 5),
        "ms_min": round(per_launch[0], 5),
        "ms_max": round(per_launch[-1], 5),
        **({"ms_launches": [round(x, 5) for x in in_order]} if args.per_launch else {}),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.describe(), "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "seed": w.seed,
                   "sigma_qk": w.sigma_qk, "sigma_v": w.sigma_v},
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "hbm": {"compulsory_bytes": compulsory,
                "compulsory_GBps": round(compulsory / (ms * 1e-3) / 1e9, 1),
                "measured_bytes": traffic,
                "measured_GBps": (round(traffic / (ms * 1e-3) / 1e9, 1) if traffic else None),
                "peak_GBps": HBM_PEAK_GBPS},
        "device": device_info(props),
        "kernel_hash": kernel_hash() if not args.lib else None,
        "library": os.path.relpath(attn.LIB_PATH, ROOT),
        "context_other_hardware": {
            "FlashAttention-2, A100, TFLOP/s": 225, "FlashAttention-3 FP16 fwd, H100 SXM5, TFLOP/s": 740,
            "FlashAttention-4 BF16, B200, TFLOP/s": 1613},
    }
    status = 0
    if args.cpu_rows > 0:
        cb, par = cpu_baseline(w, q, k, v, od, lsed, args.cpu_rows)
        par["pass"] = parity_ok(par, literal_max=w.name != "large_logits")
        out["cpu_baseline"] = cb
        out["parity_sampled_rows"] = par
        if not par["pass"]:
            status = 3  # the timed launch's output broke the parity bars
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    if status:
        print("bench.py: the timed launch's output fails the parity bars: %s" % out["parity_sampled_rows"],
              file=sys.stderr, flush=True)
    return status


if __name__ == "__main__":
    sys.exit(main())
