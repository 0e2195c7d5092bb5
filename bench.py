#!/usr/bin/env python3
"""One-GPU benchmark of exact tiled attention (forward + recompute backward) on MI355X.

    python bench.py [--gpus 1] [--steps 60] [--warmup 5] [--workload large_head_causal]

A step is one pass of the whole path over the workload's synthetic inputs, already
resident in HBM: fa_forward, then the two backward stages (fa_backward_dq,
fa_backward_dkdv -- exactly what fa_backward runs).  The default workload is causal
bf16 attention with B=2, H=16, N=8192, d=128 (5% of Q and K rows scaled by 8).

Printed: one JSON line on stdout.  `value` is credited TFLOP/s of the whole step:
forward 4*B*H*N^2*d and backward 10*B*H*N^2*d (five N x N x d products including the
recomputation of S), both halved for causal masking.  `roofline` describes the
kernel with the largest share of the step's time: its algorithmic flops per launch
(kernel_flops: the products that kernel needs on its own) over its average launch
time, measured here with HIP events on the stream the kernels run on, against the
MI355X dense bf16 MFMA peak (2516.6 TFLOP/s).
`cpu_baseline` times the fp64 CPU oracle on a few heads of the same workload.
"""

from __future__ import annotations

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

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "exact_tiled_attention_forward_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    """sha256 over the HIP/C++ sources of libfa.so (ties stored counter data to a build)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


KERNEL_KEYS = (("fwd16_kernel", "fwd"), ("fwd16_pp_kernel", "fwd"), ("fwd32_kernel", "fwd"), ("bwd_dq_kernel", "bwd_dq"),
               ("bwd_dkdv_kernel", "bwd_dkdv"))


def kernel_key(name: str):
    """Bench name of a library kernel from its demangled name (None for other kernels)."""
    for frag, key in KERNEL_KEYS:
        if f"fa::{frag}" in name:
            return key
    return None


def algorithmic_bytes(w):
    """HBM bytes each kernel must move at least: its inputs read once, its outputs written
    once.  fwd reads Q, K, V and writes O and the logsumexp; bwd_dq reads Q, K, V, dO and
    the logsumexp and writes fp32 dQ plus D and lse*log2(e); bwd_dkdv reads Q, K, V, dO, D
    and lse*log2(e) and writes fp32 dK, dV."""
    s = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    qrows, kvrows = w.B * w.H * w.N, w.B * w.Hkv * w.Nk
    return {"fwd": qrows * (2 * w.d * s + 4) + kvrows * 2 * w.d * s,
            "bwd_dq": qrows * (2 * w.d * s + 4 + 4 * w.d + 8) + kvrows * 2 * w.d * s,
            "bwd_dkdv": qrows * (2 * w.d * s + 8) + kvrows * (2 * w.d * s + 8 * w.d)}


def _read_counters(path):
    """{kernel key or 'copy': {counter: [value per dispatch]}} from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            key = "copy" if "copyBuffer" in name else kernel_key(name)
            if key is None:
                continue
            out.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_csv, write_csv, w, copy_mb, command):
    """Write profiles/traffic_<kernel>_<workload>.txt from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch), each scaled by what the same counter reads for a
    device-to-device copy of copy_mb MiB run in the same process."""
    fetch, write = _read_counters(fetch_csv), _read_counters(write_csv)
    mean = lambda v: sum(v) / len(v)
    copy_bytes = copy_mb * 2.0 ** 20
    f_scale = copy_bytes / (mean(fetch["copy"]["FETCH_SIZE"]) * 1024)
    w_scale = copy_bytes / (mean(write["copy"]["WRITE_SIZE"]) * 1024)
    alg = algorithmic_bytes(w)
    digest = kernel_source_digest()
    written = []
    for key in ("fwd", "bwd_dq", "bwd_dkdv"):
        if key not in fetch or key not in write:
            continue
        fk, wk = mean(fetch[key]["FETCH_SIZE"]), mean(write[key]["WRITE_SIZE"])
        traffic = fk * 1024 * f_scale + wk * 1024 * w_scale
        path = os.path.join(PROFILES, f"traffic_{key}_{w.name}.txt")
        with open(path, "w") as f:
            f.write(f"# HBM traffic of the {key} kernel on {w.name} (B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}"
                    f"{' causal' if w.causal else ''}), rocprofv3 derived counters per dispatch\n")
            f.write(f"kernel: {key}\nworkload: {w.name}\nsource_sha256: {digest}\n")
            f.write(f"dispatches: {len(fetch[key]['FETCH_SIZE'])}\n")
            f.write(f"fetch_kib_per_dispatch: {fk:.1f}\nwrite_kib_per_dispatch: {wk:.1f}\n")
            f.write(f"copy_calibration: device-to-device copy of {copy_mb} MiB reads "
                    f"{mean(fetch['copy']['FETCH_SIZE']):.1f} KiB and writes {mean(write['copy']['WRITE_SIZE']):.1f} KiB "
                    f"per dispatch (expected {copy_bytes / 1024:.1f})\n")
            f.write(f"fetch_scale: {f_scale:.4f}\nwrite_scale: {w_scale:.4f}\n")
            f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
            f.write(f"algorithmic_bytes_per_launch: {alg[key]}\n")
            f.write(f"traffic_over_algorithmic: {traffic / alg[key]:.3f}\n")
            f.write(f"command: {command}\n")
        written.append(path)
    return written


def counters_summary(csvs, w, command):
    """profiles/counters_<kernel>_<workload>.txt: the mean per dispatch of every counter that
    rocprofv3 --pmc collected for each library kernel (one CSV per counter pass)."""
    vals = {}
    for path in csvs:
        for key, counters in _read_counters(path).items():
            if key == "copy":
                continue
            for cname, v in counters.items():
                vals.setdefault(key, {})[cname] = (sum(v) / len(v), len(v))
    written = []
    for key, counters in vals.items():
        path = os.path.join(PROFILES, f"counters_{key}_{w.name}.txt")
        with open(path, "w") as f:
            f.write(f"# rocprofv3 counters of the {key} kernel on {w.name} (B={w.B} H={w.H} N={w.N} d={w.d} "
                    f"{w.dtype}{' causal' if w.causal else ''}), mean per dispatch over all SEs/XCDs\n")
            f.write(f"source_sha256: {kernel_source_digest()}\ncommand: {command}\n")
            for cname in sorted(counters):
                m, n = counters[cname]
                f.write(f"{cname}: {m:.6g}   (dispatches: {n})\n")
            c = {k: v[0] for k, v in counters.items()}
            if "SQ_INSTS_MFMA" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                f.write(f"derived_mfma_busy_cycles_per_instruction: "
                        f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / c['SQ_INSTS_MFMA']:.2f}\n")
            if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c:
                f.write(f"derived_valu_instructions_per_mfma: {(c['SQ_INSTS_VALU'] - c['SQ_INSTS_MFMA']) / c['SQ_INSTS_MFMA']:.2f}\n")
            if "SQ_LDS_BANK_CONFLICT" in c and "SQ_INSTS_LDS" in c:
                f.write(f"derived_lds_bank_conflict_cycles_per_lds_instruction: "
                        f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_INSTS_LDS'], 1):.4f}\n")
        written.append(path)
    return written


def trace_summary(stats_csv, bench_log, w, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this script."""
    import csv
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            if kernel_key(r["Name"]) is None:
                continue
            name = r["Name"].split("(")[0].replace("void ", "")
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    line = None
    with open(bench_log) as f:
        for ln in f:
            if ln.startswith("{") and '"metric"' in ln:
                line = json.loads(ln)
    path = os.path.join(PROFILES, f"kernel_trace_{w.name}.md")
    with open(path, "w") as f:
        f.write(f"# Kernel trace: {w.name} (B={w.B}, H={w.H}, N={w.N}, d={w.d}, {w.dtype}"
                f"{', causal' if w.causal else ''}), {'forward + backward' if w.backward else 'forward'}\n\n")
        f.write(f"Command (from the repository root on one MI355X):\n\n```\n{command}\n```\n\n")
        f.write("| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |\n|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| `{r[0]}` | {r[1]} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} | {r[5]:.1f}% |\n")
        if line:
            f.write("\nHIP-event averages measured inside the same run (ms): "
                    + ", ".join(f"{k} {v}" for k, v in line["kernel_ms"].items()) + "\n")
            f.write(f"Bench line: value {line['value']} TFLOP/s ({line['pct_of_peak']}% of {PEAK_BF16_TFLOPS}), "
                    f"forward {line['fwd_tflops']} TFLOP/s ({line['fwd_pct_of_peak']}%), roofline kernel "
                    f"{line['roofline']['kernel']} at {line['roofline']['achieved']} TFLOP/s algorithmic.\n")
    return path


def read_sclk():
    """Current shader clock level from sysfs (e.g. '2400Mhz'), or None where unreadable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for ln in f:
                    if ln.rstrip().endswith("*"):
                        return ln.split(":", 1)[1].strip(" *\n")
        except OSError:
            continue
    return None


def sweep(names, reps: int, out_path: str):
    """Time fa_forward (and the backward stages) of each workload with HIP events on the
    stream they run on: median and min over `reps` samples, each the mean of a burst of
    back-to-back launches of at least about 1 ms ("warm": inputs may sit in the 256 MB
    last-level cache) and, for workloads whose inputs fit in that cache, single launches
    each after a 512 MB fill ("cold")."""
    import torch
    import exact_tiled_attention_forward_amd as fa
    from exact_tiled_attention_forward_amd.workloads import (WORKLOADS, elem_bytes, workload_block_mask,
                                                             workload_inputs)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    rows = []
    for name in names:
        w = WORKLOADS[name]
        inp = workload_inputs(w)
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        ns = fa.fa_forward_split_count(q, k, w.causal)
        wsf = None
        if ns > 1:
            nbytes = fa.library().fa_forward_split_workspace_bytes(w.B, w.H, w.N, w.d, ns)
            wsf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        bm = workload_block_mask(w)
        bm = bm.to(dev) if bm is not None else None
        passes = {"fwd": lambda: fa.fa_forward(q, k, v, o, lse, causal=w.causal, stream=stream, split=ns,
                                               workspace=wsf, block_mask=bm)}
        if bm is not None:
            passes["fwd dense"] = lambda: fa.fa_forward(q, k, v, o, lse, causal=w.causal, stream=stream, split=ns,
                                                        workspace=wsf)
        if name in ("large_head_causal", "long_bf16") and w.dtype == "bf16":
            # the same workload through the E4M3 path (inputs quantized beforehand, not timed)
            q8, qs8 = fa.fa_quantize_fp8(q)
            k8, ks8 = fa.fa_quantize_fp8(k)
            v8, vs8 = fa.fa_quantize_fp8(v, per_channel=True)
            o8 = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            passes["fwd fp8"] = lambda: fa.fa_forward_fp8(q8, qs8, k8, ks8, v8, vs8, o8, lse, causal=w.causal,
                                                          stream=stream)
        if w.backward:
            do = inp["do"].to(dev)
            f32 = torch.float32
            dq = torch.empty(q.shape, dtype=f32, device=dev)
            dk, dv = (torch.empty(k.shape, dtype=f32, device=dev) for _ in range(2))
            ws = torch.empty(fa.fa_backward_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
            passes["fwd"]()
            passes["bwd"] = lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, causal=w.causal, workspace=ws,
                                                 stream=stream, block_mask=bm)
            if bm is not None:
                passes["bwd dense"] = lambda: fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, causal=w.causal,
                                                             workspace=ws, stream=stream)
        s = elem_bytes(w.dtype)
        unit = 2.0 * w.B * w.H * w.visible_pairs() * w.d
        qrows, kvrows = w.B * w.H * w.N, w.B * w.Hkv * w.Nk
        info = {"fwd": (2 * unit, qrows * (2 * w.d * s + 4) + kvrows * 2 * w.d * s),
                "bwd": (5 * unit, qrows * (3 * w.d * s + 4 * w.d + 8) + kvrows * (2 * w.d * s + 8 * w.d)),
                "3step": (2 * unit, qrows * (2 * w.d * s + 4) + kvrows * 2 * w.d * s)}
        info["fwd dense"], info["bwd dense"] = info["fwd"], info["bwd"]
        info["fwd fp8"] = (info["fwd"][0], qrows * (d8 := w.d) + kvrows * 2 * d8 + qrows * (2 * d8 + 4))
        if w.N <= 16:
            # the plain three-step path for comparison: S = Q K^T, softmax, P V as library calls
            G = w.H // w.Hkv
            qg = q.view(w.B, w.Hkv, G * w.N, w.d)
            kt = k.transpose(-1, -2).contiguous()
            vc = v.contiguous()
            sc = 1.0 / math.sqrt(w.d)

            def three_step():
                sm = torch.matmul(qg, kt).float() * sc
                p = torch.softmax(sm, dim=-1).to(q.dtype)
                return torch.matmul(p, vc)
            passes["3step"] = three_step
        small = 2 * (qrows + kvrows) * w.d * s < (256 << 20)  # inputs and outputs fit the 256 MB MALL
        for pname, fn in passes.items():
            for mode in (["warm", "cold"] if small else ["warm"]):
                for _ in range(10):
                    fn()
                # warm: each sample times `burst` launches back to back (at least about 1 ms of
                # work), so that host launch gaps do not count; cold: one launch right after the
                # fill, which keeps the queue busy until the launch starts
                burst = 1
                if mode == "warm":
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(5):
                        fn()
                    b.record(stream)
                    b.synchronize()
                    burst = max(1, min(50, int(math.ceil(1.0 / (a.elapsed_time(b) / 5)))))
                ts = []
                for _ in range(reps):
                    if mode == "cold":
                        flush.fill_(1)
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    for _ in range(burst):
                        fn()
                    b.record(stream)
                    b.synchronize()
                    ts.append(a.elapsed_time(b) / burst)
                ts.sort()
                med, mn = ts[len(ts) // 2], ts[0]
                flops, nbytes = info[pname]
                if bm is not None and pname in ("fwd", "bwd"):
                    flops *= float(bm.float().mean())  # the visible blocks' share of the work
                shape = f"{w.B}x{w.H}x{w.N}x{w.d}" if (w.Hkv, w.Nk) == (w.H, w.N) else \
                    f"{w.B}x{w.H}/{w.Hkv}x{w.N}/{w.Nk}x{w.d}"
                rows.append({"workload": name, "shape": shape, "dtype": w.dtype,
                             "causal": w.causal, "pass": pname + (f" (split {ns})" if pname == "fwd" and ns > 1 else ""), "mode": mode, "median_us": med * 1e3,
                             "min_us": mn * 1e3, "tflops": flops / (med * 1e-3) / 1e12,
                             "pct_peak": 100 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                             "gbs": nbytes / (med * 1e-3) / 1e9})
                log(f"{name} {pname} {mode}: {med * 1e3:.1f} us")
        del q, k, v, o, lse, inp
    sclk = read_sclk()
    with open(out_path, "w") as f:
        f.write("# Timing of every workload on one MI355X (HIP events on the launch stream)\n\n")
        f.write(f"Command: `python3 bench.py --sweep --sweep-reps {reps}`; shader clock level read after the run: "
                f"{sclk or 'not readable'}.\n")
        f.write("TFLOP/s use 4BHN^2d (forward) and 10BHN^2d (backward), halved when causal; % of the 2516.6 "
                "TFLOP/s bf16/fp16 dense MFMA peak (fp32 rows: the same figure, for comparison only); GB/s are "
                "algorithmic bytes (inputs read once, outputs written once) over the median time.  warm = the mean "
                "of a burst of back-to-back launches (at least about 1 ms of work per sample, so host launch "
                "gaps do not count); cold = one launch right after a 512 MB fill.  Shapes with a slash are query/key-value heads and query/key rows; "
                "3step is the plain S = QK^T, softmax, PV path as three library calls (torch matmul and softmax), "
                "timed for comparison on decode shapes.  block_sparse_local and block_sparse_butterfly run under their block masks (TFLOP/s "
                "count the visible blocks only) and again dense for comparison.  fwd fp8 is the same workload through "
                "the E4M3 path (fa_forward_fp8 on inputs quantized beforehand); its % peak is against the bf16 "
                "peak (the fp8 dense peak is twice that).\n\n")
        f.write("| workload | B x H x N x d | dtype | causal | pass | mode | median (us) | min (us) | TFLOP/s "
                "| % peak | GB/s |\n|---|---|---|---|---|---|---|---|---|---|---|\n")
        for r in rows:
            f.write(f"| {r['workload']} | {r['shape']} | {r['dtype']} | {'yes' if r['causal'] else 'no'} | {r['pass']} "
                    f"| {r['mode']} | {r['median_us']:.1f} | {r['min_us']:.1f} | {r['tflops']:.1f} | "
                    f"{r['pct_peak']:.1f} | {r['gbs']:.0f} |\n")
    return out_path


def product_flops(w):
    """Flops of one N x N x d product of the workload (half of it when causal)."""
    return 2.0 * w.B * w.H * w.visible_pairs() * w.d


def credited_flops(w):
    """Credited flops of the step's passes: the forward's two products (S = QK^T, O = PV)
    and the backward's five (S, dP = dO V^T, dV, dK, dQ)."""
    unit = product_flops(w)
    return {"fwd": 2 * unit, "bwd": 5 * unit}


def kernel_flops(w):
    """Algorithmic flops of each kernel per launch, as a kernel of its own: the forward
    computes S and PV; the dQ kernel, which produces dQ from Q, K, V, dO and the logsumexp,
    needs S, dP and dQ; the dK/dV kernel needs S, dP, dV and dK.  The two backward kernels
    together count S and dP twice (the recomputation their split costs), so this per-kernel
    figure feeds the roofline only; the step's value uses credited_flops."""
    unit = product_flops(w)
    return {"fwd": 2 * unit, "bwd_dq": 3 * unit, "bwd_dkdv": 4 * unit}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_vendor() -> str:
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg["Build Dependencies"]["blas"]
        return f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:  # pragma: no cover - older numpy
        return "unknown"


def cpu_baseline(w, inp, heads: int):
    """Time the fp64 oracle (forward, and backward where the workload has one) on `heads`
    heads of the workload.  The oracle materialises the full N x N score matrix and skips
    no masked work, so its rate is counted over the dense work it does: 4 N^2 d flop per
    head for the forward and 10 N^2 d for the backward (not halved for causal masking)."""
    from oracle import naive
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = [i for i in info if i.get("user_api") == "blas"]
        cores = int(blas[0]["num_threads"]) if blas else len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = len(os.sched_getaffinity(0))
    picks = [(b, h) for b in range(w.B) for h in range(w.H)][:heads]
    arrs = {x: inp[x].double().numpy() for x in ("q", "k", "v", "do") if x in inp}
    t0 = time.perf_counter()
    for b, h in picks:
        g = h // (w.H // w.Hkv)
        naive.forward_head(arrs["q"][b, h], arrs["k"][b, g], arrs["v"][b, g], w.scale, w.causal)
        if w.backward:
            naive.backward_head(arrs["q"][b, h], arrs["k"][b, g], arrs["v"][b, g], arrs["do"][b, h], w.scale,
                                w.causal)
    secs = time.perf_counter() - t0
    dense_per_head = (4 + (10 if w.backward else 0)) * float(w.N) * w.Nk * w.d
    return {
        "value": dense_per_head * len(picks) / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{len(picks)} of {w.B * w.H} heads of {w.name}, fp64 numpy, "
                  f"{'forward + backward' if w.backward else 'forward'}, {secs:.1f} s; rate over the oracle's "
                  f"dense work ({4 + (10 if w.backward else 0)} N^2 d flop per head, not halved for causal)",
        "seconds": round(secs, 3),
        "cpu_model": _cpu_model(),
        "blas": _blas_vendor(),
        "heads_per_second": len(picks) / secs,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_head_causal")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads of the CPU oracle sample (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run device-to-device copies of MIB MiB (a known-traffic kernel for "
                         "rocprofv3 --pmc calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write profiles/traffic_*.txt from two rocprofv3 --pmc runs")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="no GPU: write profiles/kernel_trace_<workload>.md from a --kernel-trace --stats run")
    ap.add_argument("--counters-summary", nargs="+", metavar="CSV",
                    help="no GPU: write profiles/counters_*.txt from rocprofv3 --pmc runs")
    ap.add_argument("--command", default="", help="command line recorded in the summaries")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload (forward, backward) and write profiles/timing_all_workloads.md")
    ap.add_argument("--sweep-reps", type=int, default=50)
    args = ap.parse_args()

    if args.pmc_summary or args.trace_summary or args.counters_summary:
        from exact_tiled_attention_forward_amd.workloads import WORKLOADS
        w = WORKLOADS[args.workload]
        if args.pmc_summary:
            for p in pmc_summary(*args.pmc_summary, w, args.copy_calibration, args.command):
                log("wrote", p)
        if args.trace_summary:
            log("wrote", trace_summary(*args.trace_summary, w, args.command))
        if args.counters_summary:
            for p in counters_summary(args.counters_summary, w, args.command):
                log("wrote", p)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU only: attention shards over (batch, head) with no exchange, "
            "and this library has no multi-GPU path.  Run with --gpus 1.")
        sys.exit(2)

    if args.sweep:
        names = ["single_head_f32", "prefill_bf16", "gpt2_medium_train", "long_f16", "long_bf16", "large_head_causal",
                 "gqa_causal_train", "decode_gqa", "block_sparse_local", "block_sparse_butterfly"]
        log("wrote", sweep(names, args.sweep_reps, os.path.join(PROFILES, "timing_all_workloads.md")))
        return

    import torch
    import exact_tiled_attention_forward_amd as fa
    from exact_tiled_attention_forward_amd.workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    inp = workload_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    do = inp["do"].to(dev) if w.backward else None
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if w.backward:
        f32 = torch.float32
        dq, dk, dv = (torch.empty(q.shape, dtype=f32, device=dev) for _ in range(3))
        ws = torch.empty(fa.fa_backward_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = ["fwd"] + (["bwd_dq", "bwd_dkdv"] if w.backward else [])

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        fa.fa_forward(q, k, v, o, lse, causal=w.causal, stream=stream)
        if evs:
            evs[1].record(stream)
        if w.backward:
            fa.fa_backward_dq(q, k, v, do, lse, dq, causal=w.causal, workspace=ws, stream=stream)
            if evs:
                evs[2].record(stream)
            fa.fa_backward_dkdv(q, k, v, do, ws, dk, dv, causal=w.causal, stream=stream)
            if evs:
                evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    kernel_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j, n in enumerate(names)}
    step_samples = sorted(e[0].elapsed_time(e[-1]) for e in evs)
    kernel_samples = {n: sorted(e[j].elapsed_time(e[j + 1]) for e in evs) for j, n in enumerate(names)}
    med = lambda v: v[len(v) // 2]  # noqa: E731

    flops = kernel_flops(w)
    credited = credited_flops(w)
    step_flops = credited["fwd"] + (credited["bwd"] if w.backward else 0.0)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    dom = max(names, key=lambda n: kernel_ms[n])
    achieved = flops[dom] / (kernel_ms[dom] * 1e-3) / 1e12
    fwd_tf = flops["fwd"] / (kernel_ms["fwd"] * 1e-3) / 1e12
    line = {
        "metric": "attention fwd/bwd TFLOPS and % of MI355X bf16 MFMA peak, causal N=8192",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) Q, K, V, dO rounded to the storage dtype" +
                (f"; {w.outlier_frac:.0%} of Q and K rows x{w.outlier_scale:g}" if w.outlier_frac else ""),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "passes": "forward+backward" if w.backward else "forward"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_pct_of_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
        "ms_per_step_median": round(med(step_samples), 4),
        "ms_per_step_min": round(step_samples[0], 4),
        "timed_ms": round(total_ms, 2),
        "kernel_ms": {n: round(t, 4) for n, t in kernel_ms.items()},
        "kernel_ms_median": {n: round(med(v), 4) for n, v in kernel_samples.items()},
        "kernel_ms_min": {n: round(v[0], 4) for n, v in kernel_samples.items()},
        "sclk": read_sclk(),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": stored_traffic(dom, w.name),
        },
    }
    if w.backward:
        bwd_ms = kernel_ms["bwd_dq"] + kernel_ms["bwd_dkdv"]
        bwd_tf = credited["bwd"] / (bwd_ms * 1e-3) / 1e12
        line["bwd_tflops"] = round(bwd_tf, 2)
        line["bwd_pct_of_peak"] = round(100 * bwd_tf / PEAK_BF16_TFLOPS, 2)
    log(f"{w.name}: step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s; kernels (ms): "
        + ", ".join(f"{n} {t:.3f}" for n, t in kernel_ms.items()))
    if args.copy_calibration > 0:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.cpu_heads > 0:
        log(f"timing the fp64 CPU oracle on {args.cpu_heads} heads ...")
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_heads)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
