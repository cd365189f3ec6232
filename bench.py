#!/usr/bin/env python3
"""Benchmark of the four-over-six NVFP4 quantizer on one MI355X.

One step is one pass of the hot path over the dense-activation workload
(bf16 8192x4096 drawn from N(0,1), 1x16 blocks, per-tensor global scale,
four-over-six with MSE exact error, E4M3 bound 448): the NaN-dropping tensor
amax and the quantize writing packed E2M1 codes and E4M3 scales, in one
launch (fos_quantize_fused). Inputs rotate over enough resident copies that
the footprint exceeds the 256 MB Infinity Cache, so every step reads from HBM.

`value` is the step's algorithmic HBM traffic over the measured step time.
The step's kernel holds the tensor on chip between the amax and the
quantize, so x is read once: 2 B/elem in, 0.5 + 1/16 B/elem out. The
`roofline`
object covers the step's kernel, timed with HIP events on the stream it runs
on. `cpu_baseline` times the CPU oracle on the same workload. The quantize
kernel alone with a precomputed amax (the pages' kernel metric), the
two-launch step and the other configurations (16x16 weights, the fused-QDQ
expert list, the grouped MoE tensor) are timed briefly and reported under
`other_workloads`.

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD public spec
PEAK_VALU_LANE_TPS = 256 * 64 * 2.4e9  # VALU lane-instructions/s: 256 CUs x 64 lanes x 2.4 GHz
MALL_BYTES = 256 << 20
FOOTPRINT = 1 << 30            # rotate buffers up to >= 1 GiB
METRIC = "4over6 quantize/QDQ achieved HBM GB/s and % of MI355X peak (bit-exact)"
FUSED_KERNEL = "void fos::k_fused_onchip<0, 1, 1, 0, 0, 0>(fos::Args1x16<1>, unsigned int*, float*)"
QUANT_KERNEL = "void fos::k_1x16<1, 0, 1, 1, 0, 0, 0, 0>(fos::Args1x16<1>)"
COPY_BYTES = 256 << 20         # the profile pass's calibration copy
# counter summaries per kernel: (file, readable workload, algorithmic bytes per launch)
_N = 8192 * 4096
COUNTER_FILES = {
    FUSED_KERNEL: (os.path.join(ROOT, "profiles", "fused_amax_quantize_bf16_8192x4096_counters.txt"),
                   "fos_quantize_fused: per-tensor amax and quantize in one launch, one read of x", _N * 2 + _N // 2 + _N // 16),
    QUANT_KERNEL: (os.path.join(ROOT, "profiles", "quantize_1x16_bf16_8192x4096_counters.txt"),
                   "fos_quantize with a precomputed amax", _N * 2 + _N // 2 + _N // 16),
}
KERNEL_SOURCES = [os.path.join(ROOT, "nvfp4_adaptive_block_amd", "csrc", f)
                  for f in ("fos_kernels.hip", "fos_device.h", "fos_kernels.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


KERNEL_TRACE = os.path.join(ROOT, "profiles", "kernel_trace_bench_workloads.txt")


def read_profile_value(path, key):
    """A `key = value` figure from a committed profile summary, or None when the
    file is missing or was taken on other kernel code."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.split("#", 1)[0] if not line.lstrip().startswith("#") else line.lstrip("# ")
        if "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def read_counters(kernel):
    """HBM bytes per launch of `kernel` from its committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel code."""
    return read_profile_value(COUNTER_FILES[kernel][0], "hbm_bytes_per_launch")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rotating(t, n_bytes_per_set, extra_per_set=0):
    import torch
    per = n_bytes_per_set + extra_per_set
    n = max(2, -(-FOOTPRINT // per))
    return [t.clone() for _ in range(n)] if t is not None else [None] * n


def time_loop(fn, n_sets, steps, warmup):
    """Run fn(i) for warmup untimed and `steps` timed iterations on the current
    stream; returns (total_ms, per-launch ms list from events around fn)."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        evs[i][0].record()
        fn(i % n_sets)
        evs[i][1].record()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end), [a.elapsed_time(b) for a, b in evs]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    # 400 untimed steps (about 12 ms): after 20 the clocks are still rising
    # and the step measures about 1 us slower
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-oracle sample time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other workloads")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3: a few quantize launches and a known-size copy, no JSON")
    ap.add_argument("--write-profiles", metavar="DIR",
                    help="summarize rocprofv3 CSV output under DIR (kt/, fetch/, write/, sq/) into profiles/")
    args = ap.parse_args()
    if args.write_profiles:
        write_profiles(args.write_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the quantizer's step has no cross-GPU part, so it is measured on one GPU only",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_adaptive_block_amd as fos
    import synthdata
    from synthdata import raw_bits

    torch.cuda.set_device(0)
    M, K = 8192, 4096
    n = M * K
    knobs = dict(recipe="4over6", block="1x16", scale_gran="tensor", err_metric="mse", err_prec="exact", bound=448)
    log(f"[bench] generating bf16 {M}x{K} N(0,1) (seed 21)")
    x_host = synthdata.activation_family("normal", M, K, 21, "bf16")
    x0 = x_host.to("cuda")
    in_bytes = n * 2
    out_bytes = n // 2 + n // 16
    xs = rotating(x0, in_bytes, out_bytes)
    nset = len(xs)
    codes = [torch.empty(M, K // 2, dtype=torch.uint8, device="cuda") for _ in range(nset)]
    scales = [torch.empty(M, K // 16, dtype=torch.uint8, device="cuda") for _ in range(nset)]
    sdec = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(nset)]
    amax = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(nset)]
    log(f"[bench] {nset} rotating buffer sets ({nset * (in_bytes + out_bytes) / 2**30:.2f} GiB)")

    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(i):
        fos.fos_quantize_fused(xs[i], codes=codes[i], scales=scales[i], amax=amax[i], sdec=sdec[i], workspace=ws,
                               status=status, **knobs)

    if args.profile_pass:
        # a few launches of the step's kernel and of the separate amax and
        # quantize kernels, plus a plain copy of known size for calibrating
        # the HBM counters
        for i in range(8):
            step(i % nset)
        for i in range(8):
            fos.fos_amax(xs[i % nset], "tensor", out=amax[i % nset])
            fos.fos_quantize(xs[i % nset], amax[i % nset], codes=codes[i % nset], scales=scales[i % nset],
                             sdec=sdec[i % nset], **knobs)
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] profile pass done (copy kernel: {COPY_BYTES} bytes read and written per launch)")
        return

    # ---------------------------------------------------------------- main step
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    for i in range(args.warmup):
        step(i % nset)
    torch.cuda.synchronize()
    # the step is one kernel launch: two events on the launch stream bracket
    # the timed region, and the kernel's average launch time is the region's
    # time over the step count (per-step events would add their own packets)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step((args.warmup + i) % nset)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    k_avg_ms = ms_per_step
    barrier_ok = int(status.item()) == 0
    # the step's kernel reads x once (the amax and the quantize share that
    # read) and writes codes and scales: 2 + 0.5 + 1/16 B per element
    step_bytes = in_bytes + out_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    k_gbs = step_bytes / (k_avg_ms * 1e-3) / 1e9
    log(f"[bench] step {ms_per_step * 1e3:.1f} us ({value:.0f} GB/s); fused kernel {k_avg_ms * 1e3:.1f} us "
        f"({k_gbs:.0f} GB/s, {k_gbs / PEAK_HBM_GBS:.1%} of peak); barrier ok: {barrier_ok}")

    # bit-exact spot check of the last outputs against the CPU oracle
    bit_exact = None
    try:
        import oracle
        orc = oracle.get()
        last = (args.warmup + args.steps - 1) % nset
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(0).integers(0, M, 62)]))
        a_host = orc.amax(raw_bits(x_host), "bf16", "tensor")
        want = orc.quantize(raw_bits(x_host)[rows], "bf16", a_host, **knobs)
        got_c = codes[last].cpu().numpy()[rows]
        got_s = scales[last].cpu().numpy()[rows]
        got_a = amax[last].cpu().numpy()
        bit_exact = bool(np.array_equal(got_c, want["codes"]) and np.array_equal(got_s, want["scales"])
                         and got_a.view(np.uint32)[0] == a_host.view(np.uint32)[0])
        log(f"[bench] bit-exact vs oracle on {rows.size} sampled rows and the amax: {bit_exact}")
    except Exception as e:  # the oracle is optional for timing
        log(f"[bench] oracle spot check skipped: {e}")

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        xb = raw_bits(x_host)
        reps, t0 = 0, time.perf_counter()
        while True:
            a_h = orc.amax(xb, "bf16", "tensor")
            orc.quantize(xb, "bf16", a_h, **knobs)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el > 30:
                break
        cpu = {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
               "kind": "oracle",
               "sample": f"{reps} full steps (amax + quantize of the whole bf16 {M}x{K} tensor) in {el:.1f} s"}
        log(f"[bench] CPU oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    # ---------------------------------------------------------------- other workloads
    other = {}
    if not args.no_other:
        other = other_workloads(fos, synthdata, torch, np, c2=(xs, codes, scales, amax, sdec, knobs))

    traffic = read_counters(FUSED_KERNEL)
    rocprof_us = read_profile_value(KERNEL_TRACE, "fused_kernel_avg_us")
    # the VALU co-bound beside the HBM one: the kernel's VALU wave
    # instructions (SQ_INSTS_VALU of the committed counter pass) as lane
    # instructions per second against 256 CUs x 64 lanes x 2.4 GHz
    cf = COUNTER_FILES[FUSED_KERNEL][0]
    wave_insts = read_profile_value(cf, "sq_insts_valu")
    valu = None
    if wave_insts:
        lane_rate = wave_insts * 64 / (k_avg_ms * 1e-3)
        valu = {"lane_insts_per_launch": int(wave_insts * 64),
                "lane_insts_per_element": read_profile_value(cf, "valu_lane_insts_per_element"),
                "cvt_insts_per_block": read_profile_value(cf, "valu_cvt_insts_per_block"),
                "achieved": round(lane_rate / 1e12, 2), "peak": PEAK_VALU_LANE_TPS / 1e12,
                "unit": "T lane-instructions/s", "frac": round(lane_rate / PEAK_VALU_LANE_TPS, 4)}
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "dense activation quantize, bf16 8192x4096 N(0,1) seed 21, 1x16 blocks, "
                               "per-tensor amax + four-over-six MSE exact, E4M3 bound 448, in one launch "
                               "(fos_quantize_fused)",
                   "M": M, "K": K, "input_dtype": "bf16", "recipe": "4over6", "err_metric": "mse",
                   "err_prec": "exact", "e4m3_bound": 448, "rotating_sets": nset,
                   "step_bytes": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "fos_quantize_fused (k_fused_onchip, bf16, 4over6 MSE exact)",
                     "achieved": round(k_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": step_bytes, "avg_launch_us": round(k_avg_ms * 1e3, 2),
                     "rocprof_kernel_avg_us": rocprof_us},
        "valu": valu,
        "barrier_ok": barrier_ok,
        "bit_exact_sample": bit_exact,
        "cpu_baseline": cpu,
        "other_workloads": other,
    }
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------- profile summaries

PROFILE_CMDS = {
    "kt": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o kt -- "
          "python3 $REPO/bench.py --steps 200 --no-cpu-baseline",
    "fetch": "timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/fetch -o fetch -- "
             "python3 $REPO/bench.py --profile-pass",
    "write": "timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write -o write -- "
             "python3 $REPO/bench.py --profile-pass",
    "sq": "timeout -s KILL 90 rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES "
          "SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_INSTS_VALU_CVT GRBM_GUI_ACTIVE --output-format csv "
          "-d $OUT/sq -o sq -- python3 $REPO/bench.py --profile-pass",
}
_DT = {"0": "bf16", "1": "fp16", "2": "fp32"}
_RC = {"0": "nvfp4", "1": "4over6"}
_MT = {"0": "mae", "1": "mse"}
_PR = {"0": "exact", "1": "fp16err"}
_GR = {"0": "tensor", "1": "row", "2": "grouped"}
_OUT = {"0": "quantize", "1": "qdq"}


_ORD = {"0": "", "1": " seq"}


def describe_kernel(name: str) -> str:
    """Readable mode of one of this library's kernel template instances."""
    import re
    m = re.match(r"void fos::k_1x16<(\d+), (\d), (\d), (\d), (\d), (\d), (\d), (\d)>", name)
    if m:
        nt, dt, rc, mt, pr, od, gr, out = m.groups()
        lst = f" list<{nt}>" if nt != "1" else ""
        err = f" {_MT[mt]} {_PR[pr]}{_ORD[od]}" if rc == "1" else ""
        return f"1x16 {_OUT[out]}{lst} {_DT[dt]} {_RC[rc]}{err} {_GR[gr]}"
    m = re.match(r"void fos::k_16x16<(\d), (\d), (\d), (\d), (\d), (\d)>", name)
    if m:
        dt, rc, mt, pr, gr, out = m.groups()
        err = f" {_MT[mt]} {_PR[pr]}" if rc == "1" else ""
        return f"16x16 {_OUT[out]} {_DT[dt]} {_RC[rc]}{err} {_GR[gr]}"
    m = re.match(r"void fos::k_fused(_onchip)?<(\d), (\d), (\d), (\d), (\d)(?:, (\d))?>", name)
    if m:
        form, dt, rc, mt, pr, od, out = m.groups()
        err = f" {_MT[mt]} {_PR[pr]}{_ORD[od]}" if rc == "1" else ""
        form = " (one read)" if form else " (two reads)"
        return f"fused amax + 1x16 {_OUT[out or '0']}{form} {_DT[dt]} {_RC[rc]}{err} tensor"
    m = re.match(r"void fos::k_fused_row<(\d), (\d), (\d), (\d), (\d)>", name)
    if m:
        dt, rc, mt, pr, od = m.groups()
        err = f" {_MT[mt]} {_PR[pr]}{_ORD[od]}" if rc == "1" else ""
        return f"fused per-row amaxes + 1x16 quantize {_DT[dt]} {_RC[rc]}{err} row"
    m = re.match(r"void fos::k_fused_grouped<(\d), (\d), (\d), (\d), (\d)>", name)
    if m:
        dt, rc, mt, pr, od = m.groups()
        err = f" {_MT[mt]} {_PR[pr]}{_ORD[od]}" if rc == "1" else ""
        return f"fused group amaxes + grouped 1x16 quantize {_DT[dt]} {_RC[rc]}{err}"
    m = re.match(r"void fos::k_colwise<(\d), (\d), (\d), (\d), (\d)>", name)
    if m:
        dt, rc, mt, pr, od = m.groups()
        err = f" {_MT[mt]} {_PR[pr]}{_ORD[od]}" if rc == "1" else ""
        return f"columnwise 1x16 quantize {_DT[dt]} {_RC[rc]}{err} tensor"
    m = re.match(r"void fos::k_dequant<(\d), (\d)>", name)
    if m:
        dt, gr = m.groups()
        return f"dequantize to {_DT[dt]} {_GR[gr]}"
    if "k_amax_tensor" in name:
        return "amax per tensor (" + _DT.get(name.split("<")[1][0], "?") + ")"
    if "k_zero_u32" in name:
        return "clear the amax word"
    if "copyBuffer" in name:
        return "runtime copy (buffer set clones)"
    return ""


def _counters(path):
    """{(kernel, counter): [per-dispatch values in dispatch order]} from a rocprofv3 counter CSV."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], r["Counter_Name"])
        per.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), 0.0)
        per[key][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: [v[d] for d in sorted(v)] for k, v in per.items()}


def write_profiles(d):
    """Write profiles/kernel_trace_bench_workloads.txt and the counter
    summaries of the step's fused kernel and of the precomputed-amax quantize
    kernel from the CSV files rocprofv3 wrote under d."""
    import csv
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    ksha = kernel_source_hash()

    # kernel trace summary (rocprofv3 --stats)
    stats = list(csv.DictReader(open(os.path.join(d, "kt", "kt_kernel_stats.csv"))))
    lines = ["# rocprofv3 --kernel-trace --stats summary of the default bench (all workloads)",
             "# command (after: cd /tmp && export TMPDIR=/tmp; OUT = an output folder, REPO = this repository):",
             "#   " + PROFILE_CMDS["kt"],
             f"# kernel_source_sha256_16 = {ksha}",
             "# durations in microseconds, per dispatch",
             f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'share':>6}  mode / kernel"]
    avg = {}
    for r in stats:
        name = r["Name"]
        avg[name] = float(r["AverageNs"]) / 1e3
        desc = describe_kernel(name)
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):5.1f}%  "
                     f"{desc + ' | ' if desc else ''}{name[:110]}")
    if FUSED_KERNEL in avg:
        lines.append(f"fused_kernel_avg_us = {avg[FUSED_KERNEL]:.2f}   # the bench step's one kernel")
    if QUANT_KERNEL in avg:
        lines.append(f"quantize_kernel_avg_us = {avg[QUANT_KERNEL]:.2f}   # bf16 8192x4096 quantize, precomputed amax")
    open(os.path.join(out_dir, "kernel_trace_bench_workloads.txt"), "w").write("\n".join(lines) + "\n")

    # HBM counters, calibrated on a copy of known size
    f = _counters(os.path.join(d, "fetch", "fetch_counter_collection.csv"))
    w = _counters(os.path.join(d, "write", "write_counter_collection.csv"))
    sq_path = os.path.join(d, "sq", "sq_counter_collection.csv")
    s = _counters(sq_path) if os.path.exists(sq_path) else None
    copy_name = "__amd_rocclr_copyBuffer"
    cf = f[(copy_name, "FETCH_SIZE")][-4:]   # the profile pass ends with four copies of COPY_BYTES
    cw = w[(copy_name, "WRITE_SIZE")][-4:]
    mean = lambda v: sum(v) / len(v)
    fetch_factor = COPY_BYTES / (mean(cf) * 1024)
    write_factor = COPY_BYTES / (mean(cw) * 1024)
    n = _N
    for kernel, (path, what, alg) in COUNTER_FILES.items():
        qf = f[(kernel, "FETCH_SIZE")]
        qw = w[(kernel, "WRITE_SIZE")]
        rd = mean(qf) * 1024 * fetch_factor
        wr = mean(qw) * 1024 * write_factor
        lines = [f"# rocprofv3 counter summary: {what}; 1x16 blocks, bf16 8192x4096 N(0,1), four-over-six",
                 "# MSE exact, E4M3 bound 448, per-tensor scale",
                 "# commands (after: cd /tmp && export TMPDIR=/tmp; OUT = an output folder, REPO = this repository):",
                 "#   " + PROFILE_CMDS["fetch"], "#   " + PROFILE_CMDS["write"], "#   " + PROFILE_CMDS["sq"],
                 "#   python3 $REPO/bench.py --write-profiles $OUT",
                 "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch. The factors scale them to bytes so that the",
                 f"# profile pass's plain copy of {COPY_BYTES} bytes reads and writes exactly that many bytes.",
                 f"kernel = {kernel}",
                 f"kernel_source_sha256_16 = {ksha}",
                 f"dispatches = {len(qf)}",
                 f"fetch_size_kib = {mean(qf):.1f}",
                 f"write_size_kib = {mean(qw):.1f}",
                 f"copy_fetch_size_kib = {mean(cf):.1f}",
                 f"copy_write_size_kib = {mean(cw):.1f}",
                 f"fetch_factor = {fetch_factor:.4f}",
                 f"write_factor = {write_factor:.4f}",
                 f"hbm_read_bytes_per_launch = {rd:.0f}",
                 f"hbm_write_bytes_per_launch = {wr:.0f}",
                 f"hbm_bytes_per_launch = {rd + wr:.0f}",
                 f"algorithmic_bytes_per_launch = {alg}",
                 f"traffic_over_algorithmic = {(rd + wr) / alg:.4f}"]
        if s is not None and (kernel, "SQ_INSTS_VALU") in s:
            get = lambda c: mean(s[(kernel, c)])
            valu = get("SQ_INSTS_VALU")
            lines += [f"sq_waves = {get('SQ_WAVES'):.0f}",
                      f"sq_insts_valu = {valu:.0f}   # wave instructions per dispatch",
                      f"sq_insts_valu_cvt = {get('SQ_INSTS_VALU_CVT'):.0f}",
                      f"sq_active_inst_valu = {get('SQ_ACTIVE_INST_VALU'):.0f}",
                      f"sq_wave_cycles = {get('SQ_WAVE_CYCLES'):.0f}",
                      f"sq_busy_cycles = {get('SQ_BUSY_CYCLES'):.0f}",
                      f"sq_wait_inst_any = {get('SQ_WAIT_INST_ANY'):.0f}",
                      f"grbm_gui_active = {get('GRBM_GUI_ACTIVE'):.0f}",
                      f"valu_lane_insts_per_element = {valu * 64 / n:.2f}",
                      f"valu_cvt_insts_per_block = {get('SQ_INSTS_VALU_CVT') * 64 / (n // 16):.2f}"]
        open(path, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))


def other_workloads(fos, synthdata, torch, np, c2, steps=50, warmup=5):
    """Brief kernel-only timings of the other configurations (precomputed
    amax); each figure is the median launch of its loop."""
    out = {}

    def gbs(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    # the achievable ceiling in the same run: a plain 256 MiB device-to-device
    # copy (reads and writes 256 MiB each), four buffer pairs in rotation
    srcs = [torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda") for _ in range(4)]
    dsts = [torch.empty_like(t) for t in srcs]
    _, ms = time_loop(lambda i: dsts[i].copy_(srcs[i]), len(srcs), 50, 5)
    avg = float(np.median(ms))
    out["copy_256MiB_device_to_device"] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(2 * COPY_BYTES, avg),
                                           "frac": round(gbs(2 * COPY_BYTES, avg) / PEAK_HBM_GBS, 4)}
    log(f"[bench] device copy 256 MiB: {avg * 1e3:.1f} us, {gbs(2 * COPY_BYTES, avg):.0f} GB/s (the ceiling)")
    del srcs, dsts

    # the dense activation tensor: the quantize kernel alone with a
    # precomputed amax (the pages' kernel metric), and the two-launch step
    xs, codes, scales, amax, sdec, knobs = c2
    n = xs[0].numel()
    qb = n * 2 + n // 2 + n // 16
    for i in range(len(xs)):
        fos.fos_amax(xs[i], "tensor", out=amax[i])
    _, ms = time_loop(lambda i: fos.fos_quantize(xs[i], amax[i], codes=codes[i], scales=scales[i], sdec=sdec[i],
                                                 **knobs), len(xs), 200, 10)
    avg = float(np.median(ms))
    out["quantize_1x16_bf16_8192x4096_precomputed_amax"] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(qb, avg),
                                                            "frac": round(gbs(qb, avg) / PEAK_HBM_GBS, 4)}
    log(f"[bench] quantize bf16 8192x4096, precomputed amax: {avg * 1e3:.1f} us, {gbs(qb, avg):.0f} GB/s")

    # the same tensor with per-row global scales (one amax per row)
    row_amax = [fos.fos_amax(xs[i], "row") for i in range(len(xs))]
    rknobs = dict(knobs, scale_gran="row")
    rsdec = torch.empty(xs[0].shape[0], dtype=torch.float32, device="cuda")
    _, ms = time_loop(lambda i: fos.fos_quantize(xs[i], row_amax[i], codes=codes[i], scales=scales[i], sdec=rsdec,
                                                 **rknobs), len(xs), 200, 10)
    avg = float(np.median(ms))
    out["quantize_1x16_bf16_8192x4096_per_row_amax"] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(qb, avg),
                                                        "frac": round(gbs(qb, avg) / PEAK_HBM_GBS, 4)}
    log(f"[bench] quantize bf16 8192x4096, per-row amax: {avg * 1e3:.1f} us, {gbs(qb, avg):.0f} GB/s")
    # per-row amaxes computed on the device: one launch (each row read from
    # HBM once), against fos_amax per row followed by fos_quantize
    ra = torch.empty(xs[0].shape[0], dtype=torch.float32, device="cuda")
    for key, fn in (("fused_row_amax_quantize_bf16_8192x4096",
                     lambda i: fos.fos_quantize_fused(xs[i], codes=codes[i], scales=scales[i], amax=ra, sdec=rsdec,
                                                      **rknobs)),
                    ("row_amax_then_quantize_bf16_8192x4096",
                     lambda i: (fos.fos_amax(xs[i], "row", out=ra),
                                fos.fos_quantize(xs[i], ra, codes=codes[i], scales=scales[i], sdec=rsdec, **rknobs)))):
        _, ms = time_loop(fn, len(xs), 200, 10)
        avg = float(np.median(ms))
        out[key] = {"avg_step_us": round(avg * 1e3, 2), "GB/s": gbs(qb, avg), "frac": round(gbs(qb, avg) / PEAK_HBM_GBS, 4)}
        log(f"[bench] {key}: {avg * 1e3:.1f} us, {gbs(qb, avg):.0f} GB/s (x read once + codes and scales)")
    del row_amax, ra

    # fused fake quantization of the same tensor with its amax computed on
    # the device: one launch that reads x once, against fos_amax + fos_qdq
    ys2 = [torch.empty_like(x) for x in xs]
    qkw = dict(recipe="4over6", err_metric="mse", err_prec="fp16", bound=448)
    qws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    qb2 = n * 2 + n * 2
    for key, fn in (("qdq_fused_amax_bf16_8192x4096_4over6_mse_fp16_448",
                     lambda i: fos.fos_qdq_fused(xs[i], out=ys2[i], amax=amax[i], workspace=qws, **qkw)),
                    ("amax_then_qdq_bf16_8192x4096_4over6_mse_fp16_448",
                     lambda i: (fos.fos_amax(xs[i], "tensor", out=amax[i]),
                                fos.fos_qdq(xs[i], amax[i], out=ys2[i], **qkw)))):
        _, ms = time_loop(fn, len(xs), 200, 10)
        avg = float(np.median(ms))
        out[key] = {"avg_step_us": round(avg * 1e3, 2), "GB/s": gbs(qb2, avg), "frac": round(gbs(qb2, avg) / PEAK_HBM_GBS, 4)}
        log(f"[bench] {key}: {avg * 1e3:.1f} us, {gbs(qb2, avg):.0f} GB/s (x read once, y written)")
    del ys2

    def two_launches(i):
        fos.fos_amax(xs[i], "tensor", out=amax[i])
        fos.fos_quantize(xs[i], amax[i], codes=codes[i], scales=scales[i], sdec=sdec[i], **knobs)
    _, ms = time_loop(two_launches, len(xs), 200, 10)
    avg = float(np.median(ms))
    out["amax_then_quantize_bf16_8192x4096"] = {"avg_step_us": round(avg * 1e3, 2), "GB/s": gbs(qb + 2 * n, avg)}
    log(f"[bench] fos_amax + fos_quantize (two launches): {avg * 1e3:.1f} us")

    # columnwise quantize (the transpose's codes and scales) of the same tensor
    ct = torch.empty(xs[0].shape[1], xs[0].shape[0] // 2, dtype=torch.uint8, device="cuda")
    st = torch.empty(xs[0].shape[1], xs[0].shape[0] // 16, dtype=torch.uint8, device="cuda")
    _, ms = time_loop(lambda i: fos.fos_quantize_columnwise(xs[i], amax[i], codes=ct, scales=st, sdec=sdec[i],
                                                            **knobs), len(xs), 200, 10)
    avg = float(np.median(ms))
    out["quantize_columnwise_bf16_8192x4096"] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(qb, avg),
                                                 "frac": round(gbs(qb, avg) / PEAK_HBM_GBS, 4)}
    log(f"[bench] columnwise bf16 8192x4096: {avg * 1e3:.1f} us, {gbs(qb, avg):.0f} GB/s")
    del ct, st

    # nvfp4_dequantize of the step's outputs back to bf16 (the dequantized-
    # backward recompute): reads 0.5625 B/elem, writes 2 B/elem
    ys = [torch.empty_like(x) for x in xs]
    _, ms = time_loop(lambda i: fos.nvfp4_dequantize(codes[i], scales[i], sdec[i], "tensor", torch.bfloat16,
                                                     out=ys[i]), len(xs), 200, 10)
    avg = float(np.median(ms))
    out["dequantize_bf16_8192x4096"] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(qb, avg),
                                        "frac": round(gbs(qb, avg) / PEAK_HBM_GBS, 4)}
    log(f"[bench] dequantize bf16 8192x4096: {avg * 1e3:.1f} us, {gbs(qb, avg):.0f} GB/s")
    del ys

    # 16x16 weights, bf16 4096x14336 and fp32 4096x4096, per-tensor, MSE exact, 448
    for dtype, (M, K) in (("bf16", (4096, 14336)), ("fp32", (4096, 4096))):
        w = synthdata.weight(M, K, 31, dtype).to("cuda")
        a = fos.fos_amax(w, "tensor")
        eb = 2 if dtype == "bf16" else 4
        nbytes = M * K * eb + M * K // 2 + M * K // 16
        ws = rotating(w, nbytes)
        c = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
        s = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
        sd = torch.empty(1, dtype=torch.float32, device="cuda")
        _, ms = time_loop(lambda i: fos.fos_quantize(ws[i], a, codes=c, scales=s, sdec=sd, recipe="4over6",
                                                     block="16x16", err_metric="mse", err_prec="exact"),
                          len(ws), steps, warmup)
        avg = float(np.median(ms))
        out[f"quantize_16x16_{dtype}_{M}x{K}"] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(nbytes, avg),
                                                  "frac": round(gbs(nbytes, avg) / PEAK_HBM_GBS, 4)}
        log(f"[bench] 16x16 {dtype} {M}x{K}: {avg * 1e3:.1f} us, {gbs(nbytes, avg):.0f} GB/s")
        del ws, w

    # fused QDQ over 8 expert weights 2048x7168, bf16 and fp16, the five timed modes
    lst = synthdata.expert_weight_list(8, 2048, 7168, 40, dtypes=("bf16", "fp16"))
    for dtype in ("bf16", "fp16"):
        xs = [t.to("cuda") for t in lst[dtype]]
        ams = [fos.fos_amax(t, "tensor") for t in xs]
        ys = [torch.empty_like(t) for t in xs]
        nbytes = sum(t.numel() for t in xs) * 4
        for mode in (("nvfp4", "mse", "fp16", 448), ("4over6", "mae", "fp16", 448), ("4over6", "mae", "fp16", 256),
                     ("4over6", "mse", "fp16", 448), ("4over6", "mse", "fp16", 256)):
            r, m, p, bnd = mode
            _, ms = time_loop(lambda i: fos.fos_qdq_list(xs, ams, outs=ys, recipe=r, err_metric=m, err_prec=p,
                                                         bound=bnd), 1, steps, warmup)
            avg = float(np.median(ms))
            key = f"qdq_list_8x2048x7168_{dtype}_{r}" + ("" if r == "nvfp4" else f"_{m}_{p}_{bnd}")
            out[key] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(nbytes, avg),
                        "frac": round(gbs(nbytes, avg) / PEAK_HBM_GBS, 4)}
            log(f"[bench] {key}: {avg * 1e3:.1f} us, {gbs(nbytes, avg):.0f} GB/s")
        del xs, ys
    del lst

    # grouped MoE activations: 65536 (+4096 padding) x 7168, 64 groups, MSE exact
    M, pad, K, G = 65536, 4096, 7168, 64
    x, offs, fac = synthdata.grouped_tokens(M, pad, K, G)
    x = x.to("cuda")
    offs_d = torch.from_numpy(offs).to("cuda")
    starts = np.concatenate([[0], offs[:-1]])
    gam = torch.stack([fos.fos_amax(x[s:e].contiguous(), "tensor")[0] if e > s else
                       torch.zeros((), device="cuda") for s, e in zip(starts, offs)])
    c = torch.empty(M + pad, K // 2, dtype=torch.uint8, device="cuda")
    s = torch.empty(M + pad, K // 16, dtype=torch.uint8, device="cuda")
    nbytes = M * K * 2 + (M + pad) * (K // 2 + K // 16)
    for bnd in (448, 256):
        _, ms = time_loop(lambda i: fos.fos_quantize_grouped(x, offs_d, gam, codes=c, scales=s, recipe="4over6",
                                                             err_metric="mse", err_prec="exact", bound=bnd),
                          1, steps, warmup)
        avg = float(np.median(ms))
        key = f"quantize_grouped_{M}+{pad}x{K}_G{G}_{bnd}"
        out[key] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(nbytes, avg),
                    "frac": round(gbs(nbytes, avg) / PEAK_HBM_GBS, 4)}
        log(f"[bench] {key}: {avg * 1e3:.1f} us, {gbs(nbytes, avg):.0f} GB/s")
    # the group amaxes and the grouped quantize in one launch: x's data rows
    # are read twice (amax phase, quantize phase)
    ga = torch.empty(G, dtype=torch.float32, device="cuda")
    gs = torch.empty(G, dtype=torch.float32, device="cuda")
    fbytes = nbytes + M * K * 2
    _, ms = time_loop(lambda i: fos.fos_quantize_grouped_fused(x, offs_d, codes=c, scales=s, group_amax=ga,
                                                               group_sdec=gs, recipe="4over6", err_metric="mse",
                                                               err_prec="exact", bound=448), 1, steps, warmup)
    avg = float(np.median(ms))
    key = f"fused_amax_quantize_grouped_{M}+{pad}x{K}_G{G}_448"
    out[key] = {"avg_launch_us": round(avg * 1e3, 2), "GB/s": gbs(fbytes, avg),
                "frac": round(gbs(fbytes, avg) / PEAK_HBM_GBS, 4)}
    log(f"[bench] {key}: {avg * 1e3:.1f} us, {gbs(fbytes, avg):.0f} GB/s")
    return out


if __name__ == "__main__":
    main()
