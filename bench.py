#!/usr/bin/env python3
"""Benchmark of the four-over-six NVFP4 quantizer on one MI355X.

One step is one pass of the hot path over the largest configuration, the
grouped MoE activation quantize (pytorch/ao PR "Add the four-over-six grouped
GEMM and dispatcher wiring", MoE commit): a packed bf16 token tensor of 65536
rows plus 4096 over-allocated padding rows by 7168, split into 64 expert
groups of Dirichlet(0.5) sizes rounded to 16 rows, each group N(0,1) times a
factor 10^U(-2, 2). Each group's amax is expanded to per-row global scales
and the whole tensor quantizes in one fos_quantize_grouped launch: 1x16
blocks, four-over-six with MSE exact error, E4M3 bound 448, codes and scales
written for all 69632 rows (the padding rows' as zero, never read). The
group amaxes are the launch's input, computed on the device beforehand and
not timed (the pages' precomputed-amax kernel metric); the one-launch form
that computes them too is timed under `other_workloads`.

`value` is the step's algorithmic HBM traffic (the data rows read once, 2 B
per element; codes and scales of every row written, 0.5625 B per element)
over the measured step time; the data rows alone exceed the 256 MB Infinity
Cache four times over, so every step reads from HBM. `roofline` covers the
step's kernel, timed with HIP events on the stream it runs on, beside a
hand-written streaming kernel of the same read:write mix (bench_stream.hip).
`cpu_baseline` times the CPU oracle on the same tensor and checks the GPU's
output against it in full. The other configurations (the dense activation
tensor, the 16x16 weights, the fused-QDQ expert list, the streaming
ceilings) are timed briefly under `other_workloads`, each in algorithmic
bytes (every input read once, every output written once).

Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD public spec
N_SIMD = 256 * 4               # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9               # peak engine clock
MALL_BYTES = 256 << 20
FOOTPRINT = 1 << 30            # rotate buffers up to >= 1 GiB
METRIC = "4over6 quantize/QDQ achieved HBM GB/s and % of MI355X peak (bit-exact)"
DEFAULT_STEPS = 200             # timed steps of the default run (after the untimed warmup)
COPY_BYTES = 256 << 20         # the profile pass's calibration copy

# the grouped MoE workload
M5, PAD5, K5, G5 = 65536, 4096, 7168, 64
STEP_BYTES = M5 * K5 * 2 + (M5 + PAD5) * (K5 // 2 + K5 // 16)
KNOBS = dict(recipe="4over6", err_metric="mse", err_prec="exact", bound=448)

HEADLINE_KERNEL = "void fos::k_1x16<1, 0, 1, 1, 0, 0, 2, 0>(fos::Args1x16<1>)"
_N2 = 8192 * 4096
# kernels with a counter summary: (file stem, readable workload, algorithmic bytes per launch)
COUNTER_KERNELS = {
    HEADLINE_KERNEL: ("quantize_grouped_bf16_65536x7168",
                      "fos_quantize_grouped, bf16 65536 (+4096 padding) x 7168, 64 groups, four-over-six MSE exact, "
                      "bound 448", STEP_BYTES),
    "void fos::k_16x16<0, 1, 1, 0, 0, 0>(fos::Args16x16)":
        ("quantize_16x16_bf16_4096x14336",
         "fos_quantize 16x16 tiles, bf16 4096x14336 0.02*N(0,1), per-tensor, four-over-six MSE exact, bound 448",
         4096 * 14336 * 2 + 4096 * 14336 // 2 + 4096 * 14336 // 16),
    "void fos::k_1x16<48, 0, 1, 1, 1, 0, 0, 1>(fos::Args1x16<48>)":
        ("qdq_list_bf16_8x2048x7168",
         "fos_qdq_list, 8 x bf16 2048x7168 expert weights, four-over-six MSE FP16-error, bound 448",
         8 * 2048 * 7168 * 4),
    "void fos::k_fused_onchip<0, 1, 1, 0, 0, 0>(fos::Args1x16<1>, unsigned int*, float*)":
        ("fused_amax_quantize_bf16_8192x4096",
         "fos_quantize_fused (amax and quantize in one launch, x read once), bf16 8192x4096 N(0,1), four-over-six "
         "MSE exact, bound 448", _N2 * 2 + _N2 // 2 + _N2 // 16),
    "void fos::k_1x16<1, 0, 1, 1, 0, 0, 0, 0>(fos::Args1x16<1>)":
        ("quantize_1x16_bf16_8192x4096",
         "fos_quantize with a precomputed amax, bf16 8192x4096 N(0,1), four-over-six MSE exact, bound 448",
         _N2 * 2 + _N2 // 2 + _N2 // 16),
}
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE_TRACE = os.path.join(PROFILES, "kernel_trace_quantize_grouped_bf16_65536x7168.txt")
STREAM_LIB = os.path.join(ROOT, "libbench_stream.so")


def kernel_source_hash() -> str:
    from nvfp4_adaptive_block_amd.build import kernel_source_hash as h
    return h()


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


def counter_file(kernel):
    return os.path.join(PROFILES, f"counters_{COUNTER_KERNELS[kernel][0]}.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rotating(t, bytes_per_set):
    n = max(2, -(-FOOTPRINT // bytes_per_set))
    return [t.clone() for _ in range(n)]


def time_loop(fn, n_sets, steps, warmup, reps=3):
    """Per-launch device time of fn: `warmup` untimed calls, then `steps`
    calls (buffer set i % n_sets) captured into one HIP graph, replayed
    `reps` times between two events; returns each replay's time over
    `steps`, in ms. The graph runs the launches back to back, so host-side
    call overhead (argument marshalling, a few to tens of microseconds per
    call) does not enter the time of short kernels."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i % n_sets)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / steps)
    del g
    return out


def gbs(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


def entry(nbytes, ms, **extra):
    g = gbs(nbytes, ms)
    return {"avg_launch_us": round(ms * 1e3, 2), "GB/s": g, "frac": round(g / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": int(nbytes), **extra}


# ---------------------------------------------------------------- workloads

def grouped_inputs(torch, fos, synthdata):
    """The grouped MoE tensor on the device, its offsets and its group amaxes
    (computed on the device: input preparation, not part of the step)."""
    import numpy as np
    x, offs, _ = synthdata.grouped_tokens(M5, PAD5, K5, G5)
    xd = x.to("cuda")
    od = torch.from_numpy(offs).to("cuda")
    starts = np.concatenate([[0], offs[:-1]])
    gam = torch.zeros(G5, dtype=torch.float32, device="cuda")
    for g, (s, e) in enumerate(zip(starts, offs)):
        if e > s:
            fos.fos_amax(xd[s:e], "tensor", out=gam[g:g + 1])
    return x, offs, xd, od, gam


class Stream:
    """The hand-written streaming kernels of bench_stream.hip."""

    MIXES = {"read_only": 0, "write_only": 1, "quantize_mix": 2, "qdq_mix": 3}

    def __init__(self):
        if not os.path.exists(STREAM_LIB):
            raise FileNotFoundError(f"{STREAM_LIB} is not built (run __graft_entry__.build())")
        self.lib = ctypes.CDLL(STREAM_LIB)
        self.lib.stream_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        self.lib.stream_bytes_per_unit.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                                   ctypes.POINTER(ctypes.c_int64)]

    def measure(self, torch, np, mix, units, steps=60, warmup=10):
        """Best median GB/s over the two store policies and the two unit
        orders (contiguous ranges per wave, or pairs dealt round robin), and
        each."""
        r, w = ctypes.c_int64(), ctypes.c_int64()
        self.lib.stream_bytes_per_unit(self.MIXES[mix], ctypes.byref(r), ctypes.byref(w))
        src = torch.empty(max(1, units * r.value), dtype=torch.uint8, device="cuda")
        dst = torch.empty(max(1, units * w.value), dtype=torch.uint8, device="cuda")
        src.random_(0, 255) if r.value else None
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        nbytes = units * (r.value + w.value)
        out = {}
        for il in (0, 1):
            for nt in (0, 1):
                def run(_i, nt=nt, il=il):
                    rc = self.lib.stream_run(self.MIXES[mix], nt, il, ctypes.c_void_p(src.data_ptr()),
                                             ctypes.c_void_p(dst.data_ptr()), units, ctypes.c_void_p(sink.data_ptr()),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                    assert rc == 0
                ms = float(np.median(time_loop(run, 1, steps, warmup)))
                out[("nt" if nt else "default") + ("_interleaved" if il else "")] = entry(nbytes, ms)
        best = max(out.values(), key=lambda e: e["GB/s"])
        return {"GB/s": best["GB/s"], "frac": best["frac"], "read_bytes": units * r.value,
                "write_bytes": units * w.value, "variants": out}


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    # untimed steps first: the clocks take about 12 ms to settle
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-oracle sample time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other workloads")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3: each counter-summary workload, then a known-size copy; no JSON")
    ap.add_argument("--write-profiles", metavar="DIR",
                    help="summarize rocprofv3 CSV output under DIR (kt/, kt_pass/, fetch/, write/, sq/, occ/)")
    ap.add_argument("--profiles-out", metavar="DIR", default=PROFILES,
                    help="where --write-profiles writes its summaries (default: profiles/)")
    args = ap.parse_args()
    if args.write_profiles:
        write_profiles(args.write_profiles, args.profiles_out)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "every GPU box here has one GPU, and the quantizer's step has no cross-GPU part",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_adaptive_block_amd as fos
    import synthdata
    from synthdata import raw_bits

    torch.cuda.set_device(0)
    if args.profile_pass:
        profile_pass(fos, synthdata, torch, np)
        return

    log(f"[bench] generating the grouped MoE tensor bf16 {M5}+{PAD5}x{K5}, {G5} groups (seeds 51-54)")
    x_host, offs, xd, od, gam = grouped_inputs(torch, fos, synthdata)
    codes = torch.empty(M5 + PAD5, K5 // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M5 + PAD5, K5 // 16, dtype=torch.uint8, device="cuda")
    gsdec = torch.empty(G5, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step(_i=0):
        fos.fos_quantize_grouped(xd, od, gam, codes=codes, scales=scales, group_sdec=gsdec, status=status, **KNOBS)

    # ---------------------------------------------------------------- the step
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the step is one kernel launch: two events on the launch stream bracket
    # the timed region, and the kernel's average launch time is the region's
    # time over the step count (per-step events would add their own packets)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    value = STEP_BYTES / (ms_per_step * 1e-3) / 1e9
    ok_status = int(status.item()) == 0
    log(f"[bench] step {ms_per_step * 1e3:.1f} us: {value:.0f} GB/s, {value / PEAK_HBM_GBS:.1%} of 8 TB/s; "
        f"status clean: {ok_status}")

    # ---------------------------------------------------------------- CPU oracle
    cpu, bit_exact = None, None
    if not args.no_cpu_baseline:
        cpu, bit_exact = cpu_leg(args, x_host, offs, gam, codes, scales, raw_bits, np)

    # ---------------------------------------------------------------- ceilings and other workloads
    stream = Stream()
    ceiling = stream.measure(torch, np, "quantize_mix", M5 * K5 * 2 // 4096)  # the step's read bytes
    log(f"[bench] streaming ceiling at the quantize mix (2 : 0.5625): {ceiling['GB/s']:.0f} GB/s")
    other = {}
    if not args.no_other:
        other = other_workloads(fos, synthdata, torch, np, stream, (xd, od, gam, codes, scales))

    traffic = read_profile_value(counter_file(HEADLINE_KERNEL), "hbm_bytes_per_launch")
    rocprof_us = read_profile_value(HEADLINE_TRACE, "headline_kernel_timed_avg_us")
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
        "config": {"workload": f"grouped MoE activation quantize: bf16 {M5} (+{PAD5} padding) x {K5} tokens in "
                               f"{G5} groups (Dirichlet(0.5) sizes in multiples of 16 rows, group factors "
                               "10^U(-2,2), seeds 51-54), per-group amax expanded per row, 1x16 blocks, "
                               "four-over-six MSE exact, E4M3 bound 448, one fos_quantize_grouped launch",
                   "M": M5, "pad_rows": PAD5, "K": K5, "groups": G5, "input_dtype": "bf16", "recipe": "4over6",
                   "err_metric": "mse", "err_prec": "exact", "e4m3_bound": 448, "step_bytes": STEP_BYTES},
        "roofline": roofline(ms_per_step, traffic, rocprof_us, ceiling),
        "status_clean": ok_status,
        "bit_exact": bit_exact,
        "cpu_baseline": cpu,
        "other_workloads": other,
        "context": context(value, cpu),
    }
    print(json.dumps(result), flush=True)


def context(value, cpu):
    """The pages' own figures, quoted beside ours (other hardware, other
    workloads: context, not a target), and the GPU-over-oracle ratio."""
    return {
        "pages": [
            "wolfcomos/ao PR 'Add a CuTe DSL fast-path kernel for four-over-six quantize' (description): "
            "26-30x over the pure-PyTorch reference body on GB200, training shapes not listed",
            "radixark/Megatron-LM PR 'Fuse NVFP4 fake-QAT quantize-dequantize with CuTe DSL' (Performance): "
            "8 x [4096, 6144] QDQ with precomputed amax on B300, 156.8 us standard NVFP4 and 213-216 us "
            "four-over-six FP16-error (about 5.1 and 3.7-3.8 TB/s at 4 B per element)",
        ],
        "gpu_over_oracle": round(value / cpu["value"], 1) if cpu and cpu.get("value") else None,
    }


def roofline(ms, traffic, rocprof_us, ceiling):
    achieved = STEP_BYTES / (ms * 1e-3) / 1e9
    cf = counter_file(HEADLINE_KERNEL)
    valu = None
    insts = read_profile_value(cf, "sq_insts_valu")
    if insts:
        # the VALU co-bound from the kernel's own counters: VALUBusy is the
        # fraction of each SIMD's cycles with a VALU instruction in flight;
        # SQ_ACTIVE_INST_VALU (quad-cycles) over SQ_INSTS_VALU gives the
        # measured issue cycles per wave instruction (converts included)
        valu = {"valu_busy": read_profile_value(cf, "valu_busy"),
                "valu_cycles_per_simd": read_profile_value(cf, "valu_cycles_per_simd"),
                "cycles_per_valu_inst": read_profile_value(cf, "cycles_per_valu_inst"),
                "valu_time_at_peak_clock_us": read_profile_value(cf, "valu_time_at_peak_clock_us"),
                "wave_insts_per_launch": int(insts),
                "cvt_wave_insts_per_launch": read_profile_value(cf, "sq_insts_valu_cvt"),
                "lane_insts_per_block": read_profile_value(cf, "valu_lane_insts_per_block"),
                "occupancy_waves_per_simd": read_profile_value(cf, "occupancy_waves_per_simd")}
    return {"bound": "hbm", "kernel": "fos_quantize_grouped (k_1x16 grouped, bf16, 4over6 MSE exact)",
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": STEP_BYTES, "avg_launch_us": round(ms * 1e3, 2),
            "rocprof_kernel_avg_us": rocprof_us,
            "ceiling_same_mix_GBs": ceiling["GB/s"], "frac_of_ceiling": round(achieved / ceiling["GB/s"], 4),
            "valu": valu}


def cpu_leg(args, x_host, offs, gam_dev, codes, scales, raw_bits, np):
    """The oracle on the same tensor: its group amaxes, then its grouped
    quantize, timed; the GPU's group amaxes, codes and scales are compared
    with the oracle's in full."""
    import oracle
    orc = oracle.get()
    bits = raw_bits(x_host)
    starts = np.concatenate([[0], offs[:-1]])
    log("[bench] CPU oracle: group amaxes")
    gam = np.array([orc.amax(bits[s:e], "bf16", "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                   np.float32)
    reps, t0, want = 0, time.perf_counter(), None
    while True:
        want = orc.quantize_grouped(bits, "bf16", offs, gam, **KNOBS)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or el > 30:
            break
    cpu = {"value": round(STEP_BYTES * reps / el / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
           "kind": "oracle",
           "sample": f"{reps} full steps (the grouped quantize of the whole bf16 {M5}+{PAD5}x{K5} tensor, group "
                     f"amaxes given) in {el:.1f} s"}
    log(f"[bench] CPU oracle: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['sample']})")
    same = (np.array_equal(gam_dev.cpu().numpy().view(np.uint32), gam.view(np.uint32))
            and np.array_equal(codes.cpu().numpy(), want["codes"]) and np.array_equal(scales.cpu().numpy(),
                                                                                     want["scales"]))
    log(f"[bench] bit-exact vs the oracle (group amaxes, all codes and scales): {same}")
    return cpu, bool(same)


def other_workloads(fos, synthdata, torch, np, stream, c5, steps=50, warmup=5):
    """Brief kernel-only timings of the other configurations; each figure is
    the median over graph replays of the mean launch time (time_loop), over
    the algorithmic bytes: every input read once and every output written
    once."""
    out = {}
    xd, od, gam, c, s = c5

    # ceilings: the hand-written streams (>= 1 GiB footprints) and torch's copy
    for mix in ("read_only", "write_only", "qdq_mix"):
        out[f"stream_{mix}"] = stream.measure(torch, np, mix, 262144)
        log(f"[bench] stream {mix}: {out[f'stream_{mix}']['GB/s']:.0f} GB/s")
    srcs = [torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda") for _ in range(4)]
    dsts = [torch.empty_like(t) for t in srcs]
    ms = float(np.median(time_loop(lambda i: dsts[i].copy_(srcs[i]), 4, 50, 5)))
    out["torch_copy_256MiB"] = entry(2 * COPY_BYTES, ms)
    del srcs, dsts

    # the grouped MoE tensor: bound 256, and the group amaxes in the same launch
    ms = float(np.median(time_loop(lambda i: fos.fos_quantize_grouped(xd, od, gam, codes=c, scales=s, recipe="4over6",
                                                                      err_metric="mse", bound=256), 1, steps, warmup)))
    out[f"quantize_grouped_{M5}+{PAD5}x{K5}_G{G5}_256"] = entry(STEP_BYTES, ms)
    ga = torch.empty(G5, dtype=torch.float32, device="cuda")
    gws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    gst = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = float(np.median(time_loop(lambda i: fos.fos_quantize_grouped_fused(xd, od, codes=c, scales=s, group_amax=ga,
                                                                            workspace=gws, status=gst, **KNOBS),
                                   1, steps, warmup)))
    out[f"fused_group_amax_quantize_grouped_{M5}+{PAD5}x{K5}_G{G5}_448"] = entry(
        STEP_BYTES, ms, note="one launch; its amax phase reads the data rows a second time")
    log(f"[bench] grouped: {out}")

    # the dense activation tensor, bf16 8192x4096 N(0,1), rotated over >= 1 GiB
    M, K = 8192, 4096
    n = M * K
    x0 = synthdata.activation_family("normal", M, K, 21, "bf16").to("cuda")
    qb = n * 2 + n // 2 + n // 16
    xs = rotating(x0, qb)
    ns = len(xs)
    codes = [torch.empty(M, K // 2, dtype=torch.uint8, device="cuda") for _ in range(ns)]
    scales = [torch.empty(M, K // 16, dtype=torch.uint8, device="cuda") for _ in range(ns)]
    amax = [fos.fos_amax(x, "tensor") for x in xs]
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    knobs = dict(KNOBS)
    runs = {
        "fused_amax_quantize_bf16_8192x4096": (
            lambda i: fos.fos_quantize_fused(xs[i], codes=codes[i], scales=scales[i], amax=amax[i], workspace=ws,
                                             status=st, **knobs), qb, "one launch, x read once"),
        "quantize_1x16_bf16_8192x4096_precomputed_amax": (
            lambda i: fos.fos_quantize(xs[i], amax[i], codes=codes[i], scales=scales[i], **knobs), qb, None),
        "amax_then_quantize_bf16_8192x4096": (
            lambda i: (fos.fos_amax(xs[i], "tensor", out=amax[i]),
                       fos.fos_quantize(xs[i], amax[i], codes=codes[i], scales=scales[i], **knobs)), qb,
            "two launches; x read twice"),
    }
    row_amax = [fos.fos_amax(x, "row") for x in xs]
    ra = torch.empty(M, dtype=torch.float32, device="cuda")
    rk = dict(knobs, scale_gran="row")
    runs["quantize_1x16_bf16_8192x4096_per_row_amax"] = (
        lambda i: fos.fos_quantize(xs[i], row_amax[i], codes=codes[i], scales=scales[i], **rk), qb, None)
    runs["fused_row_amax_quantize_bf16_8192x4096"] = (
        lambda i: fos.fos_quantize_fused(xs[i], codes=codes[i], scales=scales[i], amax=ra, workspace=ws, status=st,
                                         **rk), qb, "one launch, each row read once")
    ct = torch.empty(K, M // 2, dtype=torch.uint8, device="cuda")
    stt = torch.empty(K, M // 16, dtype=torch.uint8, device="cuda")
    runs["quantize_columnwise_bf16_8192x4096"] = (
        lambda i: fos.fos_quantize_columnwise(xs[i], amax[i], codes=ct, scales=stt, **knobs), qb, None)
    sd = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(ns)]
    for i in range(ns):
        fos.fos_quantize(xs[i], amax[i], codes=codes[i], scales=scales[i], sdec=sd[i], **knobs)
    ys = [torch.empty_like(x) for x in xs]
    runs["dequantize_bf16_8192x4096"] = (
        lambda i: fos.nvfp4_dequantize(codes[i], scales[i], sd[i], "tensor", torch.bfloat16, out=ys[i]), qb, None)
    qkw = dict(recipe="4over6", err_metric="mse", err_prec="fp16", bound=448)
    runs["fused_amax_qdq_bf16_8192x4096_mse_fp16_448"] = (
        lambda i: fos.fos_qdq_fused(xs[i], out=ys[i], amax=amax[i], workspace=ws, status=st, **qkw), 4 * n,
        "one launch, x read once")
    runs["amax_then_qdq_bf16_8192x4096_mse_fp16_448"] = (
        lambda i: (fos.fos_amax(xs[i], "tensor", out=amax[i]), fos.fos_qdq(xs[i], amax[i], out=ys[i], **qkw)), 4 * n,
        "two launches; x read twice")
    for key, (fn, nbytes, note) in runs.items():
        ms = float(np.median(time_loop(fn, ns, 200, 10)))
        out[key] = entry(nbytes, ms, **({"note": note} if note else {}))
        log(f"[bench] {key}: {out[key]['avg_launch_us']} us, {out[key]['GB/s']} GB/s")
    out["fused_amax_quantize_bf16_8192x4096_phases"] = fused_phases(fos, torch, np, runs[
        "fused_amax_quantize_bf16_8192x4096"][0], ns)
    del xs, codes, scales, ys, row_amax, ct, stt

    # 16x16 weights, bf16 4096x14336 and fp32 4096x4096, per-tensor, MSE exact, 448
    for dtype, (M, K) in (("bf16", (4096, 14336)), ("fp32", (4096, 4096))):
        w = synthdata.weight(M, K, 31 if dtype == "bf16" else 32, dtype).to("cuda")
        a = fos.fos_amax(w, "tensor")
        eb = 2 if dtype == "bf16" else 4
        nbytes = M * K * eb + M * K // 2 + M * K // 16
        wsets = rotating(w, nbytes)
        cc = torch.empty(M, K // 2, dtype=torch.uint8, device="cuda")
        ss = torch.empty(M, K // 16, dtype=torch.uint8, device="cuda")
        ms = float(np.median(time_loop(lambda i: fos.fos_quantize(wsets[i], a, codes=cc, scales=ss, block="16x16",
                                                                  **knobs), len(wsets), steps, warmup)))
        out[f"quantize_16x16_{dtype}_{M}x{K}"] = entry(nbytes, ms)
        log(f"[bench] 16x16 {dtype}: {out[f'quantize_16x16_{dtype}_{M}x{K}']}")
        del wsets, w

    # fused QDQ over the 8 expert weights 2048x7168, bf16 and fp16, the five
    # timed modes, each list rotated over >= 1 GiB (3 copies)
    lst = synthdata.expert_weight_list(8, 2048, 7168, 40, dtypes=("bf16", "fp16"))
    lws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    lst_status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for dtype in ("bf16", "fp16"):
        base = [t.to("cuda") for t in lst[dtype]]
        nbytes = sum(t.numel() for t in base) * 4
        nsets = max(3, -(-FOOTPRINT // nbytes))
        sets = [[t.clone() for t in base] for _ in range(nsets)]
        ams = [[fos.fos_amax(t, "tensor") for t in xs_] for xs_ in sets]
        ys = [[torch.empty_like(t) for t in xs_] for xs_ in sets]
        for r, m, p, bnd in (("nvfp4", "mse", "fp16", 448), ("4over6", "mae", "fp16", 448),
                             ("4over6", "mae", "fp16", 256), ("4over6", "mse", "fp16", 448),
                             ("4over6", "mse", "fp16", 256)):
            ms = float(np.median(time_loop(lambda i: fos.fos_qdq_list(sets[i], ams[i], outs=ys[i], recipe=r,
                                                                      err_metric=m, err_prec=p, bound=bnd),
                                           nsets, steps, warmup)))
            key = f"qdq_list_8x2048x7168_{dtype}_{r}" + ("" if r == "nvfp4" else f"_{m}_{p}_{bnd}")
            out[key] = entry(nbytes, ms, rotating_sets=nsets)
            log(f"[bench] {key}: {out[key]['avg_launch_us']} us, {out[key]['GB/s']} GB/s")
            # the same list with every weight's amax computed in the launch
            # (the end-to-end step of the fake-quantization loop)
            fa = [torch.empty(8, dtype=torch.float32, device="cuda") for _ in range(nsets)]
            ms = float(np.median(time_loop(lambda i: fos.fos_qdq_list_fused(sets[i], outs=ys[i], amax=fa[i], recipe=r,
                                                                            err_metric=m, err_prec=p, bound=bnd,
                                                                            workspace=lws, status=lst_status),
                                           nsets, steps, warmup)))
            out["fused_amax_" + key] = entry(nbytes, ms, rotating_sets=nsets,
                                             note="one launch: every amax, then the QDQ; x read twice")
            log(f"[bench] fused_amax_{key}: {ms * 1e3:.2f} us, {gbs(nbytes, ms)} GB/s")
        del sets, ys, ams, base

    # the QDQ workload the Megatron-LM page times ("Performance": 8 discrete
    # contiguous [4096, 6144] weights, precomputed per-tensor amax, 1x16 along
    # 6144, the five FP16-error modes), synthetic weights of the expert-list
    # recipe; its B300 medians are quoted beside ours (other hardware: context)
    lst = synthdata.expert_weight_list(8, 4096, 6144, 60, dtypes=("bf16", "fp16"))
    for dtype in ("bf16", "fp16"):
        base = [t.to("cuda") for t in lst[dtype]]
        nbytes = sum(t.numel() for t in base) * 4
        nsets = max(2, -(-FOOTPRINT // nbytes))
        sets = [[t.clone() for t in base] for _ in range(nsets)]
        ams = [[fos.fos_amax(t, "tensor") for t in xs_] for xs_ in sets]
        ys = [[torch.empty_like(t) for t in xs_] for xs_ in sets]
        for (r, m, bnd), pages_us in zip(PAGES_QDQ_MODES, PAGES_QDQ_US[dtype]):
            ms = float(np.median(time_loop(lambda i: fos.fos_qdq_list(sets[i], ams[i], outs=ys[i], recipe=r,
                                                                      err_metric=m, err_prec="fp16", bound=bnd),
                                           nsets, steps, warmup)))
            key = f"qdq_list_8x4096x6144_{dtype}_{r}" + ("" if r == "nvfp4" else f"_{m}_fp16_{bnd}")
            out[key] = entry(nbytes, ms, rotating_sets=nsets, pages_b300_us=pages_us)
            log(f"[bench] {key}: {out[key]['avg_launch_us']} us (B300 on the page: {pages_us} us)")
        del sets, ys, ams, base
    out["fused_calls_status_clean"] = int(lst_status.item()) == 0 and int(st.item()) == 0 and int(gst.item()) == 0
    return out


# The Megatron-LM page's precomputed-amax medians (radixark/Megatron-LM PR
# "Fuse NVFP4 fake-QAT quantize-dequantize with CuTe DSL", "Performance"),
# B300, 8 x [4096, 6144], microseconds, in the order of PAGES_QDQ_MODES.
PAGES_QDQ_MODES = (("nvfp4", "mse", 448), ("4over6", "mae", 448), ("4over6", "mae", 256), ("4over6", "mse", 448),
                   ("4over6", "mse", 256))
PAGES_QDQ_US = {"bf16": (156.813, 213.055, 213.064, 216.156, 216.315),
                "fp16": (157.402, 213.018, 213.021, 213.625, 213.596)}


def fused_phases(fos, torch, np, launch, n_sets):
    """Per-wave phase times of one one-read fused launch (the library's
    timestamp diagnostics) on a buffer set last read n_sets launches
    earlier, after 20 untimed launches: microseconds after the earliest wave
    start at which the waves' loads have landed, the barrier releases them
    and they end."""
    for i in range(20):
        launch(i % n_sets)
    buf = torch.zeros(65536, 4, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    khz = fos.set_phase_timestamps(buf)
    try:
        launch(20 % n_sets)
        torch.cuda.synchronize()
    finally:
        fos.set_phase_timestamps(None)
    t = buf.cpu().numpy()
    t = t[t[:, 0] != 0]
    us = (t - t[:, 0].min()) * (1e3 / khz)
    pct = lambda c, qs: [round(float(np.percentile(us[:, c], q)), 2) for q in qs]
    return {"waves": int(t.shape[0]), "clock_khz": khz,
            "start_us_p50_max": pct(0, (50, 100)),
            "loads_landed_us_min_p50_max": pct(1, (0, 50, 100)),
            "barrier_released_us_min_max": pct(2, (0, 100)),
            "end_us_min_p50_max": pct(3, (0, 50, 100))}


# ---------------------------------------------------------------- profile pass

def profile_pass(fos, synthdata, torch, np):
    """A few launches of each kernel with a counter summary, each workload's
    buffers rotated over >= 1 GiB, then a plain copy of known size that
    calibrates the HBM counters."""
    reps = 10
    _, _, xd, od, gam = grouped_inputs(torch, fos, synthdata)
    c = torch.empty(M5 + PAD5, K5 // 2, dtype=torch.uint8, device="cuda")
    s = torch.empty(M5 + PAD5, K5 // 16, dtype=torch.uint8, device="cuda")
    for _ in range(reps):
        fos.fos_quantize_grouped(xd, od, gam, codes=c, scales=s, **KNOBS)
    torch.cuda.synchronize()
    del xd, c, s

    w = synthdata.weight(4096, 14336, 31, "bf16").to("cuda")
    a = fos.fos_amax(w, "tensor")
    wsets = rotating(w, COUNTER_KERNELS["void fos::k_16x16<0, 1, 1, 0, 0, 0>(fos::Args16x16)"][2])
    c = torch.empty(4096, 14336 // 2, dtype=torch.uint8, device="cuda")
    s = torch.empty(4096, 14336 // 16, dtype=torch.uint8, device="cuda")
    for i in range(reps):
        fos.fos_quantize(wsets[i % len(wsets)], a, codes=c, scales=s, block="16x16", **KNOBS)
    torch.cuda.synchronize()
    del wsets, w, c, s

    base = synthdata.expert_weight_list(8, 2048, 7168, 40, dtypes=("bf16",))["bf16"]
    sets = [[t.to("cuda") for t in base] for _ in range(3)]
    ams = [[fos.fos_amax(t, "tensor") for t in xs_] for xs_ in sets]
    ys = [[torch.empty_like(t) for t in xs_] for xs_ in sets]
    for i in range(reps):
        fos.fos_qdq_list(sets[i % 3], ams[i % 3], outs=ys[i % 3], recipe="4over6", err_metric="mse", err_prec="fp16",
                         bound=448)
    torch.cuda.synchronize()
    del sets, ams, ys

    M, K = 8192, 4096
    x0 = synthdata.activation_family("normal", M, K, 21, "bf16").to("cuda")
    xs = rotating(x0, _N2 * 2 + _N2 // 2 + _N2 // 16)
    ns = len(xs)
    codes = [torch.empty(M, K // 2, dtype=torch.uint8, device="cuda") for _ in range(ns)]
    scales = [torch.empty(M, K // 16, dtype=torch.uint8, device="cuda") for _ in range(ns)]
    amax = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(ns)]
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    for i in range(reps):
        fos.fos_quantize_fused(xs[i % ns], codes=codes[i % ns], scales=scales[i % ns], amax=amax[i % ns],
                               workspace=ws, **KNOBS)
    for i in range(reps):
        fos.fos_quantize(xs[i % ns], amax[i % ns], codes=codes[i % ns], scales=scales[i % ns], **KNOBS)
    torch.cuda.synchronize()
    del xs, codes, scales

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] profile pass done (copy kernel: {COPY_BYTES} bytes read and written per launch)")


# ---------------------------------------------------------------- profile summaries

PROFILE_CMDS = {
    "kt": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt -o kt -- "
          "python3 $REPO/bench.py --no-cpu-baseline --no-other",
    "kt_pass": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/kt_pass -o kt_pass -- "
               "python3 $REPO/bench.py --profile-pass",
    "fetch": "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/fetch -o fetch -- "
             "python3 $REPO/bench.py --profile-pass",
    "write": "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write -o write -- "
             "python3 $REPO/bench.py --profile-pass",
    "sq": "timeout -s KILL 120 rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_CVT SQ_ACTIVE_INST_VALU "
          "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE --output-format csv "
          "-d $OUT/sq -o sq -- python3 $REPO/bench.py --profile-pass",
    "occ": "timeout -s KILL 120 rocprofv3 --pmc OccupancyPercent VALUBusy --output-format csv "
           "-d $OUT/occ -o occ -- python3 $REPO/bench.py --profile-pass",
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
    m = re.match(r"void fos::k_fused_(row|grouped)<(\d), (\d), (\d), (\d), (\d)>", name)
    if m:
        kind, dt, rc, mt, pr, od = m.groups()
        err = f" {_MT[mt]} {_PR[pr]}{_ORD[od]}" if rc == "1" else ""
        return f"fused {kind} amaxes + 1x16 quantize {_DT[dt]} {_RC[rc]}{err}"
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
        return "amax per tensor"
    if "k_amax_row" in name:
        return "amax per row"
    if "k_zero_u32" in name:
        return "clear the amax word"
    if "k_stream" in name:
        return "streaming ceiling"
    if "copyBuffer" in name:
        return "runtime copy"
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


def _trace(path):
    """{kernel: [(duration_ns, vgpr, lds_bytes, grid, workgroup)]} from a rocprofv3 kernel-trace CSV."""
    import csv
    per = {}
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))  # dispatch order
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), int(r["VGPR_Count"]), int(r["LDS_Block_Size"]),
             int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"])))
    return per


def alg_blocks(stem: str) -> int:
    """16-element blocks (units of quantizer work) one launch of the counter
    workload `stem` processes, padding rows of the grouped tensor included."""
    return {"quantize_grouped_bf16_65536x7168": (M5 + PAD5) * K5 // 16,
            "quantize_16x16_bf16_4096x14336": 4096 * 14336 // 16,
            "qdq_list_bf16_8x2048x7168": 8 * 2048 * 7168 // 16,
            "fused_amax_quantize_bf16_8192x4096": _N2 // 16,
            "quantize_1x16_bf16_8192x4096": _N2 // 16}[stem]


RESOURCES = os.path.join(PROFILES, "kernel_resources_gfx950.txt")


def kernel_resources(kernel: str, path: str | None = None) -> dict:
    """The compiler's resource figures of one kernel instance (VGPRs, SGPRs,
    spills, LDS, the waves per SIMD they allow) from the committed summary,
    or {} when it is absent or was taken on other kernel code."""
    path = path or RESOURCES
    if not os.path.exists(path):
        return {}
    lines = open(path).read().splitlines()
    if f"# kernel_source_sha256_16 = {kernel_source_hash()}" not in lines:
        return {}
    for line in lines:
        if line.startswith(kernel + " |"):
            return dict(kv.split("=", 1) for kv in line.split("|", 1)[1].split())
    return {}


def provenance(agent_csv=None):
    """Provenance lines: the device (from rocprofv3's agent table when given,
    else from torch), the software versions and the source hashes."""
    import csv
    import platform

    import torch
    lines = []
    gpu = cpu = None
    if agent_csv and os.path.exists(agent_csv):
        agents = list(csv.DictReader(open(agent_csv)))
        gpu = next((r for r in agents if r["Agent_Type"] == "GPU"), None)
        cpu = next((r for r in agents if r["Agent_Type"] == "CPU"), None)
    if gpu:
        lines += [f"gpu = {gpu['Name']} ({gpu['Vendor_Name']}), {gpu['Cu_Count']} CUs, {gpu['Simd_Count']} SIMDs, "
                  f"{gpu['Num_Xcc']} XCDs, {gpu['Max_Waves_Per_Simd']} waves per SIMD, {gpu['Lds_Size_In_Kb']} KiB LDS "
                  f"per CU, max engine clock {gpu['Max_Engine_Clk_Fcompute']} MHz"]
    # the profiled host's cores (rocprofv3's CPU agent), else this host's
    host = [f"profiled_host_cores = {cpu['Cpu_Cores_Count']}"] if cpu else [
        f"host_cores = {os.cpu_count()}", f"omp_num_threads = {os.environ.get('OMP_NUM_THREADS', '?')}"]
    lines += [f"torch = {torch.__version__}", f"hip = {torch.version.hip}", f"python = {platform.python_version()}",
              *host,
              f"kernel_source_sha256_16 = {kernel_source_hash()}",
              f"bench_sha256_16 = {hashlib.sha256(open(os.path.abspath(__file__), 'rb').read()).hexdigest()[:16]}"]
    return lines


def write_profiles(d, out_dir=PROFILES):
    """Write the kernel-trace summary of the step and the counter summary of
    each kernel in COUNTER_KERNELS into out_dir from the CSV files rocprofv3
    wrote under d."""
    import synthdata
    os.makedirs(out_dir, exist_ok=True)
    x, offs, _ = synthdata.grouped_tokens(M5, PAD5, K5, G5)
    prov = provenance(os.path.join(d, "kt", "kt_agent_info.csv")) + [
        f"input_sha256_grouped_bf16_{M5 + PAD5}x{K5} = {synthdata.sha256(x)}",
                           f"input_sha256_grouped_offs = {hashlib.sha256(offs.tobytes()).hexdigest()}"]
    del x
    hdr = "# command (after: cd /tmp && export TMPDIR=/tmp; OUT = an output folder, REPO = this repository):"

    # the step's kernel trace: every launch of the bench's default step (warmup included)
    kt = _trace(os.path.join(d, "kt", "kt_kernel_trace.csv"))
    durs = [t[0] for t in kt[HEADLINE_KERNEL]]
    v, l, g, wg = kt[HEADLINE_KERNEL][0][1:]
    lines = ["# rocprofv3 kernel trace of the bench's step: fos_quantize_grouped, bf16 65536 (+4096 padding) x 7168,",
             "# 64 groups, four-over-six MSE exact, bound 448 (warmup and timed launches)", hdr,
             "#   " + PROFILE_CMDS["kt"], "#   python3 $REPO/bench.py --write-profiles $OUT --profiles-out $REPO/profiles",
             *prov, "# durations in microseconds, per dispatch",
             f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9}  kernel"]
    for name, rows in sorted(kt.items(), key=lambda kv: -sum(r[0] for r in kv[1])):
        ds = [r[0] / 1e3 for r in rows]
        desc = describe_kernel(name)
        lines.append(f"{len(ds):6d} {sum(ds) / len(ds):9.2f} {min(ds):9.2f} {max(ds):9.2f}  "
                     f"{desc + ' | ' if desc else ''}{name[:100]}")
    timed = durs[-DEFAULT_STEPS:]  # the launches of the timed region (the untimed warmup comes first)
    lines += [f"headline_kernel = {HEADLINE_KERNEL}",
              f"headline_kernel_calls = {len(durs)}",
              f"headline_kernel_avg_us = {sum(durs) / len(durs) / 1e3:.2f}",
              f"headline_kernel_median_us = {sorted(durs)[len(durs) // 2] / 1e3:.2f}",
              f"headline_kernel_timed_calls = {len(timed)}",
              f"headline_kernel_timed_avg_us = {sum(timed) / len(timed) / 1e3:.2f}",
              f"grid_threads = {g}", f"workgroup = {wg}",
              *(f"compiler_{k} = {val}" for k, val in kernel_resources(HEADLINE_KERNEL).items()),
              f"algorithmic_bytes_per_launch = {STEP_BYTES}",
              f"achieved_GBs_at_avg = {STEP_BYTES / (sum(durs) / len(durs)) :.1f}"]
    open(os.path.join(out_dir, os.path.basename(HEADLINE_TRACE)), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))

    # per-workload kernel averages of the profile pass (each kernel below
    # runs for one workload only there)
    kp = _trace(os.path.join(d, "kt_pass", "kt_pass_kernel_trace.csv"))
    f = _counters(os.path.join(d, "fetch", "fetch_counter_collection.csv"))
    w = _counters(os.path.join(d, "write", "write_counter_collection.csv"))
    s = _counters(os.path.join(d, "sq", "sq_counter_collection.csv"))
    occ = _counters(os.path.join(d, "occ", "occ_counter_collection.csv"))
    copy_name = "__amd_rocclr_copyBuffer"
    cf = f[(copy_name, "FETCH_SIZE")][-4:]   # the profile pass ends with four copies of COPY_BYTES
    cw = w[(copy_name, "WRITE_SIZE")][-4:]
    mean = lambda vals: sum(vals) / len(vals)
    fetch_factor = COPY_BYTES / (mean(cf) * 1024)
    write_factor = COPY_BYTES / (mean(cw) * 1024)
    for kernel, (stem, what, alg) in COUNTER_KERNELS.items():
        rows = kp[kernel]
        us = mean([r[0] for r in rows]) / 1e3
        v, l, g, wg = rows[0][1:]
        rd = mean(f[(kernel, "FETCH_SIZE")]) * 1024 * fetch_factor
        wr = mean(w[(kernel, "WRITE_SIZE")]) * 1024 * write_factor
        get = lambda c: mean(s[(kernel, c)])
        insts, cvt = get("SQ_INSTS_VALU"), get("SQ_INSTS_VALU_CVT")
        # SQ_ACTIVE_INST_VALU counts quad-cycles (as rocprofv3's derived
        # VALUBusy and OccupancyPercent take the SQ cycle counters)
        valu_cyc = 4 * get("SQ_ACTIVE_INST_VALU") / N_SIMD
        blocks = alg_blocks(stem)
        occ_pct = mean(occ[(kernel, "OccupancyPercent")])
        lines = [f"# rocprofv3 counter summary: {what}",
                 "# commands (after: cd /tmp && export TMPDIR=/tmp; OUT = an output folder, REPO = this repository):",
                 *("#   " + PROFILE_CMDS[k] for k in ("kt_pass", "fetch", "write", "sq", "occ")),
                 "#   python3 $REPO/bench.py --write-profiles $OUT --profiles-out $REPO/profiles",
                 "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; the factors scale them to bytes so that the",
                 f"# profile pass's plain copy of {COPY_BYTES} bytes reads and writes exactly that many bytes.",
                 "# Each workload's buffers rotate over >= 1 GiB in the profile pass.",
                 f"kernel = {kernel}", *prov,
                 f"dispatches = {len(f[(kernel, 'FETCH_SIZE')])}",
                 f"kernel_avg_us = {us:.2f}   # profile-pass kernel trace",
                 f"achieved_GBs = {alg / (us * 1e3):.1f}",
                 f"fetch_size_kib = {mean(f[(kernel, 'FETCH_SIZE')]):.1f}",
                 f"write_size_kib = {mean(w[(kernel, 'WRITE_SIZE')]):.1f}",
                 f"copy_fetch_size_kib = {mean(cf):.1f}", f"copy_write_size_kib = {mean(cw):.1f}",
                 f"fetch_factor = {fetch_factor:.4f}", f"write_factor = {write_factor:.4f}",
                 f"hbm_read_bytes_per_launch = {rd:.0f}", f"hbm_write_bytes_per_launch = {wr:.0f}",
                 f"hbm_bytes_per_launch = {rd + wr:.0f}", f"algorithmic_bytes_per_launch = {alg}",
                 f"traffic_over_algorithmic = {(rd + wr) / alg:.4f}",
                 f"grid_threads = {g}",
                 *(f"compiler_{k} = {val}" for k, val in kernel_resources(kernel).items()),
                 f"occupancy_percent = {occ_pct:.1f}   # rocprofv3 OccupancyPercent (of 32 waves per CU)",
                 f"occupancy_waves_per_simd = {occ_pct / 100 * 8:.2f}",
                 f"valu_busy = {mean(occ[(kernel, 'VALUBusy')]) / 100:.4f}   # rocprofv3 VALUBusy",
                 f"sq_waves = {get('SQ_WAVES'):.0f}",
                 f"sq_insts_valu = {insts:.0f}   # wave instructions per dispatch",
                 f"sq_insts_valu_cvt = {cvt:.0f}",
                 f"sq_active_inst_valu = {get('SQ_ACTIVE_INST_VALU'):.0f}",
                 f"sq_wave_cycles = {get('SQ_WAVE_CYCLES'):.0f}",
                 f"sq_busy_cycles = {get('SQ_BUSY_CYCLES'):.0f}",
                 f"sq_wait_inst_any = {get('SQ_WAIT_INST_ANY'):.0f}",
                 f"grbm_gui_active = {get('GRBM_GUI_ACTIVE'):.0f}",
                 f"wait_over_wave_cycles = {get('SQ_WAIT_INST_ANY') / max(1.0, get('SQ_WAVE_CYCLES')):.4f}",
                 f"valu_cycles_per_simd = {valu_cyc:.0f}   # 4 x SQ_ACTIVE_INST_VALU / {N_SIMD} SIMDs",
                 f"cycles_per_valu_inst = {4 * get('SQ_ACTIVE_INST_VALU') / insts:.2f}",
                 f"valu_time_at_peak_clock_us = {valu_cyc / CLOCK_HZ * 1e6:.2f}   # at 2.4 GHz",
                 f"valu_lane_insts_per_block = {insts * 64 / blocks:.1f}   # 16-element blocks the launch processes",
                 f"valu_cvt_lane_insts_per_block = {cvt * 64 / blocks:.2f}"]
        path = os.path.join(out_dir, f"counters_{stem}.txt")
        open(path, "w").write("\n".join(lines) + "\n")
        print("\n".join(lines))


if __name__ == "__main__":
    main()
