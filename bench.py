"""Throughput of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one fa_fwd call (the whole forward: work decomposition, Q/K/V
tiles, both products, online softmax, normalisation, O and LSE stores) over
the workload's seeded synthetic inputs, already resident in HBM; decoding
workloads step through fa_fwd_splitkv, backward workloads through fa_bwd
(after an untimed forward), fp8 workloads through fa_fwd_fp8.  Prints one
JSON line on stdout; extra detail goes to stderr.

Default workload: B=8, H=32, L=4096, D=128, non-causal -- the shape the
throughput target is quoted on.  FLOPs = 4*B*H*L^2*D (halved when causal);
for queries after cached keys, 4*B*H*D per visible (query, key) pair with the
diagonal square counted half.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·L²·D, causal halved) + % of MFMA FP16 peak"
PEAK_FP16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense fp16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2  # dense E4M3: twice the fp16 rate
PEAK_HBM_GBS = 8000.0  # HBM3E, published
CSRC = os.path.join(ROOT, "tiled_attention_flash_amd", "csrc")
# the sources the kernels of each entry point are compiled from
KERNEL_SRCS = {path: [os.path.join(CSRC, f) for f in ("fa_device.h", "fa_internal.h", *srcs)]
               for path, srcs in (("forward", ("fa_fwd_kernel.hip",)), ("splitkv", ("fa_splitkv_kernel.hip",)),
                                  ("backward", ("fa_bwd_kernels.h", "fa_bwd_kernel.hip", "fa_bwd_kernel_d64.hip")),
                                  ("fp8", ("fa_fwd_fp8_kernel.hip",)))}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_sha(path: str = "forward") -> str:
    """Hash of the sources of one entry point's kernels (a workload's `path`),
    with comments and blank lines removed, so that an edit to comments alone
    keeps the counters taken on the same code, and of the extra compiler
    flags the build gives those sources."""
    from tiled_attention_flash_amd.build import SOURCE_FLAGS

    h = hashlib.sha256()
    for src in KERNEL_SRCS[path]:
        with open(src, encoding="utf-8") as f:
            code = _COMMENT.sub("", f.read())
        h.update("\n".join(line.rstrip() for line in code.splitlines() if line.strip()).encode())
        flags = SOURCE_FLAGS.get(os.path.basename(src))
        if flags:
            h.update(("\nflags: " + " ".join(flags)).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, valid
    only while the kernel source is the one the counters were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("kernel_sha") != kernel_sha(path):
        return None
    return entry.get("hbm_bytes_per_launch")


def _power_w():
    """Board power from the GPU's hwmon (power1_average, else power1_input),
    plain sysfs reads; None where not visible."""
    import glob

    for name in ("power1_average", "power1_input"):
        for p in sorted(glob.glob(f"/sys/class/drm/card*/device/hwmon/hwmon*/{name}")):
            try:
                with open(p) as f:
                    v = int(f.read().strip())
            except (OSError, ValueError):
                continue
            if v > 0:
                return v / 1e6
    return None


def sample_clock_power(step, seconds: float = 1.5, samples: int = 5):
    """Shader clock and board power while the same launches run, outside the
    timed region.  About `seconds` of launches are queued; meanwhile the
    clock probe of libfa_clock.so (one wavefront on a side stream counting
    shader cycles over a 200 us window of the 100 MHz real-time counter)
    runs `samples` times, and hwmon power is read beside it.  Medians are
    reported; None when the probe library is missing."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "tiled_attention_flash_amd", "libfa_clock.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.fa_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
    lib.fa_clock_probe.restype = ctypes.c_int
    # the result buffers are zeroed before the launches are queued: a fill
    # queued behind them would land after the probes have written
    side = torch.cuda.Stream()
    bufs = [torch.zeros(2, dtype=torch.int64, device="cuda") for _ in range(samples)]
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-4)
    for _ in range(int(seconds / one) + 1):
        step()
    watts = []
    time.sleep(0.15 * seconds)
    for b in bufs:
        with torch.cuda.stream(side):
            if lib.fa_clock_probe(b.data_ptr(), 20000, side.cuda_stream) != 0:
                return None
        p = _power_w()
        if p:
            watts.append(p)
        time.sleep(0.6 * seconds / samples)
    torch.cuda.synchronize()
    mhz = sorted(100.0 * c / r for c, r in (b.tolist() for b in bufs) if r > 0)
    watts.sort()
    if not mhz:
        return None
    return {"gfxclk_mhz": round(mhz[len(mhz) // 2]), "gfxclk_mhz_samples": [round(x) for x in mhz],
            "board_power_w": round(watts[len(watts) // 2]) if watts else None,
            "source": "libfa_clock.so probe (s_memtime cycles over a 100 MHz s_memrealtime window, "
                      "side stream) and hwmon power, while the same launches run, outside the "
                      "timed region; medians"}


def host_cpus() -> dict:
    """CPUs the host reports and the ones this process may run on."""
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        allowed = os.cpu_count() or 1
    return {"online": os.cpu_count(), "allowed": allowed}


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, q, k, v, target_s: float, descale=None):
    """The fp64 oracle timed on the host on a bounded sample of the same
    workload: whole output rows, the first ones of every (b, h) in turn."""
    import numpy as np

    import oracle

    threads = cpu_threads()

    def row_ids(n):
        rng = np.random.default_rng(0)
        b = rng.integers(0, w.B, n)
        h = rng.integers(0, w.H, n)
        i = rng.integers(0, w.L, n)
        return np.stack([b, h, i], axis=1)

    def flops(ids):
        if not w.causal:
            return 4.0 * w.keys * w.D * len(ids)
        return float(sum(4.0 * min(w.keys, int(i) + w.past_len + 1) * w.D for i in ids[:, 2]))

    def run(ids):
        if descale is not None:
            oracle.rows_fp8(q, k, v, ids, descale, causal=w.causal, scale=w.scale,
                            past_len=w.past_len, nthreads=threads)
        else:
            oracle.rows(q, k, v, ids, causal=w.causal, scale=w.scale, nthreads=threads,
                        past_len=w.past_len)

    ids = row_ids(threads * 8)
    t0 = time.perf_counter()
    run(ids)
    probe = time.perf_counter() - t0
    n = int(max(threads, min(2_000_000, len(ids) * target_s / max(probe, 1e-6))))
    ids = row_ids(n)
    t0 = time.perf_counter()
    run(ids)
    dt = time.perf_counter() - t0
    return {"value": flops(ids) / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} random output rows (b, h, i) of the same inputs, fp64, {dt:.1f} s",
            "host_cpus": host_cpus(),
            "threads_note": "oracle threads = the CPUs this process may run on, capped at 16 "
                            "(the host share of one GPU on a shared box)"}


VALU_MODES = {"exp_f32": 0, "exp_f16": 1, "fma_f32": 2}
MFMA_PROBE_MODES = {"random": 0, "structured": 1, "shared-b": 2, "low-bits": 3}


def run_probe(args) -> int:
    """The reference ceilings: a register-only stream of v_mfma_f32_32x32x16_f16
    (four independent chains per wavefront, two wavefronts per SIMD), one
    streaming read of a device buffer (16 bytes per lane, grid-strided), or
    the issue rate of one vector instruction kind (eight independent chains
    per wavefront, four wavefronts per SIMD), in cycles per wave64
    instruction per SIMD at the measured clock.
    Same timing as the workloads: warmup, then `--steps` launches between HIP
    events on the launch stream; clock and power sampled afterwards while the
    same launches run."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "tiled_attention_flash_amd", "libfa_clock.so")
    if not os.path.exists(path):
        print(f"{path} is not built", file=sys.stderr)
        return 1
    lib = ctypes.CDLL(path)
    lib.fa_probe_mfma_stream.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p,
                                         ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_valu_stream.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_mfma_stream.restype = lib.fa_probe_read_stream.restype = ctypes.c_int
    lib.fa_probe_valu_stream.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if args.mfma_probe:
        workgroups, iters = 8 * cus, 512  # 8 rounds of one 8-wavefront workgroup per CU
        mode = MFMA_PROBE_MODES[args.mfma_probe]
        out = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
        work = workgroups * 8 * iters * 32 * 32768.0  # flops per launch

        def step():
            if lib.fa_probe_mfma_stream(out.data_ptr(), out.numel(), workgroups, iters, mode,
                                        stream.cuda_stream) != 0:
                raise RuntimeError("fa_probe_mfma_stream rejected")
        name, unit, peak = f"mfma_stream_f16_{args.mfma_probe}", "TFLOP/s", PEAK_FP16_TFLOPS
    elif args.valu_probe:
        workgroups, iters = 4 * cus, 2000  # two rounds of two 8-wavefront workgroups per CU
        mode = VALU_MODES[args.valu_probe]
        out = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
        work = workgroups * 8 * iters * 8.0  # wave64 instructions per launch

        def step():
            if lib.fa_probe_valu_stream(out.data_ptr(), out.numel(), workgroups, iters, mode,
                                        stream.cuda_stream) != 0:
                raise RuntimeError("fa_probe_valu_stream rejected")
        name, unit, peak = f"valu_stream_{args.valu_probe}", "instr/ns", None
    else:
        nbytes = args.read_probe_mib * (1 << 20)
        buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        workgroups = 16 * cus
        out = torch.empty(workgroups * 256, dtype=torch.int32, device=dev)
        work = float(nbytes)  # bytes per launch

        def step():
            if lib.fa_probe_read_stream(buf.data_ptr(), nbytes, out.data_ptr(), out.numel(),
                                        workgroups, stream.cuda_stream) != 0:
                raise RuntimeError("fa_probe_read_stream rejected")
        name, unit, peak = "read_stream", "GB/s", PEAK_HBM_GBS
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize(dev)
    ms = t0.elapsed_time(t1) / args.steps
    rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    result = {"probe": name, "value": round(rate, 1), "unit": unit, "peak": peak,
              "frac_of_peak": round(rate / peak, 4) if peak else None, "ms_per_launch": round(ms, 4),
              "steps": args.steps, "warmup": args.warmup, "compute_units": cus,
              "workgroups": workgroups}
    if args.mfma_probe:
        result["flops_per_launch"] = work
    elif args.valu_probe:
        result["instructions_per_launch"] = work
        result["ns_per_instruction_per_simd"] = round(ms * 1e6 / (work / (4 * cus)), 4)
    else:
        result["bytes_per_launch"] = int(work)
    clock = sample_clock_power(step)
    if clock and args.valu_probe and (clock["gfxclk_mhz"] or 0) >= 500:
        result["cycles_per_instruction_per_simd"] = round(
            result["ns_per_instruction_per_simd"] * clock["gfxclk_mhz"] / 1000.0, 2)
    if clock and unit == "TFLOP/s" and (clock["gfxclk_mhz"] or 0) >= 500:
        clock["peak_at_clock_tflops"] = round(peak * clock["gfxclk_mhz"] / 2400.0, 1)
        clock["frac_at_clock"] = round(rate / clock["peak_at_clock_tflops"], 4)
    result["clock"] = clock
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB "
                         "`--steps` times (the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--mfma-probe", choices=sorted(MFMA_PROBE_MODES), default=None,
                    help="instead of the benchmark, time the register-only fp16 MFMA stream of "
                         "libfa_clock.so on random operands (the sustained matrix-unit ceiling "
                         "for data like the workloads'), on few distinct small values, on random "
                         "operands with B shared by four consecutive MFMAs, or on random operands "
                         "with the 5 low fraction bits zero")
    ap.add_argument("--valu-probe", choices=sorted(VALU_MODES), default=None,
                    help="instead of the benchmark, time a register-only stream of one vector "
                         "instruction kind (libfa_clock.so): cycles per wave64 instruction per SIMD")
    ap.add_argument("--read-probe-mib", type=int, default=0,
                    help="instead of the benchmark, time a streaming read of this many MiB of "
                         "device memory (libfa_clock.so): the practical HBM read ceiling")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the attention kernels here work on one GPU's "
              "share of a problem and no multi-GPU path is built.",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.float16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 2 * n, "copy_probe_bytes_written": 2 * n,
                          "launches": args.steps}), flush=True)
        return 0

    if args.mfma_probe or args.read_probe_mib or args.valu_probe:
        return run_probe(args)

    import tiled_attention_flash_amd as fa
    from tiled_attention_flash_amd.inputs import HEADLINE, WORKLOADS, workload_inputs

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.path == "backward":
        from tiled_attention_flash_amd.inputs import make_qkvdo
        q, k, v, do = make_qkvdo(w.B, w.L, w.H, w.Hkv, w.D, seed=args.seed, qk_mult=w.qk_mult)
    elif w.path == "fp8":
        q, k, v, descale = workload_inputs(w, seed=args.seed)
    else:
        q, k, v = workload_inputs(w, seed=args.seed)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty(tuple(q.shape), dtype=torch.float16, device=dev)
    peak = PEAK_FP8_TFLOPS if w.path == "fp8" else PEAK_FP16_TFLOPS
    lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if w.path == "backward":
        # the forward's O and LSE are inputs of the backward, resident before timing
        fa.forward(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse)
        dod = do.to(dev)
        gq, gk, gv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        delta = torch.empty_like(lse)
        n_splits = None

        def step():
            fa.backward(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, dq=gq, dk=gk,
                        dv=gv, delta=delta)
    elif w.path == "splitkv":
        n_splits = fa.fa_splitkv_splits(w.B, w.L, w.keys, w.H, w.Hkv, w.D, w.causal, w.past_len)
        ws = torch.empty(fa.fa_splitkv_workspace_bytes(w.B, w.L, w.H, w.D, n_splits),
                         dtype=torch.uint8, device=dev)

        def step():
            fa.forward_splitkv(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse,
                               past_len=w.past_len, n_splits=n_splits, workspace=ws)
    elif w.path == "fp8":
        n_splits = None

        def step():
            fa.forward_fp8(qd, kd, vd, descale=descale, causal=w.causal, scale=w.scale, out=o,
                           lse=lse, past_len=w.past_len)
    else:
        n_splits = None

        def step():
            fa.forward(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse,
                       past_len=w.past_len)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    # timed region: one event pair per launch (kernel duration) inside one
    # bracketing pair (whole-job time), all on the stream the kernel runs on
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t_begin.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize(dev)
    total_ms = t_begin.elapsed_time(t_end)
    per_launch = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    kernel_ms = sum(per_launch) / len(per_launch)
    ms_per_step = total_ms / args.steps

    value = w.step_flops / (ms_per_step * 1e-3) / 1e12
    traffic = measured_traffic(name, w.path)
    if w.path == "splitkv":
        # decoding reads each K/V byte once and does ~1 flop per byte: HBM-bound
        achieved = w.algorithmic_bytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes": w.algorithmic_bytes}
    else:
        achieved = w.step_flops / (kernel_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}
        if w.path == "backward":
            roofline["flops_counted"] = "2.5 x 4*B*H*L^2*D (S, dP, dV, dK, dQ), causal halved"
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if w.path == "fp8" else "f16",
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "L": w.L, "D": w.D,
                   "causal": w.causal, "layout": "BSHD", "seed": args.seed,
                   **({"Lk": w.keys, "past_len": w.past_len} if w.keys != w.L else {}),
                   **({"entry_point": "fa_fwd_splitkv", "n_splits": n_splits}
                      if n_splits is not None else {}),
                   **({"entry_point": "fa_bwd"} if w.path == "backward" else {}),
                   **({"entry_point": "fa_fwd_fp8", "inputs": "E4M3, one descale per tensor",
                       "output": "fp16"} if w.path == "fp8" else {})},
        "pct_peak": round(100.0 * value / peak, 2),
        "roofline": roofline,
        "kernel_ms_mean": round(kernel_ms, 5),
        "kernel_ms_median": round(per_launch[len(per_launch) // 2], 5),
        "kernel_sha": kernel_sha(w.path),
    }
    print(f"[bench] {name}: {ms_per_step:.4f} ms/step, kernel {kernel_ms:.4f} ms, "
          f"{value:.1f} TFLOP/s ({result['pct_peak']}% of {peak})",
          file=sys.stderr, flush=True)
    clock = sample_clock_power(step)
    if clock and (clock["gfxclk_mhz"] or 0) >= 500 and w.path != "splitkv":
        # the published peak assumes 2.4 GHz; the same peak at the clock the part ran
        peak_at_clock = peak * clock["gfxclk_mhz"] / 2400.0
        clock["peak_at_clock_tflops"] = round(peak_at_clock, 1)
        clock["frac_at_clock"] = round(achieved / peak_at_clock, 4)
    result["clock"] = clock
    if not args.no_cpu_baseline and w.path != "backward":
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds,
                                              descale if w.path == "fp8" else None)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
