#!/usr/bin/env python3
"""Benchmark of the GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the hot path: gemm_f32 on the fp32 4096^3 row-major
product (A, B ~ U[-1, 1] from fixed seeds, alpha = 1, beta = 0), inputs
resident in device memory.  W untimed steps, then exactly K timed steps
between two synchronisations; the JSON line reports TFLOP/s = 2MNK / t.
Each kernel's replay-protocol leg (below) runs before its timed steps, so
those start with the part at its loaded clock rather than ramping up from
the idle of input generation.

Also reported on the same line:
  * roofline: the GEMM kernel's achieved TFLOP/s from HIP events around each
    launch in the timed region, against the fp32 matrix peak (157.3 TFLOP/s),
    and HBM traffic per launch from the committed rocprofv3 counter summary
    when it was taken on the current kernel sources (else null);
  * timed_window: median, first and last launch of the timed steps, and the
    rate over their first and last quarter (the clock's drift inside them);
  * p4_protocol: the replay schedule of the SGEMM summary's benchmarking
    section -- floor(1000*exp((1024-n)/3100)) replays, cache flushed before
    each (outside the timed interval), mean of the second half;
  * fp16: the same for gemm_f16 on the fp16 4096^3 GEMM with beta = 0.5;
  * fp16_out_fp32: gemm_f16f32 (fp16 A and B, fp32 C and result) on the same
    shape with beta = 0.5 (launch timing only);
  * valu_ablation: gemm_f32_valu (the pages' SIMT register-blocked design on
    the vector ALUs) on the fp32 4096^3 workload, against the fp32 vector
    peak (157.3 TFLOP/s), next to the matrix-core result;
  * power (per precision): average socket power and graphics clock over a
    few seconds of back-to-back calls, read from the SMU through amdsmi, the
    energy per GEMM and GFLOP/J, and the matrix peak scaled to the measured
    clock (peak x clock / 2400 MHz); null where amdsmi is unavailable;
  * mfma_ceiling (per precision): the matrix-core ceiling probe of the
    library (gemm_probe_mfma: the GEMM's MFMA instruction on register operands
    drawn like the GEMM inputs, no memory traffic) timed with HIP events and
    under the same power window: the rate the part sustains at the clock it
    holds under matrix-core load, and each GEMM's fraction of it;
  * cpu_baseline: the CPU oracle timed on this host on a bounded sample of
    the same workload (a subset of output rows).

    python bench.py --table    one JSON row per workload of the pages'
                               measurements, GPU next to the whole-product oracle
    python bench.py --sweep    the fp32 square sweep 1024..12800
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F32 = 157.3      # TFLOP/s, MI355X dense fp32 matrix
# MI355X's published fp32 vector peak: 256 CUs x 4 SIMDs x 64 flops per clock x
# 2.4 GHz.  (A 16-lane-per-clock count would give 78.6; the vector-ALU kernel,
# non-packed v_fmac_f32 only, measures ~82 TFLOP/s, so that count is too low.)
PEAK_F32_VALU = 157.3
PEAK_F16 = 2516.6     # TFLOP/s, MI355X dense fp16 matrix
PEAK_HBM = 8000.0     # GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


from dense_gemm_fp32_amd.model import replay_count  # noqa: E402


def _code_only(text):
    """C++ source without comments or whitespace (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            if not text[i].isspace():
                out.append(text[i])
            i += 1
    return "".join(out)


# Sources of the kernels whose HBM traffic the committed counter summary
# holds (the 4096^3 GEMM kernels: their templates, tile tables and shared
# device code); the other sources build other kernels.
TRAFFIC_SOURCES = ("common.hpp", "gemm_f16.hip", "gemm_f32.hip", "internal.hpp")


def kernel_source_hash():
    """Hash of the measured kernels' sources (comments and layout excluded),
    so that a committed counter summary stays valid across comment edits and
    edits of other kernels' sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_fp32_amd", "csrc")
    for name in TRAFFIC_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(key):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_hash") != kernel_source_hash():
        return None
    ent = data.get("kernels", {}).get(key)
    if not ent:
        return None
    return ent.get("hbm_bytes_per_launch")


NOMINAL_SCLK_MHZ = 2400.0


def smi_handle(torch, dev):
    """amdsmi handle of `dev` (matched by PCI bus), or None without amdsmi."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
    except Exception:
        return None, None
    if not handles:
        return None, None
    props = torch.cuda.get_device_properties(dev)
    for h in handles:
        try:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
            if int(bdf.split(":")[1], 16) == props.pci_bus_id:
                return amdsmi, h
        except Exception:
            continue
    return amdsmi, handles[0]


def clock_sample(smi, h):
    """Mean of the per-XCD graphics clocks in MHz from the SMU's metrics
    table (refreshed every few milliseconds, so meaningful only after tens of
    milliseconds of steady load); None without amdsmi."""
    if h is None:
        return None
    try:
        m = smi.amdsmi_get_gpu_metrics_info(h)
        clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int) and c < 0xFFFF]
        return round(sum(clks) / len(clks), 1) if clks else None
    except Exception:
        return None


def smu_snapshot(smi, h):
    """The SMU's cumulative counters: energy (J) with its timestamp (s), and
    the residency accumulators of package-power (PPT) and socket-thermal
    throttling with their common denominator; None without amdsmi."""
    if h is None:
        return None
    try:
        e = smi.amdsmi_get_energy_count(h)
        m = smi.amdsmi_get_gpu_metrics_info(h)
        return {"j": e["energy_accumulator"] * e["counter_resolution"] * 1e-6,
                "t": e["timestamp"] * 1e-9, "acc": m.get("accumulation_counter"),
                "ppt": m.get("ppt_residency_acc"), "thm": m.get("socket_thm_residency_acc")}
    except Exception:
        return None


def smu_between(a, b):
    """Average socket power and throttle residencies between two snapshots
    (the energy counter refreshes about once a second: short intervals read
    as None)."""
    out = {"avg_socket_power_w": None, "ppt_throttle_residency": None,
           "thermal_throttle_residency": None}
    if not a or not b:
        return out
    if b["t"] > a["t"] and b["j"] > a["j"]:
        out["avg_socket_power_w"] = round((b["j"] - a["j"]) / (b["t"] - a["t"]), 1)
    try:
        dacc = b["acc"] - a["acc"]
        if dacc > 0:
            out["ppt_throttle_residency"] = round((b["ppt"] - a["ppt"]) / dacc, 4)
            out["thermal_throttle_residency"] = round((b["thm"] - a["thm"]) / dacc, 4)
    except Exception:
        pass
    return out


def launch_stats(launch_ms, flops):
    """How the per-launch times of a timed window move: first and last
    launch, median, and the mean of the first and of the last quarter."""
    n = len(launch_ms)
    q = max(1, n // 4)
    first_q = sum(launch_ms[:q]) / q
    last_q = sum(launch_ms[-q:]) / q
    return {"median_launch_ms": round(sorted(launch_ms)[n // 2], 5),
            "first_launch_ms": round(launch_ms[0], 5), "last_launch_ms": round(launch_ms[-1], 5),
            "first_quarter_tflops": round(flops / (first_q * 1e-3) / 1e12, 2),
            "last_quarter_tflops": round(flops / (last_q * 1e-3) / 1e12, 2)}


def power_window(torch, dev, call, flops, peak, seconds, warm=1.5):
    """Back-to-back calls for `warm` + `seconds` seconds.  Power is the SMU
    energy accumulator's increase over its own timestamps between two reads
    taken under load (the SMU refreshes it about once a second, so both
    snapshots fall inside the loaded interval); clocks are the per-XCD
    graphics clocks sampled in between.  Returns None without amdsmi."""
    smi, h = smi_handle(torch, dev)
    if h is None:
        return None

    def energy():
        e = smi.amdsmi_get_energy_count(h)
        return e["energy_accumulator"] * e["counter_resolution"] * 1e-6, e["timestamp"] * 1e-9

    def run_for(sec, samples=None):
        calls, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < sec:
            for _ in range(16):
                call()
            calls += 16
            torch.cuda.synchronize(dev)
            if samples is not None:
                try:
                    m = smi.amdsmi_get_gpu_metrics_info(h)
                    clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int) and c < 0xFFFF]
                    samples.append((sum(clks) / len(clks) if clks else None,
                                    m.get("current_socket_power")))
                except Exception:
                    pass
        return calls, time.perf_counter() - t0

    try:
        run_for(warm)
        e0, ts0 = energy()
        snap0 = smu_snapshot(smi, h)
        samples = []
        calls, wall = run_for(seconds, samples)
        e1, ts1 = energy()
        snap1 = smu_snapshot(smi, h)
    except Exception:
        return None
    if ts1 <= ts0:
        return None
    watts = (e1 - e0) / (ts1 - ts0)
    clks = [c for c, _ in samples if c]
    clk = sum(clks) / len(clks) if clks else None
    per_call_s = wall / calls
    joules = watts * per_call_s
    res = {"avg_socket_power_w": round(watts, 1),
           "window_s": round(wall, 2), "calls": calls,
           "ms_per_call": round(per_call_s * 1e3, 5),
           "energy_per_gemm_j": round(joules, 6),
           "gflop_per_j": round(flops / joules / 1e9, 1),
           "avg_gfxclk_mhz": round(clk, 1) if clk else None,
           "clock_adjusted_peak": round(peak * clk / NOMINAL_SCLK_MHZ, 1) if clk else None}
    if clk:
        res["frac_of_clock_adjusted_peak"] = round(flops / per_call_s / 1e12 / res["clock_adjusted_peak"], 4)
    thr = smu_between(snap0, snap1)
    res["ppt_throttle_residency"] = thr["ppt_throttle_residency"]
    res["thermal_throttle_residency"] = thr["thermal_throttle_residency"]
    return res


def mfma_ceiling(torch, dev, stream, dg, wl, dtype, peak, seconds):
    """The library's matrix-core ceiling probe on operands drawn like the
    GEMM inputs (U[-1, 1], rounded to the operand type): launches of ~20 ms,
    TFLOP/s from HIP events over 10 launches, then a power window."""
    tname = "f16" if dtype == 1 else "f32"
    vals = wl.draw(1, 65536 // (2 if dtype == 1 else 4), "uniform", 17, tname).reshape(-1)
    ops = torch.from_numpy(vals).to(dev)
    out = torch.empty(512 * 512, dtype=torch.float32, device=dev)

    def launch(iters):
        rc, fl = dg.gemm_probe_mfma(dtype, iters, ops, out, stream)
        if rc != 0:
            raise RuntimeError("gemm_probe_mfma returned %d: %s" % (rc, dg.gemm_status_string(rc)))
        return fl

    def timed(iters, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fl = launch(iters)
        b.record(stream)
        b.synchronize()
        return fl, a.elapsed_time(b) / n

    iters = 256
    timed(iters, 1)
    _, ms = timed(iters, 2)
    iters = max(1, int(iters * 20.0 / max(ms, 1e-3)))
    timed(iters, 5)                       # bring the clock to its loaded level
    fl, ms = timed(iters, 10)
    res = {"instruction": "v_mfma_f32_16x16x32_f16" if dtype == 1 else "v_mfma_f32_32x32x2_f32",
           "iters": iters, "ms_per_launch": round(ms, 4),
           "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
           "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / peak, 4)}
    pw = power_window(torch, dev, lambda: launch(iters), fl, peak, seconds)
    if pw:
        res.update({k: pw[k] for k in ("avg_socket_power_w", "avg_gfxclk_mhz",
                                        "clock_adjusted_peak", "frac_of_clock_adjusted_peak")
                    if k in pw})
    del ops, out
    return res


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp16", action="store_true")
    ap.add_argument("--no-f16f32", action="store_true")
    ap.add_argument("--no-valu", action="store_true")
    ap.add_argument("--no-p4", action="store_true")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the power / energy windows")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the matrix-core ceiling probe")
    ap.add_argument("--power-seconds", type=float, default=3.0,
                    help="length of each measured power window")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--table", action="store_true",
                    help="one JSON row per workload (fp32 256^3; fp32 512..4096 powers of two; fp16 "
                         "4096^3; the ragged fp32 and fp16 workloads): GPU replay protocol next to "
                         "the CPU oracle on the whole product, plus the oracle on one thread at 256^3")
    ap.add_argument("--sweep", action="store_true",
                    help="fp32 size sweep M=N=K=1024..12800 step 128, beta=1, replay protocol "
                         "with cache flush; one JSON row per size")
    ap.add_argument("--sweep-sizes", default=None,
                    help="comma-separated sizes for --sweep (default 1024..12800 step 128)")
    ap.add_argument("--sweep-clock-seconds", type=float, default=0.25,
                    help="back-to-back load per sweep size before its clock is sampled")
    ap.add_argument("--sweep-oracle", action="store_true",
                    help="after --sweep, time the CPU oracle on the same sizes, ascending")
    ap.add_argument("--sweep-oracle-cap", type=float, default=600.0,
                    help="largest predicted oracle time of one sweep size, seconds")
    ap.add_argument("--sweep-oracle-total", type=float, default=300.0,
                    help="largest total time of the oracle sweep leg, seconds")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="write profiles/hbm_traffic.json from the rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE runs under DIR (no GPU needed)")
    ap.add_argument("--only", choices=["f32", "f16", "f16f32", "valu", "copy", "ragged_f32",
                                       "ragged_f16"], default=None,
                    help="run only one kernel (profiling runs); 'copy' runs a plain "
                         "device copy of known size to calibrate HBM counters")
    return ap.parse_args()


def main():
    args = parse_args()
    if args.traffic_from:
        write_traffic(args.traffic_from)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import dense_gemm_fp32_amd as dg
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only == "copy":
        run_copy_calibration(torch, dev)
        return
    if args.sweep:
        run_sweep(args, torch, dev, stream)
        return
    if args.table:
        run_table(torch, dev, stream)
        return

    def upload(w):
        A, B, C = wl.make(w)
        return tuple(torch.from_numpy(x).to(dev) for x in (A, B, C)), (A, B, C)

    def timed_steps(fn, w, dA, dB, dC, steps, warmup):
        for _ in range(warmup):
            rc = fn(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, stream)
            if rc != 0:
                raise RuntimeError("gemm returned %d: %s" % (rc, dg.gemm_status_string(rc)))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            fn(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, stream)
            b.record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        launch_ms = [a.elapsed_time(b) for a, b in ev]
        return wall, launch_ms

    def p4_protocol(fn, w, dA, dB, dC):
        n = round((w.M * w.N * w.K) ** (1.0 / 3.0))
        reps = replay_count(n)
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.int32, device=dev)
        times = []
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(reps):
            flush.zero_()
            s.record(stream)
            fn(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, stream)
            e.record(stream)
            e.synchronize()
            times.append(s.elapsed_time(e))
        del flush
        last = times[len(times) - len(times) // 2:]
        mean = sum(last) / len(last)
        return {"replays": reps, "averaged": len(last), "flush_bytes": 512 * 1024 * 1024,
                "mean_ms": round(mean, 5), "median_ms": round(sorted(last)[len(last) // 2], 5),
                "min_ms": round(min(times), 5), "tflops": round(w.flops / (mean * 1e-3) / 1e12, 2)}

    def measure(fn, w, peak, key, steps, warmup, p4, power=False):
        (dA, dB, dC), host = upload(w)
        # The replay protocol runs first: after the inputs are generated and
        # uploaded the GPU has idled for seconds, and its clock then takes
        # ~20 launches to come up (fp32 4096^3: 129 -> 147 TFLOP/s over the
        # first 20 calls, 148 from then on), so timed steps straight after the
        # upload would measure that ramp rather than the loaded clock.
        p4_res = p4_protocol(fn, w, dA, dB, dC) if p4 else None
        wall, launch_ms = timed_steps(fn, w, dA, dB, dC, steps, warmup)
        ms_per_step = wall * 1e3 / steps
        avg_launch = sum(launch_ms) / len(launch_ms)
        achieved = w.flops / (avg_launch * 1e-3) / 1e12
        traffic = load_traffic(key)
        res = {
            "value": round(w.flops / (ms_per_step * 1e-3) / 1e12, 2),
            "ms_per_step": round(ms_per_step, 5),
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                         "traffic": traffic,
                         "avg_launch_ms": round(avg_launch, 5),
                         "algorithmic_flops_per_launch": w.flops},
            "timed_window": launch_stats(launch_ms, w.flops),
        }
        if p4_res:
            res["p4_protocol"] = p4_res
        if power:
            res["power"] = power_window(
                torch, dev,
                lambda: fn(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, stream),
                w.flops, peak, args.power_seconds)
        del dA, dB, dC
        torch.cuda.empty_cache()
        return res, host

    # --only f32 / f16 measure their workload as the full run does (the replay
    # leg first, then the timed steps), without the power window, so that a
    # profiler's trace of the leg holds the same timed launches.
    if args.only == "f16":
        f16_res, _ = measure(dg.gemm_f16, wl.F16_4096, PEAK_F16, "f16", args.steps, args.warmup,
                             not args.no_p4)
        print(json.dumps({"only": "f16", **f16_res}), flush=True)
        return
    if args.only == "valu":
        res, _ = measure(dg.gemm_f32_valu, wl.F32_4096, PEAK_F32_VALU, "valu", args.steps,
                         args.warmup, False)
        res["roofline"]["bound"] = "alu"
        print(json.dumps({"only": "valu", **res}), flush=True)
        return
    if args.only == "f16f32":
        res, _ = measure(dg.gemm_f16f32, wl.F16F32_4096, PEAK_F16, "f16f32", args.steps,
                         args.warmup, False)
        print(json.dumps({"only": "f16f32", **res}), flush=True)
        return
    if args.only in ("ragged_f32", "ragged_f16"):
        # the unaligned 1000 x 3000 x 517 workload under the library's own plan
        # (fp32: A and B copied to 16-byte rows, then the four-wave 64x64 tile;
        # fp16: element-wise and pair loads, K split 2 ways); a call's time
        # includes its copy kernel or its reduction
        w = wl.RAGGED_F32 if args.only == "ragged_f32" else wl.RAGGED_F16
        fn = dg.gemm_f32 if args.only == "ragged_f32" else dg.gemm_f16
        res, _ = measure(fn, w, PEAK_F32 if args.only == "ragged_f32" else PEAK_F16, args.only,
                         args.steps, args.warmup, False)
        res["plan"] = dg.gemm_describe(w.dtype, w.M, w.N, w.K, w.alpha, 1 << 20, w.lda, 1 << 20,
                                       w.ldb, w.beta, 1 << 20, w.ldc)[1]
        if args.only == "ragged_f16":
            # 192 flop per compulsory byte against the machine's 314.6 for fp16:
            # the floor is HBM (16.1 MB at 8 TB/s, 2.0 us)
            nbytes = compulsory_bytes(w)
            avg_s = res["roofline"]["avg_launch_ms"] * 1e-3
            res["roofline"] = {"bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 1),
                               "peak": PEAK_HBM, "unit": "GB/s",
                               "frac": round(nbytes / avg_s / 1e9 / PEAK_HBM, 4),
                               "traffic": None, "avg_launch_ms": res["roofline"]["avg_launch_ms"],
                               "algorithmic_bytes_per_launch": nbytes,
                               "floor_us": round(nbytes / (PEAK_HBM * 1e9) * 1e6, 2)}
        else:
            # 96 flop per compulsory byte against 19.7 for fp32: the floor is
            # the matrix cores (3.102e9 flop at 157.3 TFLOP/s, 19.7 us)
            res["roofline"]["floor_us"] = round(w.flops / (PEAK_F32 * 1e12) * 1e6, 2)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return
    w32 = wl.F32_4096
    main_res, host32 = measure(dg.gemm_f32, w32, PEAK_F32, "f32", args.steps, args.warmup,
                               not args.no_p4 and args.only in (None, "f32"),
                               not args.no_power and args.only is None)
    if args.only == "f32":
        print(json.dumps({"only": "f32", **main_res}), flush=True)
        return

    f16_res = None
    if not args.no_fp16:
        w16 = wl.F16_4096
        f16_res, _ = measure(dg.gemm_f16, w16, PEAK_F16, "f16", args.steps, args.warmup,
                             not args.no_p4, not args.no_power)
        f16_res = {"workload": "fp16 in/out, fp32 accumulation, M=N=K=4096, A,B,C ~ U[-1,1], "
                               "alpha=1, beta=0.5", "unit": "TFLOP/s", **f16_res}

    mixed_res = None
    if not args.no_f16f32:
        mixed_res, _ = measure(dg.gemm_f16f32, wl.F16F32_4096, PEAK_F16, "f16f32", args.steps,
                               args.warmup, False)
        mixed_res = {"workload": "fp16 A and B, fp32 C and result, fp32 accumulation, "
                                 "M=N=K=4096, A,B,C ~ U[-1,1], alpha=1, beta=0.5",
                     "unit": "TFLOP/s", **mixed_res}

    valu_res = None
    if not args.no_valu:
        valu_res, _ = measure(dg.gemm_f32_valu, w32, PEAK_F32_VALU, "valu", args.steps,
                              args.warmup, False)
        valu_res["roofline"]["bound"] = "alu"
        valu_res = {"workload": "the fp32 4096^3 workload on gemm_f32_valu (vector ALUs, "
                                "128x128 tiles, 8x8 outputs per thread)", "unit": "TFLOP/s",
                    **valu_res,
                    "matrix_core_speedup": round(main_res["value"] / valu_res["value"], 2)}

    ceiling = None
    if not args.no_ceiling and not args.no_power:
        ceiling = {"f32": mfma_ceiling(torch, dev, stream, dg, wl, 0, PEAK_F32, args.power_seconds),
                   "f16": mfma_ceiling(torch, dev, stream, dg, wl, 1, PEAK_F16, args.power_seconds)}
        if ceiling["f32"]:
            main_res["roofline"]["frac_of_mfma_ceiling"] = round(
                main_res["roofline"]["achieved"] / ceiling["f32"]["tflops"], 4)
        if ceiling["f16"] and f16_res:
            f16_res["roofline"]["frac_of_mfma_ceiling"] = round(
                f16_res["roofline"]["achieved"] / ceiling["f16"]["tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w32, host32, args.cpu_seconds)

    props = torch.cuda.get_device_properties(dev)
    line = {
        "metric": "GEMM TFLOP/s (2MNK/t) fp32 at 4096^3; % of MI355X fp32 matrix peak",
        "value": main_res["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fp32 SGEMM row-major M=N=K=4096, lda=ldb=ldc=4096, "
                               "A,B ~ U[-1,1] (seeds 2,3), alpha=1, beta=0",
                   "M": w32.M, "N": w32.N, "K": w32.K},
        "pct_of_peak": round(100.0 * main_res["value"] / PEAK_F32, 2),
        "roofline": main_res["roofline"],
        "timed_window": main_res["timed_window"],
        "p4_protocol": main_res.get("p4_protocol"),
        "power": main_res.get("power"),
        "fp16": f16_res,
        "fp16_out_fp32": mixed_res,
        "valu_ablation": valu_res,
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "torch": torch.__version__,
                   "hip": torch.version.hip},
    }
    print(json.dumps(line), flush=True)


def compulsory_bytes(w):
    """Compulsory HBM bytes of a GEMM: A and B read once, C written (and read
    first when beta != 0)."""
    s_in = 4 if w.dtype == "f32" else 2
    s_out = 2 if w.dtype == "f16" else 4
    return s_in * (w.M * w.K + w.K * w.N) + s_out * w.M * w.N * (2 if w.beta != 0 else 1)


def run_sweep(args, torch, dev, stream):
    """The square fp32 sweep of the SGEMM summary's benchmarking section:
    M = N = K = n, A, B, C ~ U[-1, 1], alpha = beta = 1, floor(1000 *
    exp((1024 - n)/3100)) replays with a 512 MiB flush before each (outside
    the timed interval), mean of the second half.  Inputs of size n are the
    leading n x n blocks of seeded 12800 x 12800 matrices."""
    import dense_gemm_fp32_amd as dg
    import workloads as wl
    sizes = ([int(x) for x in args.sweep_sizes.split(",")] if args.sweep_sizes
             else wl.sweep_sizes())
    nmax = max(sizes)
    w = wl.sweep(nmax)
    big = [torch.from_numpy(wl.draw(nmax, nmax, "uniform", seed, "f32")).to(dev)
           for seed in w.seeds]
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.int32, device=dev)
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    smi, smi_h = smi_handle(torch, dev)
    for n in sizes:
        A, B, C = (x[:n, :n].contiguous() for x in big)
        reps = replay_count(n)
        rc = dg.gemm_f32(n, n, n, 1.0, A, n, B, n, 1.0, C, n, stream)   # warm-up
        if rc != 0:
            raise RuntimeError("gemm_f32 returned %d" % rc)
        times = []
        snap0 = smu_snapshot(smi, smi_h)
        for r in range(reps):
            flush.zero_()
            s_ev.record(stream)
            dg.gemm_f32(n, n, n, 1.0, A, n, B, n, 1.0, C, n, stream)
            e_ev.record(stream)
            e_ev.synchronize()
            times.append(s_ev.elapsed_time(e_ev))
        snap1 = smu_snapshot(smi, smi_h)
        last = times[len(times) - len(times) // 2:]
        mean = sum(last) / len(last)
        rc, plan = dg.gemm_describe("f32", n, n, n, 1.0, A, n, B, n, 1.0, C, n)
        # the clock this size holds under steady load: back-to-back calls for
        # a quarter of a second (no flushes), sampled at the end
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.sweep_clock_seconds:
            for _ in range(4):
                dg.gemm_f32(n, n, n, 1.0, A, n, B, n, 1.0, C, n, stream)
            torch.cuda.synchronize(dev)
        clk = clock_sample(smi, smi_h)
        print(json.dumps({"n": n, "replays": reps, "averaged": len(last),
                          "mean_ms": round(mean, 5), "min_ms": round(min(times), 5),
                          "tflops": round(2.0 * n ** 3 / (mean * 1e-3) / 1e12, 2),
                          "pct_of_peak": round(100 * 2.0 * n ** 3 / (mean * 1e-3) / 1e12 / PEAK_F32, 2),
                          "replay_loop": smu_between(snap0, snap1),
                          "steady_gfxclk_mhz": clk,
                          "plan": plan}), flush=True)
        del A, B, C
    if args.sweep_oracle:
        run_sweep_oracle(args, sizes)


def run_sweep_oracle(args, sizes):
    """The CPU oracle on the sweep's sizes, ascending, on the same leading
    n x n blocks of the seeded 12800 x 12800 inputs, all host cores: a size
    runs while its predicted time (the previous size's time x (n/n_prev)^3)
    stays under --sweep-oracle-cap seconds and the leg's total under
    --sweep-oracle-total seconds; the rows after that say why they did not
    run."""
    import numpy as np
    import oracle
    import workloads as wl
    nmax = max(sizes)
    w = wl.sweep(nmax)
    big = [wl.draw(nmax, nmax, "uniform", seed, "f32") for seed in w.seeds]
    threads = oracle.threads()
    total, prev = 0.0, None
    stop = None
    for n in sorted(sizes):
        if stop is None and prev is not None:
            pred = prev[1] * (n / prev[0]) ** 3
            if pred > args.sweep_oracle_cap:
                stop = "oracle did not finish within cap (predicted %.0f s > %.0f s)" % (
                    pred, args.sweep_oracle_cap)
            elif total + pred > args.sweep_oracle_total:
                stop = "not run: the leg's total budget of %.0f s" % args.sweep_oracle_total
        if stop is not None:
            print(json.dumps({"n": n, "oracle": stop}), flush=True)
            continue
        A, B, C = (np.ascontiguousarray(x[:n, :n]).reshape(-1) for x in big)
        t0 = time.perf_counter()
        oracle.gemm(n, n, n, 1.0, A, n, B, n, 1.0, C, n, "f32")
        sec = time.perf_counter() - t0
        total += sec
        prev = (n, sec)
        print(json.dumps({"n": n, "oracle_s": round(sec, 3),
                          "oracle_gflops": round(2.0 * n ** 3 / sec / 1e9, 2),
                          "oracle_threads": threads}), flush=True)


def run_table(torch, dev, stream):
    """Every workload of the pages' measurements on the GPU and on the CPU
    oracle, one JSON row each.  GPU: the SGEMM summary's replay protocol
    (floor(1000*exp((1024-n)/3100)) replays with n = round(cbrt(MNK)), a
    512 MiB flush before each outside the events, mean of the second half).
    Oracle: the whole product once, timed on all the host cores it uses.
    Last row: the oracle on one thread at 256^3 (a child process with
    OMP_NUM_THREADS=1)."""
    import subprocess
    import dense_gemm_fp32_amd as dg
    import oracle
    import workloads as wl
    fns = {"f32": dg.gemm_f32, "f16": dg.gemm_f16, "f16f32": dg.gemm_f16f32}
    peaks = {"f32": PEAK_F32, "f16": PEAK_F16, "f16f32": PEAK_F16}
    works = [wl.F32_256] + [wl.square(n) for n in (512, 1024, 2048, 4096)] + \
            [wl.F16_4096, wl.RAGGED_F32, wl.RAGGED_F16]
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.int32, device=dev)
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    threads = oracle.threads()
    for w in works:
        A, B, C = wl.make(w)
        dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C))
        fn = fns[w.dtype]
        n = round((w.M * w.N * w.K) ** (1.0 / 3.0))
        reps = replay_count(n)
        rc = fn(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, stream)
        if rc != 0:
            raise RuntimeError("%s returned %d" % (fn.__name__, rc))
        times = []
        for _ in range(reps):
            flush.zero_()
            s_ev.record(stream)
            fn(w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta, dC, w.ldc, stream)
            e_ev.record(stream)
            e_ev.synchronize()
            times.append(s_ev.elapsed_time(e_ev))
        last = times[len(times) - len(times) // 2:]
        mean = sum(last) / len(last)
        rc, plan = dg.gemm_describe(w.dtype, w.M, w.N, w.K, w.alpha, dA, w.lda, dB, w.ldb, w.beta,
                                    dC, w.ldc)
        del dA, dB, dC
        t0 = time.perf_counter()
        oracle.gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta,
                    C if w.beta != 0 else None, w.ldc, w.dtype)
        cpu_s = time.perf_counter() - t0
        print(json.dumps({
            "workload": w.name, "dtype": w.dtype, "M": w.M, "N": w.N, "K": w.K,
            "lda": w.lda, "ldb": w.ldb, "ldc": w.ldc, "alpha": w.alpha, "beta": w.beta,
            "replays": reps, "averaged": len(last), "gpu_mean_ms": round(mean, 5),
            "gpu_median_ms": round(sorted(last)[len(last) // 2], 5),
            "gpu_min_ms": round(min(times), 5),
            "gpu_tflops": round(w.flops / (mean * 1e-3) / 1e12, 3),
            "pct_of_peak": round(100.0 * w.flops / (mean * 1e-3) / 1e12 / peaks[w.dtype], 2),
            "oracle_s": round(cpu_s, 3), "oracle_gflops": round(w.flops / cpu_s / 1e9, 2),
            "oracle_threads": threads, "gpu_over_oracle": round(cpu_s * 1e3 / mean, 1),
            "plan": plan}), flush=True)
    code = ("import sys, time; sys.path.insert(0, %r); import oracle, workloads as wl; "
            "w = wl.F32_256; A, B, C = wl.make(w); t = time.perf_counter(); "
            "oracle.gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, None, w.ldc, 'f32'); "
            "print(time.perf_counter() - t, oracle.threads())" % ROOT)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         check=True).stdout.split()
    sec, nthr = float(out[0]), int(out[1])
    print(json.dumps({"workload": "f32_256 oracle on one thread", "oracle_s": round(sec, 4),
                      "oracle_gflops": round(wl.F32_256.flops / sec / 1e9, 3),
                      "oracle_threads": nthr}), flush=True)


TRAFFIC_KERNELS = {"f32": "sgemm_mfma", "f16": "hgemm_mfma", "copy": "copyBuffer"}


def pmc_average(csv_path, kernel_substr, counter):
    """Average per dispatch of `counter` over the dispatches of the kernel
    whose name contains `kernel_substr`, from a rocprofv3 counter CSV;
    returns (average, dispatches, full kernel name)."""
    import csv
    vals, name = {}, None
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
                name = r["Kernel_Name"]
    if not vals:
        raise ValueError("no %s samples of %s in %s" % (counter, kernel_substr, csv_path))
    return sum(vals.values()) / len(vals), len(vals), name


def write_traffic(src_dir):
    """profiles/hbm_traffic.json from the FETCH_SIZE and WRITE_SIZE runs in
    src_dir (subdirectories pmc_<k>_<COUNTER>/p_counter_collection.csv for
    k = f32, f16 and copy, one counter per run).  Both counters are scaled by
    what they read for the plain 1 GiB copy (1 GiB read, 1 GiB written)."""
    import glob

    def avg(k, counter):
        paths = glob.glob(os.path.join(src_dir, "pmc_%s_%s" % (k, counter), "*counter_collection.csv"))
        if not paths:
            raise FileNotFoundError("no %s run for %s under %s" % (counter, k, src_dir))
        return pmc_average(paths[0], TRAFFIC_KERNELS[k], counter)

    copy_bytes = 1 << 30
    cf, _, cname = avg("copy", "FETCH_SIZE")
    cw, _, _ = avg("copy", "WRITE_SIZE")
    ff, wf = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    import workloads as wl
    out = {"source_hash": kernel_source_hash(),
           "copy_calibration": {"kernel": cname, "bytes": copy_bytes, "fetch_kib": round(cf, 2),
                                "write_kib": round(cw, 2), "fetch_factor": round(ff, 4),
                                "write_factor": round(wf, 4)},
           "kernels": {}}
    for k, w in (("f32", wl.F32_4096), ("f16", wl.F16_4096)):
        fk, n, kname = avg(k, "FETCH_SIZE")
        wk, _, _ = avg(k, "WRITE_SIZE")
        out["kernels"][k] = {"kernel": kname, "fetch_kib": round(fk, 2), "write_kib": round(wk, 2),
                             "hbm_bytes_per_launch": int(round(fk * 1024 * ff + wk * 1024 * wf)),
                             "algorithmic_bytes": compulsory_bytes(w), "dispatches": n}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def run_copy_calibration(torch, dev):
    """A plain device-to-device copy of 1 GiB (read 1 GiB, write 1 GiB) for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1024 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(json.dumps({"only": "copy", "bytes_read": n * 4, "bytes_written": n * 4}), flush=True)


def cpu_baseline(w, host, target_s):
    """Oracle (as it stands) on a bounded sample of the workload: full output
    rows of the same product, timed on this host's cores."""
    import numpy as np
    import oracle
    import workloads as wl
    A, B, C = host
    Av = wl.view(A, w.M, w.K, w.lda)
    threads = oracle.threads()

    def run_rows(nrows):
        sub = np.ascontiguousarray(Av[:nrows]).reshape(-1)
        t0 = time.perf_counter()
        oracle.gemm(nrows, w.N, w.K, w.alpha, sub, w.K, B, w.ldb, w.beta, None, w.N, w.dtype)
        return time.perf_counter() - t0

    probe_rows = max(threads, 4)
    t = run_rows(probe_rows)
    rows = int(max(probe_rows, min(w.M, probe_rows * target_s / max(t, 1e-6))))
    rows = max(threads, rows - rows % threads) if rows >= threads else rows
    t = run_rows(rows)
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(t, 3),
            "sample": "%d of the %d output rows of the fp32 4096^3 GEMM (%d x %d x %d), "
                      "double-precision oracle with |A||B| bound terms" % (rows, w.M, rows, w.N, w.K)}


if __name__ == "__main__":
    main()
