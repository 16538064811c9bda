"""Benchmark of libsdpa's attention forward on one MI355X.

One step = one sdpa_forward call over the whole workload (one kernel launch),
inputs resident in HBM.  Prints ONE JSON line (see the keys below).

Default workload: the long-sequence causal self-attention, B=4, h=16,
Lq=Lk=8192, d_k=d_v=64, bf16, inputs N(0,1)*0.5 -- the configuration on which
the fraction of bf16 matrix-core peak is the figure of merit.  Other named
workloads (--config) are available for profiling; they are parity cases, not
headline lines.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                  [--no-cpu-baseline] [--rotate R] [--settle-ms MS] [--sustain-s S]
  python bench.py --copy-mib 512      (calibration: a plain device copy)
  python bench.py --gemm-probe 8192   (calibration: a bf16 GEMM through torch;
                                       also M,K,N, e.g. 32768,1024,3072)
  python bench.py --overlap-probe 20000   (calibration: matrix-core / VALU overlap)
  python bench.py --config NAME --timeline   (per-workgroup phases of one cold launch,
                                              from the timestamped build of the library)

After the W warmup steps, untimed steps continue until the GPU has been busy for
--settle-ms (default 150 ms), so that the K timed steps see the settled clock.

Besides the metric, the line carries: the roofline of the dominant kernel (with
the measured HBM traffic per launch and its ratio to the algorithmic bytes while
the counters match the kernel source), the oracle on the host cores beside it
(all cores and one thread, with the CPU model), the GPU output compared with
the oracle's values on the oracle's sample of rows ("parity"), the shader
clock sampled during the timed window, and ("sustained", --sustain-s, default
2 s) the rate of the same launches kept up for seconds, with the board power
beside the board's power limit.

FLOPs are algorithmic: (2*d_k + 2*d_v) per (query, key) pair the mask allows
(page "Attention Is All You Need/paper/es", §4, Table 1: O(n^2 d) per layer),
counted exactly from the drawn key lengths.  Bytes are algorithmic too: Q and
O once, each key/value row a query may use once.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from head_attention_fwd_amd import perfmodel  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak (h=8/16, d_k=64) on 1 MI355X"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense peaks (matrix bf16; fp32 vector)
PEAK_HBM_GBS = 8000.0
DEFAULT_CONFIG = "long_causal_bf16"
KERNEL_SOURCE_DIR = os.path.join(ROOT, "head_attention_fwd_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    """Hash of every source of the library (names and contents): a committed
    counter figure applies only while it matches."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCE_DIR)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(KERNEL_SOURCE_DIR, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(config_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(config_name)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def host_cpu():
    """CPU model of this host (from /proc/cpuinfo) and the cores this process may use."""
    model, fam, mod = "unknown", None, None
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model == "unknown":
                    model = v
                elif k == "cpu family" and fam is None:
                    fam = v
                elif k == "model" and mod is None:
                    mod = v
    except OSError:
        pass
    if fam is not None and mod is not None:
        model = "%s (family %s, model %s)" % (model, fam, mod)
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(x, target_seconds=15.0, one_thread_seconds=4.0):
    """The fp64 oracle, as it is, on a bounded random sample of the workload's rows.

    Rows (b, h, i) are drawn uniformly, so FLOPs/s on the sample estimate the
    oracle's throughput on the whole workload.  Runs on the host cores only; a
    second, smaller sample on one thread.  Returns the record and, for the
    parity check of the GPU output, the sampled rows and the oracle's values.
    """
    import oracle

    c = x.config
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    rng = np.random.default_rng(1234)

    def sample(n):
        return np.stack([rng.integers(0, c.B, n), rng.integers(0, c.H, n),
                         rng.integers(0, c.Lq, n)], axis=1)

    def row_flops(rows):
        tot = 0
        for b, h, i in rows:
            lb = c.Lk if x.key_lengths is None else perfmodel.clamp_length(x.key_lengths[b], c.Lk)
            hi = min(lb, i + 1) if c.causal else lb          # one past the last legal key
            lo = 0
            if c.radius is not None:
                hi = min(hi, i + c.radius + 1)
                lo = max(0, i - c.radius)
            tot += (2 * c.d_k + 2 * c.d_v) * max(hi - lo, 0)
        return tot

    oracle.default()   # build/load outside the timed region
    # fp64 copies made once, outside the timed region (the oracle's input type)
    q64, k64, v64 = (np.ascontiguousarray(a, dtype=np.float64) for a in (x.q, x.k, x.v))

    def timed(rows, nthreads):
        t0 = time.perf_counter()
        out, _ = oracle.attention_rows(q64, k64, v64, rows, key_lengths=x.key_lengths,
                                       causal=c.causal, nthreads=nthreads, radius=c.radius)
        return time.perf_counter() - t0, out

    def sized(nthreads, seconds):
        # calibrate on growing samples (small ones are dominated by fixed costs),
        # then size the measured sample for about `seconds` of oracle work
        n = max(nthreads * 4, 64)
        for budget in (0.5, 2.0, seconds):
            rows = sample(n)
            dt, out = timed(rows, nthreads)
            if budget == seconds:
                break
            nxt = min(2.0, seconds) if budget == 0.5 else seconds
            n = int(n * max(1.0, nxt / max(dt, 1e-3)))
            n = max(64, min(n, c.B * c.H * c.Lq))
        return rows, dt, out

    rows, dt, out = sized(threads, target_seconds)
    f = row_flops(rows)
    rows1, dt1, _ = sized(1, one_thread_seconds)
    f1 = row_flops(rows1)
    del q64, k64, v64
    model, _ = host_cpu()
    total = perfmodel.flops(c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, c.causal, x.key_lengths,
                            radius=c.radius)
    rec = {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "%d uniformly drawn query rows (%.3g of the workload's FLOPs, %.1f s), "
                     "fp64 C oracle with OpenMP" % (len(rows), f / total, dt),
           "cpu_model": model,
           "value_1thread": f1 / dt1 / 1e12,
           "sample_1thread": "%d other uniformly drawn query rows (%.1f s) on one thread"
                             % (len(rows1), dt1)}
    return rec, rows, out


def cpu_baseline_multihead(x, target_seconds=15.0):
    """The fp64 oracle's MultiHead, as it is, on the first B' batch entries of the
    workload (B' sized for about target_seconds), FLOPs counted like the GPU's.
    Returns the record, B' and the oracle's output for those entries."""
    import oracle

    c = x.config
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    oracle.default()

    def run(nb, nthreads=threads):
        kl = None if x.key_lengths is None else x.key_lengths[:nb]
        args = [np.ascontiguousarray(a[:nb], dtype=np.float64) for a in (x.xq, x.xkv)]
        t0 = time.perf_counter()
        out = oracle.multihead(args[0], args[1], x.wq, x.wk, x.wv, x.wo, c.H, key_lengths=kl,
                               causal=c.causal, nthreads=nthreads)
        return time.perf_counter() - t0, perfmodel.multihead_flops(
            nb, c.Lq, c.Lk, c.d_model, c.H, c.d_k, c.d_v, c.causal, kl), out

    dt, f, out = run(1)
    nb = int(max(1, min(c.B, round(target_seconds / max(dt, 1e-3)))))
    if nb > 1:
        dt, f, out = run(nb)
    total = perfmodel.multihead_flops(c.B, c.Lq, c.Lk, c.d_model, c.H, c.d_k, c.d_v, c.causal,
                                      x.key_lengths)
    model, _ = host_cpu()
    rec = {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "the first %d of %d batch entries (%.3g of the workload's FLOPs, %.1f s), "
                     "fp64 C oracle with OpenMP" % (nb, c.B, f / total, dt),
           "cpu_model": model, "value_1thread": None,
           "sample_1thread": "not measured: one batch entry's projections and attention "
                             "take minutes on one thread"}
    return rec, nb, out


def parity_record(got, ref, v_absmax, dtype, what):
    """The GPU output against the oracle's values on the same inputs, with the bars
    of the parity tests (fp32: max |d| <= 1e-5; bf16: max |d| <= 2e-2 max|V|, mean
    |d| <= 2e-3)."""
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    max_abs, mean_abs = float(err.max()), float(err.mean())
    if dtype == "f32":
        bar = {"max_abs": 1e-5}
        ok = max_abs <= 1e-5
    else:
        bar = {"max_abs": 2e-2 * v_absmax, "mean_abs": 2e-3}
        ok = max_abs <= bar["max_abs"] and mean_abs <= bar["mean_abs"]
    return {"max_abs": max_abs, "mean_abs": mean_abs, "rows": what, "bar": bar, "ok": bool(ok),
            "max_rel_to_max_out": max_abs / max(float(np.abs(ref).max()), 1e-30)}


class ClockSampler:
    """Samples, from a host thread while the GPU works, the shader clock the
    driver reports (sysfs pp_dpm_sclk, the line marked current) and the board
    power with its limit (hwmon power1_input / power1_cap, microwatts; the
    driver's reading is a running average that takes ~0.4 s to follow a change
    of load)."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.hwmon = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*"))[:1]
        self.period = period_s
        self.samples = []
        self.power = []          # (seconds since start, watts)
        self.cap_w = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for p in self.paths:
            try:
                with open(p, encoding="ascii") as f:
                    for line in f:
                        if line.rstrip().endswith("*"):
                            return float(line.split(":")[1].strip().split("M")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _read_hwmon(self, name):
        for d in self.hwmon:
            try:
                with open(os.path.join(d, name), encoding="ascii") as f:
                    return int(f.read().strip()) * 1e-6
            except (OSError, ValueError):
                continue
        return None

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            w = self._read_hwmon("power1_input")
            if w is not None:
                self.power.append((time.perf_counter() - t0, w))
            time.sleep(self.period)

    def __enter__(self):
        if self.paths or self.hwmon:
            self.cap_w = self._read_hwmon("power1_cap")
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "n": len(v),
                "source": "sysfs pp_dpm_sclk (current level), sampled every 2 ms during the "
                          "timed window"}

    def power_summary(self, after_s=0.0):
        """Board power over the samples taken at least after_s into the window."""
        w = sorted(p for t, p in self.power if t >= after_s)
        if not w:
            return None
        return {"median_w": w[len(w) // 2], "min_w": w[0], "max_w": w[-1], "n": len(w),
                "cap_w": self.cap_w, "from_s": after_s,
                "source": "hwmon power1_input / power1_cap (driver's running average)"}


def sustained(torch, stream, launch, flops_per_launch, seconds, batch=20):
    """Keep the GPU on one workload for `seconds`: batches of `batch` launches, each
    batch bracketed by events on the launch stream, the board power and clock
    sampled beside them.  Reports the rate over the second half of the window,
    once the power reading has followed the load, with the power and clock of
    the same half.  Not part of `value`: it shows where the sustained rate sits
    against the board's power limit."""
    batches = []
    with ClockSampler(period_s=0.005) as smp:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(batch):
                launch()
            e1.record(stream)
            e1.synchronize()
            batches.append((time.perf_counter() - t0, e0, e1))
    half = seconds / 2
    late = [(e0, e1) for t, e0, e1 in batches if t >= half] or [(e0, e1) for _, e0, e1 in batches]
    ms = sum(e0.elapsed_time(e1) for e0, e1 in late) / (batch * len(late))
    clk = sorted(smp.samples[len(smp.samples) // 2:])
    return {"seconds": seconds, "launches_averaged": batch * len(late), "ms_per_launch": ms,
            "tflops": flops_per_launch / (ms * 1e-3) / 1e12 if flops_per_launch else None,
            "power": smp.power_summary(after_s=half),
            "clock_median_mhz": clk[len(clk) // 2] if clk else None,
            "window": "second half of %.1f s of back-to-back launches" % seconds}


TIMELINE_FILES = ("fwd", "wide", "row")   # instrumented sources (readers sdpa_timeline_<name>)
TIMELINE_WORKGROUPS, TIMELINE_EVENTS = 1 << 16, 4


def timeline_capture(torch, lib, step, rotate, reps=3):
    """Per-workgroup phases of single cold launches from libsdpa_timeline.so:
    every workgroup's lane 0 of wave 0 stamps the device's 100 MHz real-time
    counter at entry, when its first key tile is in, after its last tile and
    after issuing its stores (csrc/sdpa_timeline.h).  Before each captured
    launch every input set is run once, so the captured one (set 0) is the
    least recently used.  Returns one record per repetition and instrumented
    kernel file that ran."""
    import ctypes
    readers = {}
    for name in TIMELINE_FILES:
        fn = getattr(lib, "sdpa_timeline_" + name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        readers[name] = fn
    out = []
    buf = np.zeros(TIMELINE_WORKGROUPS * TIMELINE_EVENTS, dtype=np.uint64)
    for rep in range(reps):
        for n in range(rotate):
            step(n)
        torch.cuda.synchronize()
        for fn in readers.values():
            assert fn(None, 0, 1) == 0, "clearing the timeline records failed"
        step(0)
        torch.cuda.synchronize()
        for name, fn in readers.items():
            assert fn(buf.ctypes.data, buf.nbytes, 0) == 0, "reading the timeline records failed"
            t = buf.reshape(TIMELINE_WORKGROUPS, TIMELINE_EVENTS).astype(np.int64)
            t = t[t[:, 0] > 0]
            if len(t) == 0:
                continue
            t0 = t[:, 0].min()
            us = lambda a: a / 100.0                       # 100 MHz counter
            def pct(a, q):
                return float(np.percentile(a, q)) if len(a) else None
            ok1, ok2, ok3 = t[:, 1] > 0, (t[:, 1] > 0) & (t[:, 2] > 0), (t[:, 2] > 0) & (t[:, 3] > 0)
            start = us(t[:, 0] - t0)
            first = us(t[ok1, 1] - t[ok1, 0])
            loop = us(t[ok2, 2] - t[ok2, 1])
            epi = us(t[ok3, 3] - t[ok3, 2])
            end = us(t[t[:, 3] > 0, 3] - t0)
            out.append({"rep": rep, "file": name, "workgroups": int(len(t)),
                        "start_us": {"p50": pct(start, 50), "max": float(start.max())},
                        "first_tile_wait_us": {"p50": pct(first, 50), "p90": pct(first, 90)},
                        "tile_loop_us": {"p50": pct(loop, 50), "p90": pct(loop, 90)},
                        "epilogue_us": {"p50": pct(epi, 50), "p90": pct(epi, 90)},
                        "end_us": {"p50": pct(end, 50), "max": float(end.max()) if len(end) else None}})
    return out


def copy_calibration(torch, dev, args):
    """A plain copy of known size: reads and writes args.copy_mib MiB per launch."""
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": ms,
                      "GB_per_s_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def gemm_probe(torch, dev, args):
    """Calibration, not the product: a bf16 GEMM through torch (hipBLASLt), N x N x N
    or M x K x N ("M,K,N"), to show what a dense matrix-core kernel reaches on
    this GPU (its rate, and under rocprofv3 counters its clock and matrix-core
    busy share), e.g. on the shapes of the multi-head projections."""
    dims = [int(x) for x in str(args.gemm_probe).split(",")]
    m, k, n = dims * 3 if len(dims) == 1 else dims
    a = torch.randn(m, k, device=dev, dtype=torch.bfloat16)
    b = torch.randn(k, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(m, n, device=dev, dtype=torch.bfloat16)
    for _ in range(args.warmup):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t_busy = time.perf_counter()
    while (time.perf_counter() - t_busy) * 1e3 < args.settle_ms:
        for _ in range(5):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clk:
        t0.record()
        for _ in range(args.steps):
            torch.matmul(a, b, out=c)
        t1.record()
        torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    flop = 2.0 * m * k * n
    sust = None
    if args.sustain_s > 0:
        sust = sustained(torch, torch.cuda.current_stream(dev), lambda: torch.matmul(a, b, out=c),
                         flop, args.sustain_s, batch=5)
        sust["frac_of_peak"] = sust["tflops"] / PEAK_TFLOPS["bf16"]
    print(json.dumps({"probe": "bf16 GEMM C = A B through torch.matmul (hipBLASLt), calibration only",
                      "M": m, "K": k, "N": n, "ms_per_gemm": ms, "tflops": flop / (ms * 1e-3) / 1e12,
                      "frac_of_peak": flop / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                      "clock": clk.summary(), "sustained": sust}), flush=True)


def overlap_probe(torch, dev, args):
    """Calibration, not the product: how far a matrix-core stream and a vector-ALU
    stream from different waves on one SIMD run at the same time (kernels in
    libsdpa_calib.so): times of the matrix stream alone, the vector stream alone
    and both together, with the accumulators in VGPRs or accumulation registers."""
    import ctypes
    from head_attention_fwd_amd import build as hb
    if not os.path.exists(hb.CALIB_LIBRARY):
        raise RuntimeError("libsdpa_calib.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(hb.CALIB_LIBRARY)
    lib.sdpa_calib_overlap.restype = ctypes.c_int
    lib.sdpa_calib_overlap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    n_wg = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(n_wg * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    iters = args.overlap_probe

    def timed(mode, which):
        def go():
            rc = lib.sdpa_calib_overlap(mode, which, out.data_ptr(), n_wg, iters, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("sdpa_calib_overlap: hipError %d" % rc)
        for _ in range(3):
            go()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        with ClockSampler() as clk:
            t0.record(stream)
            for _ in range(40):
                go()
            t1.record(stream)
            torch.cuda.synchronize()
        return {"ms": t0.elapsed_time(t1) / 40, "clock": clk.summary()}

    # settle the clock first (both streams, untimed)
    t_busy = time.perf_counter()
    while (time.perf_counter() - t_busy) * 1e3 < max(args.settle_ms, 300.0):
        if lib.sdpa_calib_overlap(0, 2, out.data_ptr(), n_wg, iters, stream.cuda_stream) != 0:
            raise RuntimeError("sdpa_calib_overlap failed")
        torch.cuda.synchronize()
    res = {}
    if args.sustain_s > 0:
        def launcher(which):
            def go():
                if lib.sdpa_calib_overlap(0, which, out.data_ptr(), n_wg, iters, stream.cuda_stream) != 0:
                    raise RuntimeError("sdpa_calib_overlap failed")
            return go
        res["sustained_vgpr_accumulators"] = {
            k: sustained(torch, stream, launcher(w), None, args.sustain_s, batch=5)
            for k, w in (("matrix_only", 0), ("vector_only", 1), ("both", 2))}
    for mode, name in ((0, "vgpr_accumulators"), (1, "accumulation_registers")):
        r = {k: timed(mode, w) for k, w in (("matrix_only", 0), ("vector_only", 1), ("both", 2))}
        r["both_over_sum"] = r["both"]["ms"] / (r["matrix_only"]["ms"] + r["vector_only"]["ms"])
        res[name] = r
    print(json.dumps({"probe": "matrix-core / vector-ALU overlap on one SIMD, calibration only",
                      "workgroups": n_wg, "waves": "4 matrix + 4 vector per CU",
                      "per_iteration": "4 v_mfma_f32_32x32x16_bf16 / 32 v_fma_f32",
                      "iterations": iters, **res}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="after the warmup steps, keep launching untimed steps until the "
                         "GPU has been busy this long (its clock settles within ~50 ms)")
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(workloads.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB "
                         "(calibrates the HBM byte counters of rocprofv3)")
    ap.add_argument("--gemm-probe", default="",
                    help="instead of attention, time a bf16 GEMM through torch, N (N x N x N) "
                         "or M,K,N (calibration: what a dense matrix-core kernel reaches on "
                         "this GPU)")
    ap.add_argument("--overlap-probe", type=int, default=0,
                    help="instead of attention, run the matrix-core / vector-ALU overlap probe "
                         "with this many iterations (calibration; libsdpa_calib.so)")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="time the K steps as one replay of a captured HIP graph (no host "
                         "launch cost between steps); auto: on for the decode workloads, whose "
                         "steps are two short launches")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup phases of single cold launches (timestamped build "
                         "libsdpa_timeline.so) instead of the timed steps")
    ap.add_argument("--sustain-s", type=float, default=2.0,
                    help="after the timed steps, keep launching for this long and report the "
                         "sustained rate with the board power and its limit (0: skip)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through (0: enough for >= 1 GiB on HBM-bound "
                         "workloads, 1 otherwise)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this attention forward has no multi-GPU "
              "path (every (batch, head) is independent; sharding them needs no "
              "communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_attention_fwd_amd as sdpa
    if args.timeline:
        # the timestamped build of the same sources, loaded in place of libsdpa.so
        from head_attention_fwd_amd import _binding
        _binding.load_library(os.path.join(ROOT, "head_attention_fwd_amd", "libsdpa_timeline.so"))

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    if args.copy_mib:
        copy_calibration(torch, dev, args)
        return
    if args.gemm_probe:
        gemm_probe(torch, dev, args)
        return
    if args.overlap_probe:
        overlap_probe(torch, dev, args)
        return
    x = workloads.generate(args.config)
    c = x.config
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    if c.entry == "multihead":
        flops = perfmodel.multihead_flops(c.B, c.Lq, c.Lk, c.d_model, c.H, c.d_k, c.d_v, c.causal,
                                          x.key_lengths)
        nbytes = perfmodel.multihead_min_bytes(c.B, c.Lq, c.Lk, c.d_model, c.H, c.d_k, c.d_v,
                                               c.self_attention)
    else:
        flops = perfmodel.flops(c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, c.causal, x.key_lengths,
                                radius=c.radius)
        nbytes = perfmodel.min_bytes(c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, c.causal, x.key_lengths,
                                     elem=2 if c.dtype == "bf16" else 4, radius=c.radius)
    # Arithmetic of the path: the matrix cores (bf16 products, fp32 sums) for
    # bf16 with d_k = d_v in {16, 32, 64, 128} (restricted or not) or in
    # {256, 512} (unrestricted), and the decode and multi-head entry points;
    # fp32 on the vector units otherwise.
    wide_mfma = (c.dtype == "bf16" and c.d_k == c.d_v and c.d_k in (256, 512)
                 and c.entry != "restricted")
    mfma_path = c.entry in ("decode", "multihead") or wide_mfma or (
        c.dtype == "bf16" and c.d_k == c.d_v and c.d_k in (16, 32, 64, 128))
    arith = "bf16" if mfma_path else "f32"
    hbm_bound = flops / nbytes < (PEAK_TFLOPS[arith] * 1e12) / (PEAK_HBM_GBS * 1e9)

    rotate = args.rotate
    if rotate <= 0:
        # HBM-bound workloads cycle through copies totalling >= 1 GiB so that the
        # 256 MB Infinity Cache cannot hold the inputs between launches.
        rotate = min(64, max(1, -(-(1 << 30) // nbytes))) if (hbm_bound and nbytes >= (1 << 20)) else 1
    if c.entry == "multihead":
        rotate = 1          # one weight set and one input set (a matrix-core-bound step)

    def up(a):
        return torch.from_numpy(a).to(tdt).to(dev)

    kl = None if x.key_lengths is None else torch.as_tensor(x.key_lengths).to(dev)
    sets = []
    if c.entry == "multihead":
        xq_d = up(x.xq)
        mh = (xq_d, xq_d if c.self_attention else up(x.xkv), up(x.wq), up(x.wk), up(x.wv),
              up(x.wo))
        sets.append((mh, torch.empty((c.B, c.Lq, c.d_model), dtype=tdt, device=dev)))
    else:
        base = (up(x.q), up(x.k), up(x.v))
        for r in range(rotate):
            qkv = base if r == 0 else tuple(t.clone() for t in base)
            sets.append((qkv, torch.empty((c.B, c.H, c.Lq, c.d_v), dtype=tdt, device=dev)))

    # Validate the binding once, then time pre-marshalled C-ABI calls so that the
    # host cost per step stays far below the kernel time.
    stream = torch.cuda.current_stream(dev)
    lib = sdpa.load_library()
    dcode = sdpa.SDPA_BF16 if c.dtype == "bf16" else sdpa.SDPA_F32
    klp = None if kl is None else kl.data_ptr()
    if c.entry == "multihead":
        (xq_d, xkv_d, wq_d, wk_d, wv_d, wo_d), o0 = sets[0]
        ws_bytes = sdpa.sdpa_multihead_workspace_bytes(c.B, c.Lq, c.Lk, c.d_model, c.H, c.d_k,
                                                       c.d_v, dcode)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        sdpa.multihead(xq_d, xkv_d, wq_d, wk_d, wv_d, wo_d, c.H, key_lengths=kl, causal=c.causal,
                       out=o0, workspace=ws)
        calls = [(xq_d.data_ptr(), xkv_d.data_ptr(), wq_d.data_ptr(), wk_d.data_ptr(),
                  wv_d.data_ptr(), wo_d.data_ptr(), klp, int(c.causal), o0.data_ptr(), c.B, c.Lq,
                  c.Lk, c.d_model, c.H, c.d_k, c.d_v, dcode, ws.data_ptr(), ws_bytes,
                  stream.cuda_stream)]
        fn, fn_name = lib.sdpa_multihead_forward, "sdpa_multihead_forward"
    elif c.entry == "decode":
        (q0, k0, v0), o0 = sets[0]
        ws_bytes = sdpa.sdpa_decode_workspace_bytes(c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, dcode)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        sdpa.decode(q0, k0, v0, key_lengths=kl, out=o0, workspace=ws)
        calls = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), klp, o.data_ptr(), c.B, c.H, c.Lq,
                  c.Lk, c.d_k, c.d_v, dcode, ws.data_ptr(), ws_bytes, stream.cuda_stream)
                 for (q, k, v), o in sets]
        fn, fn_name = lib.sdpa_decode, "sdpa_decode"
    elif c.entry == "restricted":
        (q0, k0, v0), o0 = sets[0]
        sdpa.restricted(q0, k0, v0, c.radius, key_lengths=kl, causal=c.causal, out=o0)
        calls = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), klp, int(c.causal), c.radius,
                  o.data_ptr(), c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, dcode, stream.cuda_stream)
                 for (q, k, v), o in sets]
        fn, fn_name = lib.sdpa_forward_restricted, "sdpa_forward_restricted"
    else:
        (q0, k0, v0), o0 = sets[0]
        sdpa.forward(q0, k0, v0, key_lengths=kl, causal=c.causal, out=o0)
        calls = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), klp, int(c.causal), o.data_ptr(),
                  c.B, c.H, c.Lq, c.Lk, c.d_k, c.d_v, dcode, stream.cuda_stream)
                 for (q, k, v), o in sets]
        fn, fn_name = lib.sdpa_forward, "sdpa_forward"

    def step(n):
        st = fn(*calls[n % rotate])
        if st != 0:
            raise RuntimeError("%s: %s" % (fn_name, sdpa.sdpa_status_str(st)))

    for n in range(args.warmup):
        step(n)
    torch.cuda.synchronize()
    # MI355X raises its clock over the first tens of milliseconds of sustained
    # work; launches in that window run up to ~30% slower.  Keep the GPU busy
    # (untimed) until it has run for settle_ms, in batches of launches.
    settle_steps = 0
    t_busy = time.perf_counter()
    while (time.perf_counter() - t_busy) * 1e3 < args.settle_ms:
        for _ in range(10):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()

    if args.timeline:
        recs = timeline_capture(torch, lib, step, rotate)
        cols = ("workgroups", "start (p50 / max)", "first tile in (p50 / p90)",
                "tile loop (p50 / p90)", "epilogue (p50 / p90)", "end (p50 / max)")
        print("| launch | kernel file | " + " | ".join(cols) + " |")
        print("|---|---|" + "---|" * len(cols))
        f2 = lambda d, a, b: "%.2f / %.2f" % (d[a], d[b]) if d[a] is not None else "-"
        for r in recs:
            print("| %d | %s | %d | %s | %s | %s | %s | %s |" % (
                r["rep"], r["file"], r["workgroups"], f2(r["start_us"], "p50", "max"),
                f2(r["first_tile_wait_us"], "p50", "p90"), f2(r["tile_loop_us"], "p50", "p90"),
                f2(r["epilogue_us"], "p50", "p90"), f2(r["end_us"], "p50", "max")))
        print(json.dumps({"timeline": recs, "config": c.name, "entry": fn_name,
                          "input_sets": rotate, "unit": "us",
                          "clock": "s_memrealtime, 100 MHz, one device-wide counter"}), flush=True)
        return

    use_graph = args.graph == "on" or (args.graph == "auto" and c.entry in ("decode", "multihead"))
    clk = None
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if use_graph:
        # The same K calls captured on a side stream (default priority) and
        # replayed as one graph.  The library's kernels take the stream handle
        # they are given; the calls are re-marshalled with the capture stream.
        gs = torch.cuda.Stream(device=dev)
        gs.wait_stream(stream)
        gcalls = [cl[:-1] + (gs.cuda_stream,) for cl in calls]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            for n in range(args.steps):
                st = fn(*gcalls[n % rotate])
                if st != 0:
                    raise RuntimeError("%s: %s" % (fn_name, sdpa.sdpa_status_str(st)))
        # replays must reproduce the eager result bit for bit (deterministic kernels)
        for n in range(rotate):
            step(n)
        torch.cuda.synchronize()
        eager = [o.clone() for _, o in sets]
        for o in (o for _, o in sets):
            o.zero_()
        for _ in range(2):
            with torch.cuda.stream(gs):     # replay() launches on the current stream
                graph.replay()
            torch.cuda.synchronize()
            for (_, o), e in zip(sets, eager):
                if not torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                                   e.view(torch.int16) if e.dtype == torch.bfloat16 else e):
                    raise RuntimeError("graph replay differs from the eager result")
        torch.cuda.synchronize()        # barrier (one rank) + synchronize
        with ClockSampler() as clk:
            t0 = time.perf_counter()
            with torch.cuda.stream(gs):
                start.record(gs)
                graph.replay()
                end.record(gs)
            torch.cuda.synchronize()
    else:
        torch.cuda.synchronize()        # barrier (one rank) + synchronize
        with ClockSampler() as clk:
            t0 = time.perf_counter()
            start.record(stream)
            for n in range(args.steps):
                step(n)
            end.record(stream)
            torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps

    # Distribution of single launches (after the timed window; not part of
    # `value`): each step bracketed by its own pair of events on the launch
    # stream.  And, for workloads timed on rotated input sets (cold caches),
    # the same launches repeated on one set: the warm-cache figure.
    def per_launch(n_launch, fixed_set):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_launch)]
        for n, (e0, e1) in enumerate(evs):
            e0.record(stream)
            step(0 if fixed_set else n)
            e1.record(stream)
        torch.cuda.synchronize()
        return sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)

    def summary(us):
        return {"median": us[len(us) // 2], "p10": us[len(us) // 10], "p90": us[(9 * len(us)) // 10],
                "n": len(us)}

    n_dist = min(args.steps, 200)
    launch_us = summary(per_launch(n_dist, False))
    warm = None
    if rotate > 1:
        wus = per_launch(n_dist, True)
        warm = {"launch_us": summary(wus), "value": flops / (wus[len(wus) // 2] * 1e-6) / 1e12,
                "unit": "TFLOP/s", "note": "one input set reused: inputs warm in the 256 MB cache"}
    # One kernel launch per step (decode: the split kernel and its merge),
    # launched back to back on this stream: the average launch duration is the
    # event window over the launch count.
    kern_ms = ms_per_step

    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved_tflops = flops / (kern_ms * 1e-3) / 1e12
    achieved_gbs = nbytes / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.config)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved_gbs / PEAK_HBM_GBS, "traffic": traffic}
    else:
        roof = {"bound": "mfma" if mfma_path else "alu", "achieved": achieved_tflops,
                "peak": PEAK_TFLOPS[arith], "unit": "TFLOP/s",
                "frac": achieved_tflops / PEAK_TFLOPS[arith], "traffic": traffic}
    if c.entry == "decode":
        roof["kernel"] = ("sdpa_decode_row_kernel (+ sdpa_split_merge_kernel when a head's keys span "
                          "several chunks)" if c.Lq == 1 else
                          "sdpa_decode_wg_kernel, or sdpa_split_mfma_kernel + sdpa_split_merge_kernel")
    elif c.entry == "multihead":
        roof["kernel"] = ("whole step: projection GEMMs (proj_gemm_kernel) + attention "
                          "(sdpa_fwd_mfma_kernel); per-kernel split in the rocprofv3 summary")
    elif c.entry == "restricted":
        roof["kernel"] = ("sdpa_fwd_mfma_band_kernel" if mfma_path else
                          "sdpa_fwd_wide_kernel" if max(c.d_k, c.d_v) > 8 else "sdpa_fwd_generic_kernel")
    elif wide_mfma:
        roof["kernel"] = "sdpa_fwd_mfma_wide_kernel"
    else:
        roof["kernel"] = ("sdpa_fwd_mfma_kernel" if mfma_path else
                          "sdpa_fwd_wide_kernel" if max(c.d_k, c.d_v) > 8 else "sdpa_fwd_generic_kernel")
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = nbytes
    roof["traffic_ratio"] = None if traffic is None else traffic / nbytes
    roof["kernel_ms"] = kern_ms

    sust = None
    if args.sustain_s > 0:
        if use_graph:
            def launch():
                with torch.cuda.stream(gs):
                    graph.replay()
            sust = sustained(torch, gs, launch, flops * args.steps, args.sustain_s, batch=1)
            sust["launch"] = "one replay of the %d-step graph" % args.steps
        else:
            ctr = [0]

            def launch():
                step(ctr[0])
                ctr[0] += 1
            sust = sustained(torch, stream, launch, flops, args.sustain_s)

    # The output of input set 0 (written by the timed steps) against the oracle's
    # values on the rows the CPU baseline computes: the line checks itself.
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        o_host = sets[0][1].float().cpu().numpy()
        if c.entry == "multihead":
            cpu, nb, ref = cpu_baseline_multihead(x)
            parity = parity_record(o_host[:nb], ref, float(np.abs(ref).max()), c.dtype,
                                   "the first %d of %d batch entries" % (nb, c.B))
        else:
            cpu, rows, ref = cpu_baseline(x)
            got = o_host[rows[:, 0], rows[:, 1], rows[:, 2]]
            parity = parity_record(got, ref, float(np.abs(x.v).max()), c.dtype,
                                   "%d uniformly drawn query rows (the CPU baseline's sample)"
                                   % len(rows))

    rec = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settle_steps,
        "timing": "hip graph of the timed steps" if use_graph else "back-to-back launches",
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": arith, "data": "synthetic",
        "config": {"workload": c.name, "description": c.description, "entry": fn_name,
                   "B": c.B, "h": c.H,
                   "Lq": c.Lq, "Lk": c.Lk, "d_k": c.d_k, "d_v": c.d_v, "causal": c.causal,
                   "key_lengths": None if x.key_lengths is None else "U{%d..%d} seed %d" % (
                       c.key_len_range[0], c.key_len_range[1], c.seed),
                   "radius": c.radius, "d_model": c.d_model,
                   "self_attention": c.self_attention if c.entry == "multihead" else None,
                   "input_sets": rotate},
        "frac_of_peak": value / PEAK_TFLOPS[arith],
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "clock": None if clk is None else clk.summary(),
        "launch_us": launch_us,
        "warm": warm,
        "sustained": sust,
        "wall_s_timed": wall,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
