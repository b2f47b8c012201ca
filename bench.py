"""Throughput bench of the attention forward pass on one MI355X.

One step is one fa_fwd launch (the whole forward pass) over the resident
inputs of the headline workload: causal bf16 attention, B=2, H=32, N=4096,
d=128 (seeded synthetic data).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config c3] [--no-cpu-baseline]
  python bench.py --splitkv S [--config s1]   (split-KV path against the direct one)
  python bench.py --backward [--config c3]     (backward pass, fa_bwd)

FLOPs per launch are the nominal 4*B*H*N^2*d, halved for causal.  The roofline
entry compares the average launch duration (HIP events around every launch on
the launch stream, inside the timed region) with the bf16 dense MFMA peak.
The cpu_baseline entry times the fp64 oracle on a bounded sample of whole
heads of the same workload on the host cores.

Profiling helpers (for rocprofv3 runs of this same script):
  --calibrate-copy       also launch a plain elementwise copy of known size
                         (for scaling FETCH_SIZE / WRITE_SIZE counters)
  --summarize DIR        print per-kernel figures from rocprofv3 output in DIR
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, causal, N=4096 d=128) + % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
KERNEL_SRC = os.path.join(ROOT, "io_aware_tiled_04_amd", "csrc", "fa_fwd_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_c3_trace_and_counters.md")
COPY_BYTES = 512 << 20


def kernel_sha(text=None) -> str:
    """Hash of the kernel source's code: comments and whitespace are left out,
    so that a change of wording does not count as a change of the kernel."""
    import re
    if text is None:
        with open(KERNEL_SRC, encoding="utf-8") as f:
            text = f.read()
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.strip().startswith("- "):
            key, _, val = line.strip()[2:].partition(":")
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256_16") != kernel_sha():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, q, k, v, budget_s: float):
    """The oracle as it stands, on whole (batch, head) units of the workload,
    in order, until all are done or about ``budget_s`` seconds have passed."""
    import numpy as np
    import oracle
    from io_aware_tiled_04_amd.workloads import as_f64_numpy
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q64 = as_f64_numpy(q)
    k64 = as_f64_numpy(k)
    v64 = as_f64_numpy(v)
    g = w.Hq // w.Hkv
    per_head = w.nominal_flops() / (w.B * w.Hq)
    heads, t0 = 0, time.perf_counter()
    while heads < w.B * w.Hq and (time.perf_counter() - t0) < budget_s:
        b, h = divmod(heads, w.Hq)
        o, lse = oracle.attention_head(q64[b, h], k64[b, h // g], v64[b, h // g], w.scale,
                                       w.causal)
        assert np.all(np.isfinite(o))
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": per_head * heads / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "threads_note": "matrix products on the BLAS threads counted in cores; numpy's exp "
                            "and elementwise passes on one thread",
            "sample": f"{heads} of {w.B * w.Hq} whole (batch, head) units of {w.name}, "
                      f"N={w.N} d={w.d}, "
                      f"fp64 numpy, {dt:.1f} s; nominal FLOPs as for the GPU "
                      f"(the oracle computes all N^2 scores)"}


def cpu_model() -> str | None:
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


CLOCK_LIB = os.path.join(ROOT, "io_aware_tiled_04_amd", "libfa_clock.so")


class ClockProbe:
    """The shader clock under load: a one-wave probe kernel (libfa_clock.so)
    on a second stream, at the default priority, spins for a fixed window of
    the GPU's constant-rate real-time counter while launches of the
    attention kernel run, and counts the shader-clock cycles that pass.
    clock = cycles / window, with the window timed by HIP events on the
    probe's stream.  The caller keeps launching for longer than the window,
    so that the probe sees only the attention kernel's load.  ``mhz`` is
    None when the probe library is missing or the window could not be
    timed."""

    def __init__(self, window_ms: float):
        import ctypes
        import torch
        self.mhz = None
        self.window_ms = window_ms
        self._lib = None
        if os.path.exists(CLOCK_LIB):
            self._lib = ctypes.CDLL(CLOCK_LIB)
            self._lib.fa_bench_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
            self._lib.fa_bench_clock_probe.restype = ctypes.c_int
        self._out = torch.zeros(2, dtype=torch.int64, device="cuda")
        self._stream = torch.cuda.Stream()
        self._e0 = torch.cuda.Event(enable_timing=True)
        self._e1 = torch.cuda.Event(enable_timing=True)

    def start(self):
        if self._lib is None:
            return
        # ticks of the 100 MHz real-time counter; the window is timed by
        # events, so the counter's exact rate does not enter the result
        ticks = int(self.window_ms * 1e5)
        self._e0.record(self._stream)
        rc = self._lib.fa_bench_clock_probe(self._out.data_ptr(), ticks, self._stream.cuda_stream)
        self._e1.record(self._stream)
        if rc != 0:
            self._lib = None

    def finish(self):
        import torch
        if self._lib is None:
            return
        torch.cuda.synchronize()
        cycles, rticks = (int(x) for x in self._out.tolist())
        ms = self._e0.elapsed_time(self._e1)
        if ms > 0 and cycles > 0:
            self.mhz = cycles / (ms * 1e3)
            self.realtime_mhz = rticks / (ms * 1e3)


def summarize(d: str, skip: int = 0, count: int = 0) -> None:
    """Per-kernel figures from a rocprofv3 output directory (its rocpd SQLite
    database): average dispatch duration from a kernel trace (leaving out
    each kernel's first ``skip`` dispatches, the warm-up), and per-dispatch
    counter values from a --pmc run, with the FETCH_SIZE / WRITE_SIZE scale
    factors implied by the elementwise copy of --calibrate-copy (which reads
    and writes COPY_BYTES each)."""
    import sqlite3
    for path in sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)):
        con = sqlite3.connect(path)
        views = {r[0] for r in con.execute("select name from sqlite_master")}
        print(f"# {os.path.relpath(path, d)}" + (f" (first {skip} dispatches of each kernel left out)"
                                                  if skip else "")
              + (f" (at most {count} dispatches of each kernel after those)" if count else ""))
        if "kernels" in views:
            per = {}
            for name, dur in con.execute("select name, duration from kernels order by start"):
                per.setdefault(name, []).append(dur)
            for name, durs in sorted(per.items(), key=lambda kv: -sum(kv[1])):
                kept = durs[skip:] if len(durs) > skip else durs
                if count:
                    kept = kept[:count]
                print(f"trace | {name[:80]} | calls={len(kept)} avg_us={sum(kept) / len(kept) / 1e3:.2f} "
                      f"min_us={min(kept) / 1e3:.2f} max_us={max(kept) / 1e3:.2f}")
        if "counters_collection" in views:
            rows = list(con.execute(
                "select kernel_name, counter_name, count(*), avg(value), min(value), max(value) "
                "from counters_collection group by kernel_name, counter_name"))
            copy_kib = COPY_BYTES / 1024
            factors = {}
            for kname, cname, n, avg, mn, mx in rows:
                if "vectorized_elementwise_kernel" in kname and "MulFunctor" in kname or \
                        ("AUnaryFunctor" in kname and cname in ("FETCH_SIZE", "WRITE_SIZE")):
                    factors[cname] = copy_kib / avg
            for kname, cname, n, avg, mn, mx in rows:
                f = factors.get(cname)
                extra = f" scale={f:.4f} scaled_bytes={avg * 1024 * f:.6g}" if f else ""
                print(f"pmc | {kname[:80]} | {cname} dispatches={n} avg_kib={avg:.6g} "
                      f"min={mn:.6g} max={mx:.6g}{extra}")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The shader clock ramps up over roughly the first 100 launches of the
    # forward kernel (launch time falls from about 310 to 265 us on c3, then
    # stays flat), so the default warm-up covers that ramp.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default=None,
                    help="workload (default c3; s1 with --splitkv)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--count", type=int, default=0,
                    help="with --summarize: keep at most this many dispatches of each kernel after --skip")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --summarize: leave out each kernel's first SKIP dispatches (the warm-up)")
    ap.add_argument("--splitkv", type=int, default=0,
                    help="time fa_fwd_splitkv with this many splits (and fa_fwd beside it)")
    ap.add_argument("--backward", action="store_true", help="time the backward pass (fa_bwd)")
    ap.add_argument("--kvouter", action="store_true",
                    help="time fa_fwd_kvouter (the K/V-outer loop order) beside fa_fwd")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="time fa_fwd_dropout with this drop probability (and fa_fwd beside it)")
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize, args.skip, args.count)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this forward pass shards over (batch, head) "
              "units with no communication, so run it with --gpus 1 (one process per GPU).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import oracle
    from io_aware_tiled_04_amd import fa
    from io_aware_tiled_04_amd.workloads import CONFIGS, EXTRA, as_f64_numpy, make_inputs

    if args.splitkv:
        return bench_splitkv(args)
    if args.backward:
        return bench_backward(args)
    if args.kvouter:
        return bench_kvouter(args)
    if args.dropout:
        return bench_dropout(args)
    w = CONFIGS[args.config or "c3"]
    if w.dtype != "bf16":
        print("the bench times the bf16 entry point; pick a bf16 configuration", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())

    def launch():
        rc = fa.fa_fwd(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale,
                       stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    region0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = region0.elapsed_time(region1)
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_ms = sum(launch_ms) / len(launch_ms)

    # The shader clock under this load, probed after the timed region over
    # extra untimed launches: the probe's wave holds a compute unit while it
    # runs, which would slow the timed launches (a grid of whole rounds of
    # workgroups, such as c3's 4 per CU, loses a fifth of a round).
    clock = ClockProbe(10.0)
    n_probe = int(12.0 / max(1e-3, launch_ms[-1])) + 2
    clock.start()
    for _ in range(n_probe):
        launch()
    clock.finish()

    if args.calibrate_copy:
        _calibrate_copy(dev)

    # parity of the timed outputs on sampled rows (oracle row by row)
    rng = np.random.default_rng(0)
    rows = [(b, h, int(i)) for b in range(w.B) for h in range(w.Hq)
            for i in [0, w.N - 1] + list(rng.integers(0, w.N, 2))]
    q64, k64, v64 = as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v)
    o_ref, lse_ref = oracle.attention_rows(q64, k64, v64, w.causal, w.scale, rows)
    idx = tuple(np.array(rows).T)
    o_got = as_f64_numpy(o)[idx]
    lse_got = as_f64_numpy(lse)[idx]
    err = np.abs(o_got - o_ref)
    lerr = np.abs(lse_got - lse_ref)
    parity_ok = bool(err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3)

    flops = w.nominal_flops()
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    # The shader clock ramps up over roughly the first 100 launches of a
    # process; the first and last few launches of the timed region show
    # where in that ramp the region sits.
    n_edge = min(5, len(launch_ms))
    first_us = 1e3 * sum(launch_ms[:n_edge]) / n_edge
    last_us = 1e3 * sum(launch_ms[-n_edge:]) / n_edge
    # Peak at the sampled clock: 256 CUs x 4 SIMDs x 1024 bf16 FLOP per clock
    # per SIMD (the published 2.5 PFLOP/s is this at 2.4 GHz).
    clk = clock.mhz
    clock_peak = 256 * 4 * 1024 * clk * 1e6 / 1e12 if clk else None
    # the committed counter summary covers the headline workload only
    traffic = read_traffic() if w.name == "c3" else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "N": w.N, "d": w.d, "causal": w.causal, "seed": w.seed,
                   "scale": w.scale, "flops_per_step": flops},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": f"fwd_bf16_kernel<{w.d}, {'causal' if w.causal else 'full'}>",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "min_launch_us": round(min(launch_ms) * 1e3, 2),
                     "first5_launch_us": round(first_us, 2),
                     "last5_launch_us": round(last_us, 2),
                     "last5_tflops": round(flops / (last_us * 1e-6) / 1e12, 2),
                     "sclk_mhz": round(clk, 1) if clk else None,
                     "sclk_source": "s_memtime cycles of a one-wave probe on a second stream over "
                                    f"{clock.window_ms:.1f} ms of {n_probe} untimed launches right after the "
                                    "timed ones" if clk else None,
                     "peak_at_sclk": round(clock_peak, 1) if clock_peak else None,
                     "frac_at_sclk": round(achieved / clock_peak, 4) if clock_peak else None},
        "parity": {"rows": len(rows), "max_abs_o": float(err.max()),
                   "mean_abs_o": float(err.mean()), "max_abs_lse": float(lerr.max()),
                   "ok": parity_ok},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0 if parity_ok else 1


def _calibrate_copy(dev):
    """Three elementwise copies of COPY_BYTES (read and write COPY_BYTES
    each): the reference that scales FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _time_launches(launch, stream, steps, warmup):
    """Average per-launch milliseconds (HIP events on the launch stream) and
    the timed region's total milliseconds."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    r1.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return sum(per) / len(per), r0.elapsed_time(r1)


def bench_splitkv(args) -> int:
    """fa_fwd_splitkv against fa_fwd on the same resident inputs; one JSON line.
    The merge kernel is HBM-bound: its algorithmic bytes are the partials read
    once (S * rows * (d + 1) * 4) plus O and LSE written once."""
    import numpy as np
    import torch

    import oracle
    from io_aware_tiled_04_amd import fa
    from io_aware_tiled_04_amd.workloads import CONFIGS, EXTRA, as_f64_numpy, make_inputs

    name = args.config or "s1"
    w = EXTRA.get(name) or CONFIGS[name]
    S = args.splitkv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    need = fa.fa_fwd_splitkv_workspace_size(w.B, w.Hq, w.N, w.d, S)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())

    def launch_split():
        rc = fa.fa_fwd_splitkv(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, S,
                               ws.data_ptr(), need, stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    def launch_direct():
        rc = fa.fa_fwd(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale,
                       stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    direct_ms, _ = _time_launches(launch_direct, stream, args.steps, args.warmup)
    split_ms, split_total = _time_launches(launch_split, stream, args.steps, args.warmup)

    rng = np.random.default_rng(0)
    rows = [(b, h, int(i)) for b in range(w.B) for h in range(w.Hq)
            for i in [0, w.N - 1] + list(rng.integers(0, w.N, 6))]
    o_ref, lse_ref = oracle.attention_rows(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                           w.causal, w.scale, rows)
    idx = tuple(np.array(rows).T)
    err = np.abs(as_f64_numpy(o)[idx] - o_ref)
    lerr = np.abs(as_f64_numpy(lse)[idx] - lse_ref)
    ok = bool(err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3)
    flops = w.nominal_flops()
    rows_total = w.B * w.Hq * w.N
    # The merge reads, for each row, the partials of the key ranges the row
    # sees (all ranges with keys; when causal, those starting at or before
    # the row), and writes O (bf16) and LSE once.
    bc = 64 if w.d == 128 else 128                 # keys per tile of the kernel
    n_kt = -(-w.N // bc)
    kq, kr = divmod(n_kt, S)
    starts = [(s * kq + min(s, kr)) * bc for s in range(S) if kq + (1 if s < kr else 0) > 0]
    if w.causal:
        seen = sum(sum(1 for st in starts if st <= r) for r in range(w.N))
    else:
        seen = len(starts) * w.N
    merge_bytes = w.B * w.Hq * seen * (w.d + 1) * 4 + rows_total * (2 * w.d + 4)
    out = {
        "metric": "attention fwd TFLOP/s, split-KV path (bf16)",
        "value": round(flops * args.steps / (split_total * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(split_total / args.steps, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "N": w.N, "d": w.d, "causal": w.causal, "seed": w.seed, "splits": S,
                   "flops_per_step": flops},
        "split_avg_launch_us": round(split_ms * 1e3, 2),
        "direct_avg_launch_us": round(direct_ms * 1e3, 2),
        "direct_tflops": round(flops / (direct_ms * 1e-3) / 1e12, 2),
        "speedup_vs_direct": round(direct_ms / split_ms, 3),
        "merge_algorithmic_bytes": merge_bytes,
        "parity": {"rows": len(rows), "max_abs_o": float(err.max()),
                   "mean_abs_o": float(err.mean()), "max_abs_lse": float(lerr.max()), "ok": ok},
    }
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


def bench_dropout(args) -> int:
    """fa_fwd_dropout against fa_fwd on the same resident inputs (default
    c3); one JSON line.  FLOPs are the nominal forward count: dropout adds
    generator and integer work, not matrix work.  Parity: sampled rows
    against the oracle's dropout forward."""
    import numpy as np
    import torch

    import oracle
    from io_aware_tiled_04_amd import fa
    from io_aware_tiled_04_amd.workloads import CONFIGS, EXTRA, as_f64_numpy, make_inputs

    name = args.config or "c3"
    w = EXTRA.get(name) or CONFIGS[name]
    p, seed, offset = float(args.dropout), 0x5EED5EED12345678, 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())

    def launch_direct():
        rc = fa.fa_fwd(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    def launch_drop():
        rc = fa.fa_fwd_dropout(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, p, seed,
                               offset, stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    direct_ms, _ = _time_launches(launch_direct, stream, args.steps, args.warmup)
    drop_ms, drop_total = _time_launches(launch_drop, stream, args.steps, args.warmup)

    rng = np.random.default_rng(0)
    rows = [(0, 0, 0), (w.B - 1, w.Hq - 1, w.N - 1)] + [
        (int(rng.integers(0, w.B)), int(rng.integers(0, w.Hq)), int(rng.integers(0, w.N))) for _ in range(30)]
    o_ref, lse_ref = oracle.attention_dropout_rows(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v),
                                                   w.causal, w.scale, p, seed, offset, rows)
    idx = tuple(np.array(rows).T)
    err = np.abs(as_f64_numpy(o)[idx] - o_ref)
    excess = err - 2.0 ** -8 * np.abs(o_ref)
    lerr = np.abs(as_f64_numpy(lse)[idx] - lse_ref)
    factor = 1.0 / (1.0 - float(np.float32(p)))
    ok = bool(excess.max() <= 2e-2 and err.mean() <= 2e-3 * factor and lerr.max() <= 1e-3)
    flops = w.nominal_flops()
    out = {
        "metric": "attention fwd TFLOP/s with dropout on the weights (bf16)",
        "value": round(flops * args.steps / (drop_total * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(drop_total / args.steps, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N,
                   "d": w.d, "causal": w.causal, "seed": w.seed, "p_drop": p,
                   "flops_per_step": flops},
        "kernel": f"fwd_bf16_kernel<{w.d}, {'causal' if w.causal else 'full'}, dropout>",
        "dropout_avg_launch_us": round(drop_ms * 1e3, 2),
        "direct_avg_launch_us": round(direct_ms * 1e3, 2),
        "dropout_tflops_per_launch": round(flops / (drop_ms * 1e-3) / 1e12, 2),
        "direct_tflops_per_launch": round(flops / (direct_ms * 1e-3) / 1e12, 2),
        "slowdown_vs_direct": round(drop_ms / direct_ms, 3),
        "parity": {"rows": len(rows), "max_abs_o": float(err.max()), "mean_abs_o": float(err.mean()),
                   "max_abs_lse": float(lerr.max()), "ok": ok},
    }
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


def kvouter_structural_bytes(w) -> dict:
    """Bytes the K/V-outer loop order moves by construction, from the loop
    structure of fa_fwd_kvouter: K and V once per head; per visible (32-row
    query block, 64-key tile) pair the block's Q (bf16), and its fp32 output
    accumulator plus row max and row sum read (all but the first tile) and
    written (all but the last); O (bf16) and LSE written once."""
    d, N, heads = w.d, w.N, w.B * w.Hq
    nblk, ntile = -(-N // 32), -(-N // 64)
    pairs = reads = writes = 0
    for rb in range(nblk):
        last = min(ntile - 1, (min(N, 32 * rb + 32) - 1) // 64) if w.causal else ntile - 1
        pairs += last + 1
        reads += last          # tiles 1..last read the state
        writes += last         # tiles 0..last-1 write it
    state = 32 * d * 4 + 2 * 64 * 4      # O accumulator + per-lane m and l of one block
    per_head = pairs * 32 * d * 2 + (reads + writes) * state
    kv = w.B * w.Hkv * N * d * 2 * 2
    out = heads * N * d * 2 + heads * N * 4
    return {"pairs_per_head": pairs, "read_bytes": heads * (pairs * 32 * d * 2 + reads * state) + kv,
            "write_bytes": heads * writes * state + out,
            "total_bytes": heads * per_head + kv + out}


def bench_kvouter(args) -> int:
    """fa_fwd_kvouter against fa_fwd on the same resident inputs (default c3);
    one JSON line with both per-launch times and the K/V-outer order's
    structural bytes.  Parity: sampled rows against the oracle."""
    import numpy as np
    import torch

    import oracle
    from io_aware_tiled_04_amd import fa
    from io_aware_tiled_04_amd.workloads import CONFIGS, EXTRA, as_f64_numpy, make_inputs

    name = args.config or "c3"
    w = EXTRA.get(name) or CONFIGS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    need = fa.fa_fwd_kvouter_workspace_size(w.B, w.Hq, w.N, w.d)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr())

    def launch_direct():
        rc = fa.fa_fwd(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    def launch_kv():
        rc = fa.fa_fwd_kvouter(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, ws.data_ptr(), need,
                               stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    direct_ms, _ = _time_launches(launch_direct, stream, args.steps, args.warmup)
    kv_ms, kv_total = _time_launches(launch_kv, stream, args.steps, args.warmup)
    if args.calibrate_copy:
        _calibrate_copy(dev)

    rng = np.random.default_rng(0)
    rows = [(0, 0, 0), (w.B - 1, w.Hq - 1, w.N - 1)] + [
        (int(rng.integers(0, w.B)), int(rng.integers(0, w.Hq)), int(rng.integers(0, w.N))) for _ in range(30)]
    o_ref, lse_ref = oracle.attention_rows(as_f64_numpy(q), as_f64_numpy(k), as_f64_numpy(v), w.causal, w.scale,
                                           rows)
    idx = tuple(np.array(rows).T)
    err = np.abs(as_f64_numpy(o)[idx] - o_ref)
    lerr = np.abs(as_f64_numpy(lse)[idx] - lse_ref)
    ok = bool(err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3)
    flops = w.nominal_flops()
    sb = kvouter_structural_bytes(w)
    alg = w.B * w.Hq * w.N * w.d * 2 * 2 + w.B * w.Hkv * w.N * w.d * 2 * 2 + w.B * w.Hq * w.N * 4
    out = {
        "metric": "attention fwd TFLOP/s, K/V-outer loop order (bf16)",
        "value": round(flops * args.steps / (kv_total * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(kv_total / args.steps, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "seed": w.seed, "flops_per_step": flops},
        "kernel": f"fwd_kvouter_kernel<{w.d}, {'causal' if w.causal else 'full'}>",
        "kvouter_avg_launch_us": round(kv_ms * 1e3, 2),
        "direct_avg_launch_us": round(direct_ms * 1e3, 2),
        "slowdown_vs_direct": round(kv_ms / direct_ms, 3),
        "algorithmic_bytes": alg,
        "kvouter_structural_bytes": sb["total_bytes"],
        "kvouter_structural_GBps": round(sb["total_bytes"] / (kv_ms * 1e-3) / 1e9, 1),
        "parity": {"rows": len(rows), "max_abs_o": float(err.max()), "mean_abs_o": float(err.mean()),
                   "max_abs_lse": float(lerr.max()), "ok": ok},
    }
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


def bench_backward(args) -> int:
    """fa_bwd on resident inputs (the forward's O and LSE computed once
    beforehand); one JSON line.  Nominal FLOPs: five N^2 d products per head
    (S, dP, dV, dQ, dK), i.e. 2.5 times the forward's, halved for causal; the
    kernels recompute S and dP (8 products), which is not credited.  With
    --dropout P: fa_fwd_dropout, then fa_bwd_dropout with its state."""
    import numpy as np
    import torch

    import oracle
    from io_aware_tiled_04_amd import fa
    from io_aware_tiled_04_amd.workloads import CONFIGS, EXTRA, as_f64_numpy, make_grad, make_inputs

    name = args.config or "c3"
    w = EXTRA.get(name) or CONFIGS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(w)
    do = make_grad(w)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    pdrop, seed, offset = float(args.dropout), 0x5EED5EED12345678, 1
    if pdrop:
        o, lse, _ = fa.fwd_dropout(qd, kd, vd, pdrop, seed, offset, causal=w.causal, scale=w.scale)
    else:
        o, lse = fa.fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    need = fa.fa_bwd_workspace_size(w.B, w.Hq, w.N)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptrs = tuple(t.data_ptr() for t in (qd, kd, vd, o, lse, dod, dq, dk, dv))

    def launch():
        if pdrop:
            rc = fa.fa_bwd_dropout(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, pdrop, seed,
                                   offset, ws.data_ptr(), need, stream.cuda_stream)
        else:
            rc = fa.fa_bwd(*ptrs, w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.scale, ws.data_ptr(),
                           need, stream.cuda_stream)
        if rc != fa.FA_OK:
            raise fa.FaError(rc)

    avg_ms, total_ms = _time_launches(launch, stream, args.steps, args.warmup)
    if args.calibrate_copy:
        _calibrate_copy(dev)
    # parity of the first GQA group of batch 0 (its query heads and its K/V
    # head) against the oracle's gradients; tolerances relative to each
    # gradient's magnitude, as in the backward tests
    q64, k64, v64, do64 = (as_f64_numpy(t) for t in (q, k, v, do))
    g = w.Hq // w.Hkv
    dk_ref = np.zeros_like(k64[0, 0])
    dv_ref = np.zeros_like(v64[0, 0])
    rel = []
    for h in range(g):
        if pdrop:
            gq, gk, gv = oracle.attention_dropout_backward_head(q64[0, h], k64[0, 0], v64[0, 0], do64[0, h],
                                                                w.scale, w.causal, pdrop, seed, offset, h)
        else:
            gq, gk, gv = oracle.attention_backward_head(q64[0, h], k64[0, 0], v64[0, 0], do64[0, h],
                                                        w.scale, w.causal)
        dk_ref += gk
        dv_ref += gv
        rel.append(("dq", as_f64_numpy(dq[0, h]), gq))
    rel += [("dk", as_f64_numpy(dk[0, 0]), dk_ref), ("dv", as_f64_numpy(dv[0, 0]), dv_ref)]
    worst = {}
    ok = True
    for name_, got, ref in rel:
        mag = max(float(np.abs(ref).max()), 1e-4)
        e = np.abs(got - ref)
        worst[name_] = max(worst.get(name_, 0.0), float(e.max() / mag))
        ok = ok and bool(e.max() <= 2e-2 * mag and e.mean() <= 2e-3 * mag)
    flops = 2.5 * w.nominal_flops()
    out = {
        "metric": "attention bwd TFLOP/s (bf16, nominal 2.5x forward FLOPs)"
                  + (f", dropout p={pdrop}" if pdrop else ""),
        "value": round(flops * args.steps / (total_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "N": w.N, "d": w.d, "causal": w.causal, "seed": w.seed, "p_drop": pdrop,
                   "flops_per_step": flops},
        "avg_launch_us": round(avg_ms * 1e3, 2),
        "pct_of_peak": round(100 * flops / (avg_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "parity": {"heads": g, "max_abs_rel": worst, "ok": ok},
    }
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
