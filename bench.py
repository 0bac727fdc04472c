"""Benchmark of the attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--tile R,C]
                    [--shape B,H,N] [--num-splits S] [--no-cpu-baseline] [--gpus 1]

A step is one attention forward (one fa_fwd call) over the whole workload,
inputs already resident in HBM. Prints ONE JSON line. The default workload is
bf16, causal, d=128, N=8192, B=2, H=32. Before the W warm-up steps the step
runs back to back for at least --settle-ms (300 ms) so that the GPU has left
its idle clock, which it takes a few hundred milliseconds of load to do (the
first ten launches after idle average 1.5 ms, the sustained rate is 1.05
ms), and on (at most 3 s) until the SMU's metrics table, refreshed about once
a second, has been read under load; the JSON line reports that phase as
`settle`, and as `clock` the kernel's clock from the committed rocprofv3
counters of this kernel and shape (GRBM_GUI_ACTIVE cycles over kernel time)
next to the SMU's readings of the shader clock and the socket power (with
the power cap) from the settle phase and the timed steps.

--bwd times the backward (one fa_bwd call per step: the D/LSE pass, the
dK/dV kernel and the dQ kernel) on the forward's output, with nominal
FLOPs 2.5x the forward's (the five products S, dP, dV, dK, dQ; the kernels
also recompute S and dP once more, which is not counted).

--workload sm_* times the standalone row softmax instead (one fa_softmax_fwd
call per step; HBM-bound, reported in GB/s of algorithmic traffic: x read
once, y and LSE written once).

--workload fp8_* times the FP8 (E4M3) forward (one fa_fwd_fp8 call per step,
--max-offset 8 by default), against the dense FP8 MFMA peak.

--shape replaces the workload's (B, H, N), or (rows, cols) for sm_* workloads (the workload is then reported as
NAME@BxHxN). --num-splits S times the split-KV entry point instead (S = 0:
the library's choice); a step is then its two launches, attention and merge,
and the per-launch time in `roofline` covers both.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X dense MFMA peak for bf16/fp16: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3,
               # fp8: twice the 16-bit rate, 256 x 8192 FLOP/clk x 2.4 GHz
               "e4m3": 5033.2}
# MI355X HBM3E peak bandwidth.
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_causal_n8192_d128"
KERNEL_PREFIX = "attn_fwd_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--tile", default=None, help="block_r,block_c")
    ap.add_argument("--shape", default=None, help="B,H,N")
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--bwd", action="store_true")
    ap.add_argument("--max-offset", type=int, default=8, help="fp8 workloads: 8 or 0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="after the timed steps, time 5 more launches each preceded by a write of this many MiB "
                         "(0: skip); reported as roofline.flushed_*")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up steps, run the step back to back for this long so the GPU leaves "
                         "its idle clock (0: skip); reported as `settle`")
    return ap.parse_args()


def cpu_baseline(w, x, target_s):
    """Times the float64 oracle on a bounded random sample of rows of the same
    workload, on this host's cores; reports nominal TFLOP/s of that sample.
    FP8 workloads run the FP8 oracle (E4M3 decode, then the same three-pass
    attention)."""
    import numpy as np
    import oracle

    B, H, N, d = w.B, w.H, w.N, w.d
    rng = np.random.default_rng(123)
    threads = oracle.max_threads()
    fp8 = w.in_dtype == "e4m3"
    # the oracle reads float32 containers of the input values; convert once
    if fp8:
        q, k, v = (x[n] for n in ("q", "k", "v"))
    else:
        q, k, v = (x[n].float().numpy() for n in ("q", "k", "v"))
    mask = None if x["mask"] is None else x["mask"].numpy()

    def attention(b, h, rr):
        sl = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
        mk = None if mask is None else mask[b:b + 1]
        if fp8:
            oracle.fp8.attention_fp8(sl(q), sl(k), sl(v), x["scale"], *x["descale"], causal=x["causal"], mask=mk,
                                     rows=rr, nthreads=threads)
        else:
            oracle.attention(sl(q), sl(k), sl(v), x["scale"], x["causal"], mk, rows=rr, nthreads=threads)

    def run(nrows, cap=float("inf")):
        # rows of the sample, head by head; stops after the head that passes
        # `cap` seconds (all heads are drawn alike, so the rows done so far are
        # still a uniform sample of query positions)
        rows = np.sort(rng.choice(B * H * N, size=nrows, replace=False))
        flops, done = 0.0, 0
        t0 = time.perf_counter()
        for bh in np.unique(rows // N):
            b, h = divmod(int(bh), H)
            rr = rows[(rows // N) == bh] - bh * N
            attention(b, h, rr)
            keys = (rr + 1) if w.causal else np.full(rr.shape, N)
            flops += float(4.0 * d * keys.sum())
            done += len(rr)
            if time.perf_counter() - t0 > cap:
                break
        return time.perf_counter() - t0, flops, done

    run(64)                      # loads the oracle library and warms the caches
    dt, fl, n = run(2048)        # calibration sample
    # grow the sample until it takes about target_s, at most 4x per step; the
    # rate per row is not constant (thread use, per-head setup, a host whose
    # CPU share shrinks under sustained load), so each run also stops once it
    # has taken 1.5 * target_s
    for _ in range(8):
        if dt >= 0.7 * target_s or n >= B * H * N:
            break
        n = int(min(B * H * N, max(2048, n * min(4.0, target_s / max(dt, 1e-3)))))
        dt, fl, n = run(n, cap=1.5 * target_s)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} rows of {w.name} drawn uniformly at random (seed 123), float64 three-pass "
                      f"oracle{' of the decoded E4M3 inputs' if fp8 else ''}, nominal 4*d*(allowed keys) FLOP "
                      f"per row, {dt:.1f} s"}


def traffic(workload, kernel=KERNEL_PREFIX, tile=None):
    """(HBM bytes per launch, detail) from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, when it was taken on the current kernel sources and
    the same tile shape; else (None, None)."""
    from online_softmax_03_amd import profiling
    t = profiling.current_traffic(workload, kernel, tile)
    if t is None:
        return None, None
    return round(t["hbm_bytes_per_launch"]), {
        "read_bytes": round(t["hbm_read_bytes_per_launch"]),
        "write_bytes": round(t["hbm_write_bytes_per_launch"]),
        "source": os.path.relpath(profiling.traffic_file(workload, kernel), ROOT)}


class ClockSampler:
    """Reads the GPU's shader clock from the SMU metrics table through amdsmi
    (current_gfxclk, MHz), with the socket power (W) and the power cap, in a
    background thread while `active`. The table is refreshed about once a
    second and its clock is an average over the period before the refresh,
    so the first refresh after the sampler starts still covers time before
    the load: only the readings of later refreshes count, and a run shorter
    than two refresh periods gets none."""

    def __init__(self, period_s=0.005):
        self.period_s = period_s
        self.samples = []
        self.watts = []
        self.power_cap_w = None
        self.active = False
        self.source = None
        self._stop = False
        self._start_stamp = None
        self._read = self._open()
        self._thread = None
        if self._read is not None:
            import threading
            self._start_stamp = self._read()[0]
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()

    def _open(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handle = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                try:
                    w = float(amdsmi.amdsmi_get_power_info(handle)["current_socket_power"])
                except Exception:
                    w = None
                return m["system_clock_counter"], float(m["current_gfxclk"]), w
            read()
            try:
                cap = float(amdsmi.amdsmi_get_power_cap_info(handle)["power_cap"]) / 1e6
            except Exception:
                cap = None
            self.power_cap_w = cap
            self.source = "amdsmi gpu_metrics current_gfxclk, power_info current_socket_power"
            return read
        except Exception:
            return None

    def _loop(self):
        last = self._start_stamp
        refreshes = 0
        while not self._stop:
            if self.active:
                try:
                    stamp, mhz, watts = self._read()
                    if stamp != last:
                        refreshes += 1
                        if refreshes >= 2:
                            self.samples.append(mhz)
                            if watts is not None:
                                self.watts.append(watts)
                        last = stamp
                except Exception:
                    pass
            time.sleep(self.period_s)

    def available(self):
        return self._read is not None

    def close(self):
        self._stop = True
        if self._thread is not None:
            self._thread.join()

    def report(self):
        if not self.samples:
            return None
        return {"median_mhz": _median(self.samples),
                "median_socket_w": _median(self.watts) if self.watts else None,
                "power_cap_w": self.power_cap_w, "samples": len(self.samples), "source": self.source}


def clock_report(sampler, workload, kernel, tile):
    """The clock the kernel runs at: GRBM_GUI_ACTIVE cycles over kernel time
    from the committed rocprofv3 counter summary of this kernel, workload and
    tile (when taken on the current sources), and the SMU's clock and power
    readings under the run's load (ClockSampler)."""
    from online_softmax_03_amd import profiling
    c = profiling.current_counters(workload, kernel, tile)
    return {"counter_ghz": None if c is None else round(c["clock_ghz"], 3),
            "counter_mfma_busy": None if c is None else round(c["mfma_busy"], 4),
            "counter_source": None if c is None else os.path.relpath(profiling.counters_file(workload, kernel), ROOT),
            "smu": sampler.report()}


def settle(step, settle_ms, clock=None, max_ms=3000.0):
    """Runs `step` back to back for `settle_ms` of wall time (at least once),
    and on until `clock` (a ClockSampler) holds a reading of the SMU's
    metrics table, at most `max_ms` in all; then synchronises and returns the
    number of steps run and the milliseconds they took. After idle the GPU
    starts its clock at a few hundred MHz and takes a few hundred
    milliseconds of load to reach its working clock (the first ten 1 ms launches of the default workload
    average 1.5 ms, the next ones 1.05); the table refreshes about once a
    second, and its first refresh under load still averages the idle time
    before, so a reading of the loaded clock and power takes one to two
    seconds of this phase."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while True:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3
            waiting = clock is not None and clock.available() and not clock.samples
            if ms >= max_ms or (ms >= settle_ms and not waiting):
                break
    torch.cuda.synchronize()
    return n, round((time.perf_counter() - t0) * 1e3, 1)


def timed_steps(step, stream, steps, warmup, clock=None):
    """Runs `warmup` untimed steps, then `steps` timed ones back to back with
    one HIP event pair on `stream` around all of them. Returns (wall seconds,
    average ms per step by the events). An event pair around every launch
    would add its own ~6 us of wall time to each step (the next launch waits
    for the end-of-kernel timestamp): 0.5% of the default step, 7% of a
    90 us d = 64 step. `clock` (a ClockSampler) stops sampling when the
    timed steps end."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if clock is not None:
        clock.active = False
    return wall, a.elapsed_time(b) / steps


def per_launch(step, stream, n):
    """`n` more launches after the timed ones, each inside its own HIP event
    pair on `stream` (median and minimum per launch; not part of `value`)."""
    import torch
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def flushed_launches(step, stream, n, flush_mib):
    """`n` launches, each after a write of `flush_mib` MiB to a scratch buffer
    (so the previous launch's inputs are no longer in the last-level cache),
    timed with a HIP event pair on `stream` around the launch only. Returns
    the per-launch ms list."""
    import torch
    scratch = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda:0")
    times = []
    for _ in range(n):
        scratch.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del scratch
    return times


def _median(xs):
    ys = sorted(xs)
    m = len(ys) // 2
    return ys[m] if len(ys) % 2 else 0.5 * (ys[m - 1] + ys[m])


def softmax_cpu_baseline(w, x, target_s):
    """Times the float64 row-softmax oracle on a bounded random sample of rows
    of the same workload; reports GB/s of the workload's algorithmic bytes."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(123)
    xf = x.float().numpy()
    per_row = w.algorithmic_bytes() / w.rows

    def run(n):
        rows = np.sort(rng.choice(w.rows, size=n, replace=False))
        t0 = time.perf_counter()
        for i in range(0, n, 64):
            oracle.softmax_rows(xf[rows[i:i + 64]])
        return time.perf_counter() - t0

    run(8)
    dt = run(64)
    n = int(min(w.rows, max(64, 64 * target_s / max(dt, 1e-3))))
    dt = run(n)
    return {"value": round(per_row * n / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} rows of {w.name} drawn uniformly at random (seed 123), float64 numpy three-pass "
                      f"oracle in one thread, bytes counted as for the GPU, {dt:.1f} s"}


def bench_softmax(args):
    import torch
    from online_softmax_03_amd import softmax as S
    from online_softmax_03_amd import workloads as W

    w = W.SOFTMAX_BY_NAME[args.workload]
    if args.shape:
        rows, cols = (int(t) for t in args.shape.split(","))
        w = w.with_shape(rows=rows, cols=cols, name=f"{w.name}@{rows}x{cols}")
    x = W.generate_softmax(w)
    dev = torch.device("cuda:0")
    xd = x.to(dev)
    y = torch.empty(x.shape, dtype=W.DTYPES[w.out_dtype], device=dev)
    lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        S.softmax_rows(xd, out_dtype=y.dtype, out=y, lse=lse)

    clock = ClockSampler()
    clock.active = True
    settled, settled_ms = settle(step, args.settle_ms, clock) if args.settle_ms > 0 else (0, 0.0)
    wall, avg_ms = timed_steps(step, stream, args.steps, args.warmup, clock)
    clock.close()
    launch_ms = per_launch(step, stream, args.steps)
    avg_s = avg_ms / 1e3
    nbytes = w.algorithmic_bytes()
    # the library's choice: registers (up to 8192 16-byte vectors), registers
    # + LDS (up to 20480 vectors for 16-bit inputs, 32768 for fp32), streamed
    per_vec = 4 if w.in_dtype == "f32" else 8
    nvec = w.cols // per_vec
    if w.cols % per_vec != 0 or nvec > (32768 if w.in_dtype == "f32" else 20480):
        kernel = "softmax_stream_kernel"
    elif nvec > 8192:
        kernel = "softmax_resident_lds_kernel"
    else:
        kernel = "softmax_resident_kernel"
    hbm_bytes, hbm_detail = traffic(w.name, kernel)
    result = {
        "metric": "row softmax HBM GB/s (algorithmic bytes: x read once, y and LSE written once)",
        "value": round(nbytes * args.steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "cols": w.cols, "in_dtype": w.in_dtype,
                   "out_dtype": w.out_dtype, "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / avg_s / 1e9, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(nbytes / avg_s / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": hbm_bytes, "traffic_detail": hbm_detail, "kernel": kernel,
                     "avg_launch_ms": round(avg_s * 1e3, 4),
                     "min_launch_ms": round(min(launch_ms), 4)},
        "clock": clock_report(clock, w.name, kernel, None),
        "settle": {"ms": settled_ms, "min_ms": args.settle_ms, "steps": settled},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = softmax_cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard over (batch, head) with no exchange: run one process per GPU on its share of the heads)",
              file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("sm_"):
        return bench_softmax(args)

    import torch
    from online_softmax_03_amd import attention as A
    from online_softmax_03_amd import capi
    from online_softmax_03_amd import workloads as W

    fp8 = args.workload in W.FP8_BY_NAME
    w = W.FP8_BY_NAME[args.workload] if fp8 else W.BY_NAME[args.workload]
    if fp8 and (args.tile or args.num_splits is not None or args.bwd):
        sys.exit("fp8 workloads take none of --tile, --num-splits, --bwd")
    if args.shape:
        B, H, N = (int(t) for t in args.shape.split(","))
        w = w.with_shape(B=B, H=H, N=N, name=f"{w.name}@{B}x{H}x{N}")
    x = W.generate(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    mask = None if x["mask"] is None else x["mask"].to(dev)
    out_dt = W.DTYPES[w.out_dtype]
    o = torch.empty(q.shape, dtype=out_dt, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    tile = tuple(int(t) for t in args.tile.split(",")) if args.tile else None
    if fp8:
        tile = (128, 64)  # the FP8 kernel's one shape: 4 waves x 32 queries, 64-key tiles
    elif tile is None:
        st, tile = capi.fa_default_tile(w.B, w.H, w.N, w.d, A._DT[q.dtype], A._DT[out_dt], int(w.causal),
                                        int(mask is not None))
        assert st == 0

    stream = torch.cuda.current_stream(dev)
    splits, ws = args.num_splits, None
    if splits is not None:
        if args.tile:
            sys.exit("--num-splits uses the default tile; drop --tile")
        if splits == 0:
            splits = capi.fa_splitkv_num_splits(w.B, w.H, w.N, w.d, A._DT[q.dtype], w.causal)
        ws = torch.empty(capi.fa_splitkv_workspace_bytes(w.B, w.H, w.N, w.d, splits), dtype=torch.uint8,
                         device=dev)

    if args.bwd:
        if splits is not None or args.tile:
            sys.exit("--bwd takes neither --num-splits nor --tile")
        fo, flse = A.attention_fwd(q, k, v, scale=w.scale, causal=w.causal, key_padding_mask=mask)
        dout = W.generate_dout(w).to(dev)
        grads = tuple(torch.empty(q.shape, dtype=q.dtype, device=dev) for _ in range(3))
        bws = torch.empty(capi.fa_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def step():
        if fp8:
            A.attention_fwd_fp8(q, k, v, scale=w.scale, descale_q=w.descale[0], descale_k=w.descale[1],
                                descale_v=w.descale[2], causal=w.causal, key_padding_mask=mask, out_dtype=out_dt,
                                max_offset=args.max_offset, out=o, lse=lse)
        elif args.bwd:
            A.attention_bwd(q, k, v, fo, dout, flse, scale=w.scale, causal=w.causal, key_padding_mask=mask,
                            workspace=bws, out=grads)
        elif splits is None:
            A.attention_fwd(q, k, v, scale=w.scale, causal=w.causal, key_padding_mask=mask,
                            out_dtype=out_dt, tile=tile, out=o, lse=lse)
        else:
            A.attention_fwd(q, k, v, scale=w.scale, causal=w.causal, key_padding_mask=mask,
                            out_dtype=out_dt, out=o, lse=lse, num_splits=splits, workspace=ws)

    # the GPU leaves its idle clock first; then the timed steps inside one HIP
    # event pair on the stream the kernel is launched on, with the shader
    # clock sampled alongside
    clock = ClockSampler()
    clock.active = True
    settled, settled_ms = settle(step, args.settle_ms, clock) if args.settle_ms > 0 else (0, 0.0)
    wall, avg_ms = timed_steps(step, stream, args.steps, args.warmup, clock)
    clock.close()
    launch_ms = per_launch(step, stream, args.steps)
    avg_launch_s = avg_ms / 1e3
    flushed = flushed_launches(step, stream, 5, args.flush_mib) if args.flush_mib > 0 else None

    flops = w.nominal_flops() * (2.5 if args.bwd else 1.0)
    value = flops * args.steps / wall / 1e12
    achieved = flops / avg_launch_s / 1e12
    effective = None
    if x["lens"] is not None:
        # allowed (query, key) pairs under the key mask (and the causal mask):
        # the FLOPs the kernel must do, not the nominal count
        n = torch.arange(w.N, dtype=torch.float64)
        pairs = sum(float(torch.minimum(n + 1, torch.tensor(float(l))).sum()) if w.causal else float(w.N * l)
                    for l in x["lens"].tolist()) * w.H
        eff_flops = 4.0 * w.d * pairs * (2.5 if args.bwd else 1.0)
        effective = {"flops_per_step": eff_flops, "tflops": round(eff_flops / avg_launch_s / 1e12, 2),
                     "fraction_of_nominal": round(eff_flops / flops, 4)}
    peak = PEAK_TFLOPS[w.in_dtype]
    kernel = "attn_fwd_fp8_kernel" if fp8 else ("attn_fwd_f32_kernel" if w.in_dtype == "f32" else KERNEL_PREFIX)
    hbm_bytes, hbm_detail = (traffic(w.name, kernel, None if fp8 else tile) if (splits is None and not args.bwd)
                             else (None, None))
    # the roofline credits only the allowed (query, key) pairs: padded keys
    # are work the kernel skips, not work it does
    credited = effective["flops_per_step"] if effective else flops
    result = {
        "metric": ("attention bwd TFLOP/s (nominal 2.5x the forward's FLOPs) and % of MFMA bf16 peak"
                   if args.bwd else
                   "FP8 attention fwd TFLOP/s and % of MFMA fp8 peak (causal, d=128, N=8192)" if fp8 else
                   "attention fwd TFLOP/s and % of MFMA bf16 peak (causal, d=128, N=8192)"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "key_padding": w.key_padding, "in_dtype": w.in_dtype, "out_dtype": w.out_dtype,
                   "block_r": tile[0], "block_c": tile[1], "num_splits": splits, "pass": "bwd" if args.bwd else "fwd",
                   "flops_per_step": flops},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        **({"effective": effective} if effective else {}),
        **({"max_offset": args.max_offset, "descale": list(w.descale)} if fp8 else {}),
        "roofline": {"bound": "mfma", "achieved": round(credited / avg_launch_s / 1e12, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(credited / avg_launch_s / 1e12 / peak, 4),
                     **({"nominal_achieved": round(achieved, 2), "nominal_frac": round(achieved / peak, 4),
                         "credited": "allowed (query, key) pairs"} if effective else {}),
                     "traffic": hbm_bytes, "traffic_detail": hbm_detail,
                     "kernel": "attn_bwd (prep + dkdv + dq)" if args.bwd else kernel,
                     "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                     "median_launch_ms": round(_median(launch_ms), 4),
                     "min_launch_ms": round(min(launch_ms), 4),
                     **({"flushed_mib": args.flush_mib, "flushed_median_launch_ms": round(_median(flushed), 4),
                         "flushed_min_launch_ms": round(min(flushed), 4)} if flushed else {})},
        "clock": clock_report(clock, w.name, kernel, None if fp8 else tile) if (splits is None and not args.bwd)
        else {"smu": clock.report()},
        "settle": {"ms": settled_ms, "min_ms": args.settle_ms, "steps": settled},
    }
    if not args.no_cpu_baseline and not args.bwd:
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
