#!/usr/bin/env python3
"""Benchmark: attention forward + backward throughput on one MI355X.

The default run times every configuration of the benchmark set, each in its own phase, and prints
one JSON line:
  c1  B=1 H=1  N=256   d=64  non-causal forward (seed 0)
  c2  B=4 H=16 N=2048  d=64  non-causal forward
  c3  B=2 H=32 N=4096  d=128 causal forward
  c4  B=1 H=16 N=16384 d=128 causal forward, every 64th query row x8
  c5  B=2 H=16 N=4096  d=128 causal forward + backward
The line's ``value`` is c5's: one step is one pass of the whole path (the fused forward kernel, then
the two launches attn_bwd makes: the dQ kernel, which also forms D = rowsum(dO o O), then the dK/dV
kernel) over resident synthetic inputs.  ``configs`` holds every configuration's kernel times
(median, min, max), TFLOP/s and fraction of the bf16 MFMA peak, its seed and the SHA-256 of its
inputs, the GPU clock and power measured while it ran, and the CPU oracle timed on a sample of its
inputs together with the largest error of the GPU result on that sample.
``--workload NAME`` times one workload instead: one of the five, or a widened one (dec: split-key
decoding; c3f8/c4f8: the 8-bit forward; c5g, c5u, c5d256: grouped heads, unequal lengths, d = 256;
fa3: FlashAttention v3's ablation workload).

Each phase first runs its step untimed for --ramp-seconds (2 s): an idle MI355X needs a fraction of
a second under load before its clocks settle, and the timed K steps are meant to measure the
steady state.  A background thread samples the GPU's gfx clock and socket power (amdsmi) throughout;
each configuration reports the samples of its timed steps and of its steady state (the last second
of the ramp through the timed steps).

FLOP convention: 4*B*H*N^2*d for the forward, halved when causal; the backward counts 2.5x the
forward.  Kernel times come from HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # twice the bf16 rate (MI355X dense fp8: 5.0 PFLOP/s)
PEAK_HBM_GBS = 8000.0
# The pages' own figure for the fa3 workload: FlashAttention v3's forward at 3.538 ms on an H100
# (FP16), i.e. 661.0 TFLOP/s in the same convention ("GPU Programming and Kernel Optimization",
# item 61; "digest_existing.txt", answer q03_fa3).  Another machine: context, not a target.
PAGES_FA3_TFLOPS = 661.0
DEFAULT_SET = ["c1", "c2", "c3", "c4", "c5"]


def fwd_flop(B, H, N, d, causal) -> float:
    """Forward FLOP by the convention: 4*B*H*N^2*d, halved when causal."""
    return 4.0 * B * H * N * N * d * (0.5 if causal else 1.0)


def step_flop(B, H, N, d, causal, backward) -> float:
    return fwd_flop(B, H, N, d, causal) * (3.5 if backward else 1.0)


def visible_pairs(Nq, Nk, causal) -> int:
    """(query, key) pairs that the mask keeps; causal masks align to the bottom-right corner."""
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    return sum(min(Nk, max(0, i + off + 1)) for i in range(Nq))


def workload_fwd_flop(w) -> float:
    """Forward FLOP of a workload: the convention for equal lengths, 4*d per visible pair otherwise
    (both count query heads, so grouped K/V heads change nothing)."""
    if w.nq == w.nk:
        return fwd_flop(w.B, w.H, w.N, w.d, w.causal)
    return 4.0 * w.B * w.H * w.d * visible_pairs(w.nq, w.nk, w.causal)


def workload_flop(w) -> float:
    """FLOP of one step: the forward, times 3.5 with the backward (which counts 2.5x)."""
    return workload_fwd_flop(w) * (3.5 if w.backward else 1.0)


def kernel_algorithmic_flop(kernel, w) -> float:
    """Algorithmic FLOP one launch performs, in units of one Nq x Nk x d product (the
    forward is two of them): fwd 2 (QK^T, PV); dkdv 4 (the recomputed S, dP, dV, dK);
    dq 1 (dQ; its recomputed S and dP are counted in dkdv); preprocess 0 (the step entry point
    attn_bwd_preprocess); bwd 5 (the two backward kernels of one attn_bwd_qk call, timed
    together)."""
    unit = workload_fwd_flop(w) / 2.0
    return unit * {"fwd": 2, "fwd_fp8": 2, "dkdv": 4, "dq": 1, "preprocess": 0, "bwd": 5}[kernel]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None when the
    kernel sources changed since the counters were taken.  The split-key forward is two
    launches (pieces, then their merge): its traffic is their sum.  With few query rows per head
    the pieces come from the decoding kernel (fwd_decode), else from the forward kernel (fwd)."""
    if kernel == "fwd_splitkv":
        pieces = "fwd_decode" if os.path.exists(os.path.join(ROOT, "profiles", "hbm_traffic_fwd_decode_%s.txt" % workload)) else "fwd"
        parts = [stored_traffic(pieces, workload), stored_traffic("combine", workload)]
        return None if None in parts else sum(parts)
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    try:
        rec = json.loads(open(path).read().split("JSON:", 1)[1].strip().splitlines()[0])
    except Exception:
        return None
    from tiled_online_softmax_02_amd.profiling import kernel_source_sha
    if rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


class HipTimer:
    """HIP events recorded on the launch stream, created with hipEventDisableSystemFence: the
    events only time the kernels between them, so recording one needs no system-scope fence (a
    cache write-back and invalidate that torch.cuda.Event's default events perform, which slowed
    the step by about 2%).  The runtime is the libamdhip64 that torch already loaded (the
    attention library resolves to the same one)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch
        self.ct = ctypes
        # the runtime torch loaded (dlopen of the same file returns the loaded library)
        bundled = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(bundled if os.path.exists(bundled) else "libamdhip64.so.7")
        P, U = ctypes.c_void_p, ctypes.c_uint
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), U]
        self.hip.hipEventRecord.argtypes = [P, P]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.hip.hipEventDestroy.argtypes = [P]
        for f in (self.hip.hipEventCreateWithFlags, self.hip.hipEventRecord, self.hip.hipEventElapsedTime,
                  self.hip.hipEventDestroy):
            f.restype = ctypes.c_int
        self.events = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError("%s failed with hipError_t %d" % (what, rc))

    def new(self):
        ev = self.ct.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE), "hipEventCreateWithFlags")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        self._check(self.hip.hipEventRecord(ev, stream), "hipEventRecord")

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b), "hipEventElapsedTime")
        return ms.value

    def runtime_versions(self) -> dict:
        v, dv = self.ct.c_int(), self.ct.c_int()
        out = {}
        if self.hip.hipRuntimeGetVersion(self.ct.byref(v)) == 0:
            out["hip_runtime_version"] = v.value
        if self.hip.hipDriverGetVersion(self.ct.byref(dv)) == 0:
            out["hip_driver_version"] = dv.value
        return out

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


class GpuMonitor:
    """The GPU's gfx clock (mean over its XCDs) and socket power, sampled every `period` seconds by a
    background thread through amdsmi (read-only sensor queries).  If amdsmi is unavailable the
    monitor records why and every window reports None."""

    def __init__(self, period: float = 0.02):
        self.period = period
        self.samples = []  # (perf_counter time, clock MHz, power W)
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                raise RuntimeError("no GPU handle")
            self._amdsmi, self._h = amdsmi, handles[0]
            self._read()  # fail early if the metrics table is not readable
        except Exception as e:  # noqa: BLE001 - any failure only disables the monitor
            self.error = "%s: %s" % (type(e).__name__, e)

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        clks = m.get("current_gfxclks")
        vals = [c for c in (clks if isinstance(clks, (list, tuple)) else []) if isinstance(c, (int, float)) and 0 < c < 10000]
        if not vals:
            c = m.get("current_gfxclk", m.get("average_gfxclk_frequency"))
            vals = [c] if isinstance(c, (int, float)) and 0 < c < 10000 else []
        p = m.get("current_socket_power", m.get("average_socket_power"))
        power = p if isinstance(p, (int, float)) and 0 < p < 5000 else None
        return (sum(vals) / len(vals) if vals else None), power

    def _run(self):
        while not self._stop.is_set():
            try:
                clk, pw = self._read()
                self.samples.append((time.perf_counter(), clk, pw))
            except Exception as e:  # noqa: BLE001
                self.error = "%s: %s" % (type(e).__name__, e)
                return
            self._stop.wait(self.period)

    def start(self):
        if self.error is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def window(self, t0: float, t1: float) -> dict:
        """Median clock and power of the samples taken in [t0, t1]."""
        sel = [s for s in self.samples if t0 <= s[0] <= t1]
        clk = sorted(s[1] for s in sel if s[1] is not None)
        pw = sorted(s[2] for s in sel if s[2] is not None)
        return {"gfx_clock_mhz_median": clk[len(clk) // 2] if clk else None,
                "gfx_clock_mhz_min": clk[0] if clk else None, "gfx_clock_mhz_max": clk[-1] if clk else None,
                "socket_power_w_median": pw[len(pw) // 2] if pw else None, "samples": len(sel),
                "error": self.error}


def host_cpu() -> dict:
    """CPU model and logical core count of the host the oracle runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def device_info(timer) -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    out = {"name": p.name, "gfx_arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "memory_gib": round(p.total_memory / 2 ** 30, 1), "torch_hip_version": torch.version.hip,
           "torch_version": torch.__version__}
    out.update(timer.runtime_versions())
    return out


def oracle_threads() -> int:
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _parallel(fn, items, threads):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def cpu_baseline(w, inp, gpu, budget_s: float) -> dict:
    """The fp64 CPU oracle timed on a bounded sample of the workload's own inputs, and the largest
    error of the GPU's result on that sample.

    Backward workloads: whole heads (forward by the plain C definition, one thread per head, then
    the backward by fp64 numpy matmuls), as many as fit the budget.  Forward-only workloads: every
    row of the first heads when they are small, else sampled rows (every 64th row, which the
    long-sequence workload scales by 8, plus evenly spaced ones) of sampled heads, by the per-row
    definition, rows split over the threads.  The rate is the sample's FLOP (same convention) over
    the oracle's wall time; `cores` is the number of threads it used."""
    import numpy as np
    import torch
    import oracle

    threads = oracle_threads()
    if w.fp8:
        return cpu_baseline_fp8(w, budget_s, threads)

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    err = {}
    if w.backward:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        # one head first, to size the sample
        b0, h0 = heads[0]

        def bwd_head(bh):
            b, h = bh
            sl = (slice(b, b + 1), slice(h, h + 1))
            G = w.H // w.hk
            q, do = f64(inp["q"][sl]), f64(inp["do"][sl])
            k = f64(inp["k"][b:b + 1, h // G:h // G + 1])
            v = f64(inp["v"][b:b + 1, h // G:h // G + 1])
            o, lse = oracle.attn_fwd(q, k, v, w.causal, w.scale, nthreads=1)
            dq, dk, dv, _ = oracle.attn_bwd_matmul(q, k, v, do, w.causal, w.scale)
            return bh, o, lse, dq, dk, dv

        t0 = time.perf_counter()
        first = bwd_head((b0, h0))
        one = time.perf_counter() - t0
        # the timed sample: the next heads, as many as the threads finish within the budget
        n = int(max(1, min(len(heads) - 1, threads * max(1, int(budget_s // max(one, 1e-3))))))
        sample = heads[1:1 + n]
        t0 = time.perf_counter()
        res = _parallel(bwd_head, sample, min(threads, n)) if sample else []
        dt = time.perf_counter() - t0
        if not sample:  # a single head: the sizing run is the sample
            res, dt, n = [first], one, 1
        else:
            res = [first] + res
        flop = workload_flop(w) / (w.B * w.H) * n
        G = w.H // w.hk
        for bh, o, lse, dq, dk, dv in res:
            b, h = bh
            sl = (slice(b, b + 1), slice(h, h + 1))
            pairs = [("O", gpu["o"][sl], o), ("dQ", gpu["dq"][sl], dq)]
            if G == 1:  # a K/V head's gradient is one query head's only without grouping
                pairs += [("dK", gpu["dk"][sl], dk), ("dV", gpu["dv"][sl], dv)]
            for name, g, r in pairs:
                err[name] = max(err.get(name, 0.0), float(np.abs(f64(g) - r).max()))
            rel = np.abs(f64(gpu["lse"][sl]) - lse) / np.abs(lse)
            err["lse_rel"] = max(err.get("lse_rel", 0.0), float(rel.max()))
        desc = ("%d of %d heads timed, all rows (Nq=%d Nk=%d d=%d), the workload's own inputs; forward by the plain "
                "fp64 C definition (one thread per head), backward by fp64 numpy matmuls; %.1f s wall; errors over "
                "those heads and one more" % (n, w.B * w.H, w.nq, w.nk, w.d, dt))
        cores = min(threads, n)
    else:
        G = w.H // w.hk
        small = w.nq * w.nk <= 4096 * 4096 // 4
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        step = max(1, len(heads) // 4)
        heads = heads[::step][:4]
        if small:
            rows = np.arange(w.nq)
        else:
            rows = np.unique(np.concatenate([np.arange(0, w.nq, 64), np.linspace(0, w.nq - 1, 193).astype(np.int64)]))
        # visible keys per row (same convention as the FLOP count), for the sample's FLOP
        off = w.nk - w.nq
        keys = np.minimum(w.nk, np.maximum(0, rows + off + 1)) if w.causal else np.full(rows.shape, w.nk)
        chunks = [rows[i::threads] for i in range(min(threads, len(rows)))]
        work = [(bh, c) for bh in heads for c in chunks]
        cache = {}
        for (b, h) in heads:
            cache[(b, h)] = (f64(inp["q"][b, h]), f64(inp["k"][b, h // G]), f64(inp["v"][b, h // G]))

        def fwd_rows(item):
            (b, h), rs = item
            q, k, v = cache[(b, h)]
            o, lse = oracle.attn_fwd_rows(q[rs], rs, k, v, w.nq, w.causal, w.scale)
            return (b, h), rs, o, lse

        t0 = time.perf_counter()
        res = _parallel(fwd_rows, work, threads)
        dt = time.perf_counter() - t0
        flop = 4.0 * w.d * float(keys.sum()) * len(heads)
        o_gpu = {bh: f64(gpu["o"][bh[0], bh[1]]) for bh in heads}
        l_gpu = {bh: f64(gpu["lse"][bh[0], bh[1]]) for bh in heads}
        for bh, rs, o, lse in res:
            err["O"] = max(err.get("O", 0.0), float(np.abs(o_gpu[bh][rs] - o).max()))
            err["lse_rel"] = max(err.get("lse_rel", 0.0), float((np.abs(l_gpu[bh][rs] - lse) / np.abs(lse)).max()))
        desc = ("%d of %d heads, %s of %d rows (Nq=%d Nk=%d d=%d), the workload's own inputs; per-row fp64 C "
                "definition, rows split over %d threads; %.1f s wall"
                % (len(heads), w.B * w.H, "all" if small else "%d (every 64th plus evenly spaced)" % len(rows), w.nq,
                   w.nq, w.nk, w.d, threads, dt))
        cores = threads
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle", "sample": desc,
            "max_err_vs_oracle": {k: float("%.3e" % v) for k, v in err.items()}}


def cpu_baseline_fp8(w, budget_s: float, threads: int):
    """The oracle's 8-bit forward (decode, scale, fp64 attention) on whole heads."""
    import oracle
    from tiled_online_softmax_02_amd.inputs import make_fp8_inputs

    def run(heads, seed, nthreads):
        x = make_fp8_inputs(1, heads, w.N, w.d, nk=w.nk, seed=seed, boost_every=w.boost_every, boost=w.boost)
        c = {n: x[n + "8"].view(__import__("torch").uint8).numpy() for n in "qkv"}
        ds = [x["descale_" + n].double().numpy() for n in "qkv"]
        t0 = time.perf_counter()
        oracle.attn_fwd_fp8(c["q"], c["k"], c["v"], *ds, w.causal, w.scale, nthreads=nthreads)
        return time.perf_counter() - t0

    one = run(1, w.seed + 1000, 1)
    heads = int(max(1, min(w.B * w.H, threads, budget_s // max(one, 1e-3))))
    dt = run(heads, w.seed + 1001, min(threads, heads))
    flop = workload_flop(w) / (w.B * w.H) * heads
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": min(threads, heads),
        "kind": "oracle",
        "sample": "%d of %d heads (Nq=%d Nk=%d d=%d per head), same FLOP convention, %.1f s wall; e4m3 codes "
                  "decoded and scaled, then the plain fp64 C definition (one thread per head)"
                  % (heads, w.B * w.H, w.nq, w.nk, w.d, dt),
    }


def inputs_digest(inp: dict) -> str:
    from tiled_online_softmax_02_amd.inputs import inputs_sha256
    return inputs_sha256(inp)


def run_workload(w, args, timer, monitor, dev):
    """Time one workload: ramp, warmup, then args.steps timed steps.  Returns (record, gpu tensors)."""
    import torch
    import tiled_online_softmax_02_amd as A
    from tiled_online_softmax_02_amd.inputs import workload_inputs

    inp = workload_inputs(w)
    digest = inputs_digest(inp)
    fp8 = w.fp8
    if fp8:
        q, k, v = (inp[n + "8"].to(dev) for n in ("q", "k", "v"))
        dsq, dsk, dsv = (inp["descale_" + n].to(dev) for n in ("q", "k", "v"))
    else:
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    # grouped heads or unequal lengths: the _qk entry points (the backward's two kernels are
    # then one call and are timed together)
    qk = Hk != H or Nk != N
    split = w.name == "dec"  # decoding: the split-key forward (partial pieces, then their merge)
    if split:
        ns = A.attn_fwd_splitkv_default_splits_qk(B, H, Hk, N, Nk, d)
        ws_bytes = A.attn_fwd_splitkv_workspace_size(B, H, N, d, ns)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    causal, scale = w.causal, w.scale
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if w.backward:
        do = inp["do"].to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)

    bwd_kernels = ["bwd"] if qk else ["dq", "dkdv"]
    kernels = (["fwd_splitkv"] if split else ["fwd_fp8"] if fp8 else ["fwd"]) + (bwd_kernels if w.backward else [])
    ev = {kname: [] for kname in kernels}
    stream = torch.cuda.current_stream(dev).cuda_stream
    pool = [[timer.new() for _ in range(len(kernels) + 1)] for _ in range(args.steps)]

    def step(record):
        e = pool.pop() if record else None
        if record:
            timer.record(e[0], stream)
        if split:
            A.attn_fwd_splitkv(q, k, v, o, lse, B, H, H, N, Nk, d, causal, scale, ns, ws, ws_bytes)
        elif fp8:
            A.attn_fwd_fp8(q, k, v, dsq, dsk, dsv, o, lse, B, H, H, N, Nk, d, causal, scale)
        elif qk:
            A.attn_fwd_qk(q, k, v, o, lse, B, H, Hk, N, Nk, d, causal, scale)
        else:
            A.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale)
        if record:
            timer.record(e[1], stream)
        if w.backward and qk:
            A.attn_bwd_qk(q, k, v, o, do, lse, dq, dk, dv, delta, B, H, Hk, N, Nk, d, causal, scale)
            if record:
                timer.record(e[2], stream)
        elif w.backward:
            A.attn_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, B, H, N, d, causal, scale)
            if record:
                timer.record(e[2], stream)
            A.attn_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, B, H, N, d, causal, scale)
            if record:
                timer.record(e[3], stream)
        if record:
            for i, kname in enumerate(kernels):
                ev[kname].append((e[i], e[i + 1]))

    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_seconds:
        for _ in range(10):
            step(False)
        torch.cuda.synchronize()
    # the GPU's power and clock readings average over a fraction of a second: the steady-state window is
    # the ramp's last second (or half, for short ramps) plus the warmup and timed steps
    t_settled = time.perf_counter() - min(1.0, 0.5 * args.ramp_seconds)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    kernel_ms, kernel_stats = {}, {}
    for kname, pairs in ev.items():
        ts = sorted(timer.elapsed_ms(a, b) for a, b in pairs)
        kernel_ms[kname] = sum(ts) / len(ts)
        kernel_stats[kname] = {"median": round(ts[len(ts) // 2], 4), "min": round(ts[0], 4), "max": round(ts[-1], 4)}
    flop = workload_flop(w)
    value = flop / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS  # the products' own dtype
    dom = max(kernels, key=lambda kname: kernel_ms[kname])
    if split:
        # decoding reads every key and value once and does 4*d FLOP per key: the HBM roof bounds it
        fwd_t = flop / (kernel_ms["fwd_splitkv"] * 1e-3) / 1e12
        alg_bytes = 2 * (2 * B * H * N * d) + 2 * (2 * B * H * Nk * d) + 4 * B * H * N
        achieved = alg_bytes / (kernel_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": stored_traffic(dom, w.name),
                "algorithmic_bytes": alg_bytes, "num_splits": ns}
    else:
        fwd_t = workload_fwd_flop(w) / (kernel_ms[kernels[0]] * 1e-3) / 1e12
        achieved = kernel_algorithmic_flop(dom, w) / (kernel_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": stored_traffic(dom, w.name)}
    config = {"workload": w.describe(), "B": B, "H": H, "N": N, "d": d, "causal": causal,
              "scale": scale, "global_batch": B, "seq_len": N, "parallelism": "single GPU"}
    if Nk != N:
        config["Nk"] = Nk
    if Hk != H:
        config["Hk"] = Hk
    rec = {"value": value, "ms_per_step": ms_per_step, "config": config, "peak": peak, "fwd_tflops": fwd_t,
           "kernel_ms": kernel_ms, "kernel_ms_stats": kernel_stats, "roofline": roof, "fp8": fp8,
           "seed": w.seed, "inputs_sha256": digest,
           "gpu_during_timed_steps": monitor.window(t0, t1),
           "gpu_steady_state": monitor.window(t_settled, t1)}
    if w.backward:
        bwd_ms = sum(kernel_ms[x] for x in bwd_kernels)
        rec["bwd_tflops"] = 2.5 * workload_fwd_flop(w) / (bwd_ms * 1e-3) / 1e12
    gpu = {"o": o, "lse": lse}
    if w.backward:
        gpu.update(dq=dq, dk=dk, dv=dv)
    return rec, gpu, inp


def summary(w, rec, cpu):
    """The per-configuration record of the JSON line."""
    out = {"workload": rec["config"]["workload"], "seed": rec["seed"], "inputs_sha256": rec["inputs_sha256"],
           "kernel_ms_stats": rec["kernel_ms_stats"], "fwd_tflops": round(rec["fwd_tflops"], 2),
           "fwd_pct_of_peak": round(100.0 * rec["fwd_tflops"] / rec["peak"], 2),
           "step_tflops": round(rec["value"], 2), "ms_per_step": round(rec["ms_per_step"], 4),
           "roofline": rec["roofline"], "gpu_during_timed_steps": rec["gpu_during_timed_steps"],
           "gpu_steady_state": rec["gpu_steady_state"]}
    if "bwd_tflops" in rec:
        out["bwd_tflops"] = round(rec["bwd_tflops"], 2)
        out["bwd_pct_of_peak"] = round(100.0 * rec["bwd_tflops"] / rec["peak"], 2)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all", choices=["all", "c1", "c2", "c3", "c4", "c5", "dec", "c3f8", "c4f8",
                                                         "c5g", "c5d256", "c5u", "fa3"])
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline of the headline workload (c5); each "
                         "forward-only configuration takes a fixed row sample")
    ap.add_argument("--ramp-seconds", type=float, default=2.0,
                    help="untimed steps for this long before the warmup steps, so that the GPU clocks "
                         "have left their idle state when timing starts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X and this build has no "
              "multi-GPU code; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_online_softmax_02_amd.inputs import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = DEFAULT_SET if args.workload == "all" else [args.workload]
    headline = "c5" if args.workload == "all" else args.workload

    # A plain copy of known size, outside the timed region: under rocprofv3 --pmc its
    # FETCH_SIZE / WRITE_SIZE calibrate the counters against known bytes.
    cal_src = torch.empty(64 << 20, dtype=torch.int32, device=dev).fill_(1)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    timer = HipTimer()
    monitor = GpuMonitor()
    monitor.start()
    recs = {}
    try:
        for name in names:
            w = WORKLOADS[name]
            rec, gpu, inp = run_workload(w, args, timer, monitor, dev)
            cpu = None
            if not args.no_cpu_baseline:
                budget = args.cpu_budget if name == headline else 3.0
                cpu = cpu_baseline(w, inp, gpu, budget)
                cpu.update(host_cpu())
            recs[name] = (w, rec, cpu)
            del gpu, inp
            torch.cuda.empty_cache()
    finally:
        monitor.stop()
        devinfo = device_info(timer)
        timer.close()

    w, rec, cpu = recs[headline]
    value = rec["value"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rec["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_FA3_TFLOPS, 3) if w.name == "fa3" else None,
        "dtype": "fp8_e4m3" if rec["fp8"] else "bf16",
        "data": "synthetic",
        "config": rec["config"],
        "pct_of_peak": round(100.0 * value / rec["peak"], 2),
        "peak_tflops": rec["peak"],
        "fwd_tflops": round(rec["fwd_tflops"], 2),
        "kernel_ms": {kname: round(t, 4) for kname, t in rec["kernel_ms"].items()},
        "kernel_ms_stats": rec["kernel_ms_stats"],
        "roofline": rec["roofline"],
    }
    if "bwd_tflops" in rec:
        out["bwd_tflops"] = round(rec["bwd_tflops"], 2)
    if w.name == "fa3":
        out["baseline"] = {"value": PAGES_FA3_TFLOPS, "unit": "TFLOP/s", "source": "FlashAttention v3 forward, "
                           "H100 SXM5, FP16, 3.538 ms (the pages' ablation table); another machine and precision"}
    out["cpu_baseline"] = cpu
    if len(names) > 1:
        out["configs"] = {name: summary(wx, rx, cx) for name, (wx, rx, cx) in recs.items()}
    out["device"] = devinfo
    out["gpu_monitor"] = {"source": "amdsmi gpu_metrics (current gfx clocks averaged over XCDs, socket power)",
                          "period_s": monitor.period, "error": monitor.error}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
