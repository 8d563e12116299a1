#!/usr/bin/env python3
"""Benchmark: attention forward + backward throughput on one MI355X.

One step is one pass of the whole path over resident synthetic inputs: the fused
forward kernel, then the two launches attn_bwd makes (the dQ kernel, which also forms
D = rowsum(dO o O), then the dK/dV kernel).  The default
workload is the forward+backward causal case
B=2, H=16, N=4096, d=128; ``--workload c2|c3|c4`` times forward-only workloads, ``dec`` the
split-key forward of a decoding shape, and ``c3f8|c4f8`` the 8-bit forward on the shapes of
c3 and c4.

Before the W warmup steps the step runs untimed for --ramp-seconds (1 s by default): an
idle MI355X needs a fraction of a second under load before its clocks settle, and the timed
K steps are meant to measure the steady state.

FLOP convention: 4*B*H*N^2*d for the forward, halved when causal; the backward counts
2.5x the forward.  Printed: one JSON line with the whole-job TFLOP/s, the dominant
kernel's roofline (achieved algorithmic TFLOP/s against the dense MFMA peak of its dtype,
measured with HIP events on the launch stream) and the fp64 CPU oracle timed on a
bounded sample of the same workload on the host cores.
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

METRIC = "attention fwd/bwd TFLOP/s on 1 MI355X and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # twice the bf16 rate (MI355X dense fp8: 5.0 PFLOP/s)
PEAK_HBM_GBS = 8000.0
# The pages' own figure for the fa3 workload: FlashAttention v3's forward at 3.538 ms on an H100
# (FP16), i.e. 661.0 TFLOP/s in the same convention ("GPU Programming and Kernel Optimization",
# item 61; "digest_existing.txt", answer q03_fa3).  Another machine: context, not a target.
PAGES_FA3_TFLOPS = 661.0


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
    launches (pieces, then their merge): its traffic is their sum."""
    if kernel == "fwd_splitkv":
        parts = [stored_traffic("fwd", workload), stored_traffic("combine", workload)]
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

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


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


def cpu_baseline(w, budget_s: float):
    """Time the fp64 CPU oracle on whole heads of the workload until ~budget_s of work."""
    import numpy as np
    import oracle
    from tiled_online_softmax_02_amd.inputs import make_inputs

    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    if w.fp8:
        return cpu_baseline_fp8(w, budget_s, threads)
    inp = make_inputs(1, 1, w.N, w.d, nk=w.nk, seed=w.seed + 1000, backward=w.backward,
                      boost_every=w.boost_every, boost=w.boost)
    f64 = {k: t.to(dtype=__import__("torch").float64).numpy() for k, t in inp.items()}
    # one head first, to size the sample
    t0 = time.perf_counter()
    oracle.attn_fwd(f64["q"], f64["k"], f64["v"], w.causal, w.scale, nthreads=1)
    if w.backward:
        oracle.attn_bwd_matmul(f64["q"], f64["k"], f64["v"], f64["do"], w.causal, w.scale)
    one = time.perf_counter() - t0
    heads = int(max(1, min(w.B * w.H, threads, budget_s // max(one, 1e-3))))
    inp = make_inputs(1, heads, w.N, w.d, nk=w.nk, seed=w.seed + 1001, backward=w.backward,
                      boost_every=w.boost_every, boost=w.boost)
    f64 = {k: t.to(dtype=__import__("torch").float64).numpy() for k, t in inp.items()}
    t0 = time.perf_counter()
    oracle.attn_fwd(f64["q"], f64["k"], f64["v"], w.causal, w.scale, nthreads=min(threads, heads))
    if w.backward:
        oracle.attn_bwd_matmul(f64["q"], f64["k"], f64["v"], f64["do"], w.causal, w.scale)
    dt = time.perf_counter() - t0
    flop = workload_flop(w) / (w.B * w.H) * heads
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": min(threads, heads) if not w.backward else threads,
        "kind": "oracle",
        "sample": "%d of %d heads (%s per head), same FLOP convention, %.1f s wall; forward by the plain "
                  "fp64 C definition (one thread per head), backward by fp64 numpy matmuls"
                  % (heads, w.B * w.H, "Nq=%d Nk=%d d=%d" % (w.nq, w.nk, w.d), dt),
    }


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", choices=["c2", "c3", "c4", "c5", "dec", "c3f8", "c4f8", "c5g", "c5d256", "c5u",
                                                        "fa3"])
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--ramp-seconds", type=float, default=1.0,
                    help="untimed steps for this long before the warmup steps, so that the GPU clocks "
                         "have left their idle state when timing starts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X and this build has no "
              "multi-GPU code; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_online_softmax_02_amd as A
    from tiled_online_softmax_02_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workload_inputs(w)
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
        ns = A.attn_fwd_splitkv_default_splits(B, H, N, Nk, d)
        ws_bytes = A.attn_fwd_splitkv_workspace_size(B, H, N, d, ns)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    causal, scale = w.causal, w.scale
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if w.backward:
        do = inp["do"].to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)

    # A plain copy of known size, outside the timed region: under rocprofv3 --pmc its
    # FETCH_SIZE / WRITE_SIZE calibrate the counters against known bytes.
    cal_src = torch.empty(64 << 20, dtype=torch.int32, device=dev).fill_(1)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    # the backward kernels in attn_bwd's order: dQ first, forming D of its rows on the way
    # (attn_bwd_dq_delta), then dK/dV
    bwd_kernels = ["bwd"] if qk else ["dq", "dkdv"]
    kernels = (["fwd_splitkv"] if split else ["fwd_fp8"] if fp8 else ["fwd"]) + (bwd_kernels if w.backward else [])
    ev = {kname: [] for kname in kernels}

    # HIP events for the timed steps, created before timing starts; recorded on the stream the
    # library launches on (torch's current stream, which the binding passes)
    timer = HipTimer()
    stream = torch.cuda.current_stream(dev).cuda_stream
    pool = [[timer.new() for _ in range(len(kernels) + 1)] for _ in range(args.steps)]

    class _Ev:
        def __init__(self, h):
            self.h = h

        def record(self):
            timer.record(self.h, stream)

        def elapsed_time(self, other):
            return timer.elapsed_ms(self.h, other.h)

    def step(record):
        e = [_Ev(h) for h in pool.pop()] if record else None
        if record:
            e[0].record()
        if split:
            A.attn_fwd_splitkv(q, k, v, o, lse, B, H, H, N, Nk, d, causal, scale, ns, ws, ws_bytes)
        elif fp8:
            A.attn_fwd_fp8(q, k, v, dsq, dsk, dsv, o, lse, B, H, H, N, Nk, d, causal, scale)
        elif qk:
            A.attn_fwd_qk(q, k, v, o, lse, B, H, Hk, N, Nk, d, causal, scale)
        else:
            A.attn_fwd(q, k, v, o, lse, B, H, N, d, causal, scale)
        if record:
            e[1].record()
        if w.backward and qk:
            A.attn_bwd_qk(q, k, v, o, do, lse, dq, dk, dv, delta, B, H, Hk, N, Nk, d, causal, scale)
            if record:
                e[2].record()
        elif w.backward:
            A.attn_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, B, H, N, d, causal, scale)
            if record:
                e[2].record()
            A.attn_bwd_dkdv(q, k, v, do, lse, delta, dk, dv, B, H, N, d, causal, scale)
            if record:
                e[3].record()
        if record:
            for i, kname in enumerate(kernels):
                ev[kname].append((e[i], e[i + 1]))

    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < args.ramp_seconds:
        for _ in range(10):
            step(False)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps

    kernel_ms = {kname: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) for kname, pairs in ev.items()}
    kernel_stats = {}
    for kname, pairs in ev.items():
        ts = sorted(a.elapsed_time(b) for a, b in pairs)
        kernel_stats[kname] = {"median": round(ts[len(ts) // 2], 4), "min": round(ts[0], 4), "max": round(ts[-1], 4)}
    timer.close()
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
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_FA3_TFLOPS, 3) if w.name == "fa3" else None,
        "dtype": "fp8_e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100.0 * value / peak, 2),
        "peak_tflops": peak,
        "fwd_tflops": round(fwd_t, 2),
        "kernel_ms": {kname: round(t, 4) for kname, t in kernel_ms.items()},
        "kernel_ms_stats": kernel_stats,
        "roofline": roof,
    }
    if w.name == "fa3":
        out["baseline"] = {"value": PAGES_FA3_TFLOPS, "unit": "TFLOP/s", "source": "FlashAttention v3 forward, "
                           "H100 SXM5, FP16, 3.538 ms (the pages' ablation table); another machine and precision"}
    if w.backward:
        bwd_ms = sum(kernel_ms[x] for x in bwd_kernels)
        out["bwd_tflops"] = round(2.5 * workload_fwd_flop(w) / (bwd_ms * 1e-3) / 1e12, 2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
        out["cpu_baseline"].update(host_cpu())
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
