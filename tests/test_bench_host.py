"""Host-side logic of bench.py (no GPU): the FLOP convention and the multi-GPU refusal."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_flop_convention_reproduces_the_pages_throughputs():
    with open(os.path.join(ROOT, "tests", "golden", "flop_convention.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        tflops = bench.fwd_flop(c["B"], c["H"], c["N"], c["d"], c["causal"]) / (c["ms"] * 1e-3) / 1e12
        # the printed figures carry 3-4 significant digits
        assert tflops == pytest.approx(c["tflops"], rel=3e-3), c


def test_causal_halves_and_backward_is_two_and_a_half_forwards():
    f = bench.fwd_flop(2, 16, 4096, 128, False)
    assert bench.fwd_flop(2, 16, 4096, 128, True) == f / 2
    assert bench.step_flop(2, 16, 4096, 128, True, True) == pytest.approx(3.5 * f / 2)
    # per-kernel algorithmic counts add up to the whole step, and so does the backward timed as one
    from tiled_online_softmax_02_amd.inputs import WORKLOADS
    c5 = WORKLOADS["c5"]
    parts = sum(bench.kernel_algorithmic_flop(k, c5) for k in ("fwd", "preprocess", "dkdv", "dq"))
    assert parts == pytest.approx(bench.step_flop(2, 16, 4096, 128, True, True))
    assert bench.kernel_algorithmic_flop("fwd", c5) + bench.kernel_algorithmic_flop("bwd", c5) == pytest.approx(parts)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_visible_pairs_bottom_right_alignment():
    # non-causal: every pair; causal with equal lengths: the lower triangle with its diagonal
    assert bench.visible_pairs(7, 5, False) == 35
    assert bench.visible_pairs(6, 6, True) == 21
    # five queries, two keys: the first three queries see nothing, then 1 and 2 keys
    assert bench.visible_pairs(5, 2, True) == 3
    # one query against many keys sees all of them
    assert bench.visible_pairs(1, 16384, True) == 16384
    # more keys than queries: query i sees i + (Nk - Nq) + 1 keys
    assert bench.visible_pairs(3, 10, True) == 8 + 9 + 10


def test_decoding_workload_flop():
    from tiled_online_softmax_02_amd.inputs import WORKLOADS
    w = WORKLOADS["dec"]
    assert (w.nq, w.nk) == (1, 65536)
    assert bench.workload_flop(w) == 4.0 * w.B * w.H * w.d * 65536
    # the equal-length workloads keep the convention
    c5 = WORKLOADS["c5"]
    assert bench.workload_flop(c5) == bench.step_flop(2, 16, 4096, 128, True, True)


def test_widened_workloads_flop():
    from tiled_online_softmax_02_amd.inputs import WORKLOADS
    # grouped heads: FLOP count query heads, the same as c5
    assert bench.workload_flop(WORKLOADS["c5g"]) == bench.workload_flop(WORKLOADS["c5"])
    # 2048 queries against 4096 keys, causal bottom-right: query i sees 2048 + i + 1 keys
    w = WORKLOADS["c5u"]
    pairs = sum(2048 + i + 1 for i in range(2048))
    assert bench.workload_flop(w) == pytest.approx(3.5 * 4.0 * 2 * 16 * 128 * pairs)
    assert bench.workload_flop(WORKLOADS["c5d256"]) == bench.step_flop(2, 16, 4096, 256, True, True)


def test_gpu_monitor_reports_why_it_has_no_samples():
    """Without a readable GPU (this host) the clock and power monitor stays silent and says why."""
    m = bench.GpuMonitor(period=0.01)
    m.start()
    m.stop()
    w = m.window(0.0, 1e12)
    if m.error is not None:
        assert w["samples"] == 0 and w["gfx_clock_mhz_median"] is None and w["error"] == m.error
    else:  # a GPU host: the sampled clocks are plausible
        assert w["gfx_clock_mhz_median"] is None or 100 < w["gfx_clock_mhz_median"] < 5000
