"""The bf16 rounding the GPU parity tests compare against: nearest-even rounding to 8 significant bits,
checked against PyTorch's float32 -> bfloat16 conversion, and half-ulp spacings at known points."""
import numpy as np
import torch

from parity_util import bf16_half_ulp, bf16_round, grad_bound


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-3, 1.0, 7.0, 300.0)]).astype(np.float32)
    # values halfway between bf16 neighbours, where the tie goes to the even one
    ties = (np.arange(-4096, 4096, dtype=np.int64) * 2 + 1).astype(np.float32) * np.float32(2.0 ** -8)
    x = np.concatenate([x, ties, np.array([0.0, 1.0, -2.5, 8.0, 255.5], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), want)


def test_bf16_half_ulp():
    x = np.array([1.0, 1.99, 2.0, 3.9, 4.0, 7.99, 8.0, 15.0, -4.5, 0.5, 0.0])
    want = np.array([2 ** -8, 2 ** -8, 2 ** -7, 2 ** -7, 2 ** -6, 2 ** -6, 2 ** -5, 2 ** -5, 2 ** -6, 2 ** -9, 0.0])
    assert np.array_equal(bf16_half_ulp(x), want)
    # every finite value is within half an ulp of its rounding
    rng = np.random.default_rng(1)
    y = rng.standard_normal(10000) * 20
    assert np.all(np.abs(bf16_round(y) - y) <= bf16_half_ulp(y))


def test_grad_bound_adds_rounding_only_from_four():
    ref = np.array([0.5, 3.9, 4.0, 7.9, 8.0, -12.0])
    want = np.array([2e-2, 2e-2, 2e-2 + 2 ** -6, 2e-2 + 2 ** -6, 2e-2 + 2 ** -5, 2e-2 + 2 ** -5])
    assert np.array_equal(grad_bound(ref), want)
