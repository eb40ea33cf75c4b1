"""The rounding helpers behind the GPU parity gates, checked on the CPU
against torch's own float64 -> bfloat16 conversion (round to nearest even)."""
import numpy as np
import torch

from tests import _gpu_util as U


def _samples():
    rng = np.random.default_rng(17)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, size=20000))
    # exact bf16 values, and the midpoints between neighbours (ties)
    bt = torch.from_numpy(x).to(torch.bfloat16)
    b = bt.double().numpy()
    # the neighbouring bf16 number one step further from zero (bit pattern + 1)
    nb = (bt.view(torch.int16) + 1).view(torch.bfloat16).double().numpy()
    mids = (b + nb) / 2
    return np.concatenate([x, b, mids, [0.0, 1.0, -4.0, 4.0, 7.99, 8.0]])


def test_bf16_rne_matches_torch():
    x = _samples()
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(U.bf16_rne_from_f64(x), ref)


def test_bf16_half_ulp_bounds_the_rounding_error_and_is_reached():
    x = _samples()
    err = np.abs(U.bf16_rne_from_f64(x) - x)
    half = U.bf16_half_ulp(x)
    assert np.all(err <= half)
    # the bound is tight: ties between neighbours sit exactly half an ulp away
    assert np.any((err == half) & (half > 0))
    # 4 .. 8: 8 significant bits leave a spacing of 2^-5
    assert U.bf16_half_ulp(np.array([4.0, 5.5, 7.99]))[0] == 2.0 ** -6
    assert U.bf16_half_ulp(np.array([0.0]))[0] == 0.0
