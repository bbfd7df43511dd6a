"""CPU checks of the parity helpers themselves."""

import numpy as np
import torch

from tests.parity_util import bf16_rounding_ok, max_abs_rms, rel_l2


def _heavy_tailed(n, seed):
    rng = np.random.default_rng(seed)
    g, u = rng.standard_normal(n), rng.standard_normal(n)
    return g / (1 + np.exp(-g)) * u * 4  # silu(g) * u, scaled: outliers ~20x rms


def test_bf16_rounding_bound_accepts_round_to_nearest():
    ref = _heavy_tailed(200_000, 1)
    got = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert bf16_rounding_ok(got, ref)


def test_bf16_rounding_bound_rejects_one_ulp_too_far():
    ref = _heavy_tailed(10_000, 2)
    got = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).double().numpy()
    i = int(np.argmax(np.abs(ref)))
    ulp = 2.0 ** (np.floor(np.log2(abs(ref[i]))) - 7)
    bad = got.copy()
    bad[i] += 2 * ulp * np.sign(ref[i])
    assert not bf16_rounding_ok(bad, ref)


def test_rel_l2_and_max_abs_rms_definitions():
    ref = np.array([3.0, -4.0])
    got = np.array([3.0, -4.5])
    assert np.isclose(rel_l2(got, ref), 0.5 / 5.0)
    assert np.isclose(max_abs_rms(got, ref), 0.5 / np.sqrt(12.5))
