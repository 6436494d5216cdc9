"""The GPU tests' tolerance helper: its half-ulp must be exactly half the spacing of the
output format (numpy's float16 spacing, torch's bfloat16 neighbours)."""
import numpy as np
import torch

from gpu_helpers import half_ulp, tolerance


def test_half_ulp_f16_matches_numpy_spacing():
    x = np.concatenate([np.geomspace(1e-4, 6e4, 2000), -np.geomspace(1e-4, 6e4, 50)])
    x16 = x.astype(np.float16)
    ref = np.spacing(np.abs(x16)).astype(np.float64) / 2
    got = half_ulp(x16.astype(np.float64), "f16")
    assert np.array_equal(got, ref)


def test_half_ulp_bf16_matches_torch_neighbours():
    x = torch.tensor(np.geomspace(1e-30, 1e30, 3000), dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).to(torch.int32)
    nxt = (bits + 1).to(torch.int16).view(torch.bfloat16)
    ref = (nxt.to(torch.float64) - x.to(torch.float64)).numpy() / 2
    got = half_ulp(x.to(torch.float64).numpy(), "bf16")
    assert np.array_equal(got, ref)


def test_tolerance_is_the_stated_bound_below_the_format_limit():
    x = np.array([0.0, 0.3, 1.0, 1.99, 2.0, 3.5, 100.0])
    t = tolerance(x, "bf16")
    assert (t[:4] == 4e-3).all()
    assert np.allclose(t[4:], [2 ** -7 + 1e-4, 2 ** -7 + 1e-4, 2 ** -2 + 1e-4])
    assert (tolerance(x, "f16")[:6] == 4e-3).all()
    assert (tolerance(x, "f32") == 1e-5).all()
