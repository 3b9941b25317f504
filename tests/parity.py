"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle,
compare. Tolerances for bf16 inputs with fp32 accumulation: max-abs 2e-2 and
mean-abs 2e-3 over every compared element of O (and dQ, dK, dV); LSE, computed
in fp32 from the same bf16 inputs, within 1e-3."""
import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def to64(t):
    return t.detach().float().cpu().double().numpy()


def assert_close(got, want, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mean <= mean_abs, f"{what}: max-abs {mx:.3g}, mean-abs {mean:.3g}"
    return mx, mean


def device():
    return torch.device("cuda", 0)
