"""Shared comparison helpers for the GPU parity tests.

Tolerances: bf16 inputs with fp32 accumulation: max abs error <= 2e-2 and
mean abs error <= 2e-3; fp32 path: max abs error <= 1e-4 (the stated bounds
of the build).

lse: the bf16 kernels accumulate the row sum l over the weights after their
rounding to bf16 (the very weights that multiply V), each within a relative
2^-9 of the exact weight, so ln(l) is within 2^-9 of the exact log-sum-exp;
the bound adds 1e-4 for fp32 arithmetic.
"""

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4
LSE_ABS = 2.0 ** -9 + 1e-4


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close(got, ref, dtype, what=""):
    got = to64(got) if torch.is_tensor(got) else np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    if dtype == torch.float32:
        assert mx <= F32_MAX_ABS, f"{what}: max abs err {mx:.3e} > {F32_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{what}: max abs err {mx:.3e} > {BF16_MAX_ABS}"
        assert mean <= BF16_MEAN_ABS, f"{what}: mean abs err {mean:.3e} > {BF16_MEAN_ABS}"
    return mx, mean


def assert_lse_close(got, ref, what=""):
    got = to64(got)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - ref[fin])
    assert err.size == 0 or err.max() <= LSE_ABS, f"{what}: lse max err {err.max():.3e}"
