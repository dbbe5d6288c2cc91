"""GPU parity of attn_add_rmsnorm (residual add fused with RMSNorm) against
the fp64 oracle.

Tolerance, from the arithmetic (u = 2^-8 is the unit roundoff of bf16
round-to-nearest-even: a rounded value lies within u of the value rounded,
relatively):
  * h = x + r of two bf16 values is formed in fp32 (exact unless their
    magnitudes differ by more than 2^16, then within 2^-24 relative) and
    rounded once to bf16: |dh| <= (u + 2^-24)(1 + 2^-24) |h| < (u + 2^-22)|h|.
  * y is computed in fp32 from the unrounded sum: the sum of squares of at
    most 16384 terms (chains of at most 64 additions per thread, then a
    256-way tree: a relative error below 72 * 2^-24 ~ 4.3e-6), the mean, eps,
    the reciprocal square root (about 1 ulp) and two products: below 1e-5
    relative in all, so below 5e-6 on y after the square root. y is then
    rounded once to bf16: |dy| <= u (1 + 1e-5)|y| + 1e-5 |y| < (u + 2^-16)|y|.
Both are checked element by element, over every element; y also gets 1e-30
of absolute slack for rows whose reference is exactly 0."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_H = 2.0 ** -8 + 2.0 ** -22
REL_Y = 2.0 ** -8 + 2.0 ** -16


def check(x, r, w, eps, y, h, what):
    ry, rh = oracle.add_rmsnorm(x, r, w, eps)
    gy = y.float().cpu().double().numpy()
    gh = h.float().cpu().double().numpy()
    assert np.all(np.isfinite(gy)), what
    ey = np.abs(gy - ry) - (REL_Y * np.abs(ry) + 1e-30)
    eh = np.abs(gh - rh) - REL_H * np.abs(rh)
    assert ey.max() <= 0, f"{what}: y off by {ey.max():.3e} beyond the bound"
    assert eh.max() <= 0, f"{what}: h off by {eh.max():.3e} beyond the bound"


@pytest.mark.parametrize("rows,hidden,eps,seed", [
    (1, 8, 1e-6, 120), (3, 64, 1e-5, 121), (7, 2048, 1e-6, 122), (5, 2056, 1e-6, 123),
    (16, 4096, 1e-6, 124), (4, 8192, 0.0, 125), (2, 16384, 1e-6, 126), (33, 4104, 1e-2, 127),
])
def test_add_rmsnorm_matches_oracle(rows, hidden, eps, seed):
    print(f"[rmsnorm] rows={rows} hidden={hidden}", flush=True)
    x, r, w = inputs.norm_inputs(rows, hidden, seed)
    y, h = attn.add_rmsnorm(x.to(DEV), r.to(DEV), w.to(DEV), eps)
    torch.cuda.synchronize()
    check(x, r, w, eps, y, h, f"rows={rows} hidden={hidden}")


def test_add_rmsnorm_in_place_residual():
    print("[rmsnorm] in place", flush=True)
    x, r, w = inputs.norm_inputs(64, 4096, 128)
    rd = r.to(DEV)
    y, h = attn.add_rmsnorm(x.to(DEV), rd, w.to(DEV), 1e-6, residual_out=rd)
    torch.cuda.synchronize()
    assert h.data_ptr() == rd.data_ptr()
    check(x, r, w, 1e-6, y, h, "in place")


def test_add_rmsnorm_full_size():
    # the benchmarked shape: 4096 rows of hidden 4096 (a 4096-token chunk of a
    # 32-head x 128 model), every element against the oracle
    print("[rmsnorm] 4096 x 4096", flush=True)
    x, r, w = inputs.norm_inputs(4096, 4096, 129, device=DEV)
    y, h = attn.add_rmsnorm(x, r, w, 1e-6)
    torch.cuda.synchronize()
    check(x.cpu(), r.cpu(), w.cpu(), 1e-6, y, h, "4096 x 4096")


def test_add_rmsnorm_rejects_bad_requests_on_the_host():
    x, r, w = inputs.norm_inputs(2, 64, 130, device=DEV)
    with pytest.raises(attn.AttnError) as e:
        attn.add_rmsnorm(x.float(), r.float(), w.float(), 1e-6)
    assert e.value.name == "ATTN_ERR_UNSUPPORTED"
    with pytest.raises(attn.AttnError) as e:  # output aliasing an input
        attn.add_rmsnorm(x, r, w, 1e-6, out=x)
    assert e.value.name == "ATTN_ERR_SHAPE"
