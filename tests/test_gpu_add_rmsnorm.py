"""GPU parity of attn_add_rmsnorm (residual add fused with RMSNorm) against
the fp64 oracle.

Tolerance, from the arithmetic: the sum h = x + r of two bf16 values is
exact in fp32 unless their magnitudes differ by more than 2^16 (then it is
within 2^-24 relative), and it is rounded once to bf16, so
|dh| <= (2^-9 + 2^-24) |h|. y is computed in fp32 (the sum of
squares of at most 16384 terms, accumulated in 64-term runs and a 256-way
tree, a relative error ~1e-5; rsqrt and two products a few ulp) and rounded
once to bf16 (2^-9 relative). Both are checked against 2^-8 of the reference
magnitude, element by element, over every element."""

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL = 2.0 ** -8


def check(x, r, w, eps, y, h, what):
    ry, rh = oracle.add_rmsnorm(x, r, w, eps)
    gy = y.float().cpu().double().numpy()
    gh = h.float().cpu().double().numpy()
    assert np.all(np.isfinite(gy)), what
    ey = np.abs(gy - ry) - (REL * np.abs(ry) + 1e-7)
    eh = np.abs(gh - rh) - REL * np.abs(rh)
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
