"""Shared comparison helpers for the GPU parity tests.

Tolerances: bf16 inputs with fp32 accumulation: max abs error <= 2e-2 and
mean abs error <= 2e-3; fp32 path: max abs error <= 1e-4 (the stated bounds
of the build).

lse: the bf16 kernels form their scores from q * c with c = scale * log2(e),
each element rounded to bf16 once (the softmax scale is folded into the
query), and sum the unrounded fp32 weights. The reference lse is therefore
the oracle's on kernel_q(q) = bf16(q * c) / c, which holds exactly the
scores the kernels form (computed here from the inputs, by that rounding
rule). Against it only fp32 rounding remains; the bound, 2^-9 + 1e-4, is
the one that would hold even for a row sum over the bf16-rounded weights
(each within a relative 2^-9). Outputs o are always compared with the
oracle on the original inputs. The fp32 path rounds nothing and is compared
with the original inputs throughout.
"""

import numpy as np
import torch

import oracle

LOG2E = 1.4426950408889634

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


def kernel_q(q, scale):
    """The query the bf16 kernels form their scores from, in fp64: each bf16
    element times c = fp32(scale) * fp32(log2 e) (an fp32 product), rounded to
    bf16 (nearest even), divided by c again."""
    c = float(np.float32(scale) * np.float32(LOG2E))
    qs = (torch.as_tensor(q).to(torch.float32) * c).to(torch.bfloat16)
    return qs.to(torch.float64) / c


def ref_prefill(q, k, v, scale, *args, **kw):
    """(o, lse) references for a bf16 prefill: o from the oracle on q, lse
    from the oracle on kernel_q(q)."""
    ro, _ = oracle.prefill(q, k, v, scale, *args, **kw)
    _, rl = oracle.prefill(kernel_q(q, scale), k, v, scale, *args, **kw)
    return ro, rl


def ref_decode(q, k_cache, v_cache, block_table, seq_lens, scale, *args, **kw):
    """(o, lse) references for a bf16 paged call: o from the oracle on q, lse
    from the oracle on kernel_q(q)."""
    ro, _ = oracle.decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale, *args, **kw)
    _, rl = oracle.decode_paged(kernel_q(q, scale), k_cache, v_cache, block_table, seq_lens,
                                scale, *args, **kw)
    return ro, rl
