"""Shared comparison helpers for the GPU parity tests.

Every reference here is the plain oracle on the ORIGINAL inputs; nothing in
this file re-creates a rounding step of the kernels.

Outputs o. bf16 inputs with fp32 accumulation: max abs error <= 2e-2 and mean
abs error <= 2e-3; fp32 path: max abs error <= 1e-4 (the stated bounds).

lse. The bf16 kernels form their scores from bf16(q * c), c = scale *
log2(e): each element of q is multiplied by c in fp32 and rounded to bf16
once (round to nearest even, relative error at most u = 2^-8). So a score
q.k_j moves by at most

    u * scale * sum_i |q_i| |k_ji|            (in natural-log units)

and lse = log sum_j exp(s_j), a softmax-weighted mean of the score moves,
moves by at most the largest of them over the keys the row sees. On top of
that come fp32 effects:
  * the score's fp32 accumulation over d products, and the reference max the
    score MFMA starts from: (d + 1) * 2^-24 relative to the same sum;
  * the row sum (a chain of at most T/16 + 64 fp32 additions, exp2 within
    one ulp, the rescales and the final log): well below 1e-4 for every
    sequence length tested (T/16 * 2^-24 < 1e-4 for T < 2.7e7).
So, per row, |lse - lse_oracle| <= (2^-8 + (d + 1) 2^-24)(1 + 2^-8) * scale
* max_j sum_i |q_i||k_ji| + 1e-4, computed below from the inputs. The fp32
path rounds nothing: its lse is held to 1e-4 outright.
"""

import numpy as np
import torch

import oracle

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4
U_BF16 = 2.0 ** -8          # unit roundoff of bf16 round-to-nearest-even
U_F32 = 2.0 ** -24
LSE_FP32_ABS = 1e-4         # the fp32 row-sum / log part of the lse bound


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def _abs64(x):
    if torch.is_tensor(x):
        return np.abs(x.detach().to("cpu").to(torch.float64).numpy())
    return np.abs(np.asarray(x, dtype=np.float64))


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


def _lse_bound_from_sums(max_abs_dot, scale, d):
    rel = (U_BF16 + (d + 1) * U_F32) * (1.0 + U_BF16)
    return rel * float(scale) * max_abs_dot + LSE_FP32_ABS


def lse_bound_prefill(q, k, scale, causal=True, rows=None, heads=None):
    """Per-row bound on |lse_bf16_kernel - lse_oracle| for attn_prefill, from
    the inputs: shape [B, Hq, R] like the oracle's lse (NaN for heads not
    evaluated). Uses max over the visible keys of sum_i |q_i||k_ji|."""
    aq, ak = _abs64(q), _abs64(k)
    B, Hq, T, d = aq.shape
    G = Hq // ak.shape[1]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    out = np.full((B, Hq, len(rows)), np.nan)
    for b in range(B):
        for h in heads:
            g = h // G
            for r0 in range(0, len(rows), 2048):
                rr = rows[r0:r0 + 2048]
                kv = int(rr.max()) + 1 if causal else T
                A = aq[b, h, rr] @ ak[b, g, :kv].T
                if causal:
                    A = np.where(np.arange(kv)[None, :] > rr[:, None], 0.0, A)
                out[b, h, r0:r0 + len(rr)] = A.max(axis=1)
    return _lse_bound_from_sums(out, scale, d)


def lse_bound_paged(q, k_cache, block_table, seq_lens, scale, query_start_loc=None):
    """Per-(token, head) bound on |lse_kernel - lse_oracle| for
    attn_decode_paged, from the inputs (keys gathered through the table by
    the oracle's own gather; bottom-right causal for q_len > 1)."""
    aq = _abs64(q)
    num_tokens, Hq, d = aq.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    lens = np.asarray(seq_lens.cpu() if torch.is_tensor(seq_lens) else seq_lens, dtype=np.int64)
    table = np.asarray(block_table.cpu() if torch.is_tensor(block_table) else block_table,
                       dtype=np.int64)
    n = len(lens)
    if query_start_loc is None:
        qsl = np.arange(n + 1)
    else:
        qsl = np.asarray(query_start_loc.cpu() if torch.is_tensor(query_start_loc)
                         else query_start_loc, dtype=np.int64)
    out = np.full((num_tokens, Hq), np.nan)
    for s in range(n):
        t0, t1, L = int(qsl[s]), int(qsl[s + 1]), int(lens[s])
        if t1 == t0:
            continue
        if L == 0:
            out[t0:t1] = 0.0
            continue
        K = np.abs(oracle.gather_paged_kv(k_cache, table[s], L))  # [L, Hkv, d]
        pos = L - (t1 - t0) + np.arange(t1 - t0)
        for h in range(Hq):
            A = aq[t0:t1, h] @ K[:, h // G].T
            A = np.where(np.arange(L)[None, :] > pos[:, None], 0.0, A)
            out[t0:t1, h] = A.max(axis=1)
    return _lse_bound_from_sums(out, scale, d)


def assert_lse_close(got, ref, bound, what=""):
    """|got - ref| <= bound element by element (bound: an array of ref's shape
    or a scalar); the -inf pattern must match exactly."""
    got = to64(got)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.broadcast_to(np.asarray(bound, dtype=np.float64), ref.shape)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - ref[fin])
    over = err - bound[fin]
    assert err.size == 0 or over.max() <= 0, (
        f"{what}: lse error {err[over.argmax()]:.3e} over its bound {bound[fin][over.argmax()]:.3e}")
    return float(err.max()) if err.size else 0.0


def ref_prefill(q, k, v, scale, *args, **kw):
    """(o, lse, lse_bound) for a bf16 prefill: the oracle on the inputs and the
    per-row lse bound above."""
    ro, rl = oracle.prefill(q, k, v, scale, *args, **kw)
    causal = kw.get("causal", args[0] if args else True)
    return ro, rl, lse_bound_prefill(q, k, scale, causal=causal, rows=kw.get("rows"),
                                     heads=kw.get("heads"))


def ref_decode(q, k_cache, v_cache, block_table, seq_lens, scale, query_start_loc=None):
    """(o, lse, lse_bound) for a bf16 paged call."""
    ro, rl = oracle.decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale,
                                 query_start_loc=query_start_loc)
    return ro, rl, lse_bound_paged(q, k_cache, block_table, seq_lens, scale, query_start_loc)
