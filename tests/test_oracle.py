"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-worked example, a
closed form, an invariant of the definition, brute force on tiny inputs, or a
library routine for a special case. Together they are chosen so that a
plausible slip in the oracle (a dropped scale, a wrong mask direction, a
transposed operand, a wrong GQA head map, an off-by-one in the block-table
translation) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_tiled_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(20261202)


# ----------------------------------------------------------------------------
# brute force: the definition with pure-Python loops and math.exp
# ("Hugging Face attention profiling guide", second paragraph)
# ----------------------------------------------------------------------------

def brute_attention_row(qrow, keys, vals, scale, last_key):
    """One query row: scores, scale, mask keys after last_key, softmax, @ V."""
    s = []
    for j, krow in enumerate(keys):
        if last_key is not None and j > last_key:
            s.append(-math.inf)
        else:
            s.append(scale * sum(a * b for a, b in zip(qrow, krow)))
    m = max(s)
    if m == -math.inf:
        return [0.0] * len(vals[0]), -math.inf
    w = [math.exp(x - m) for x in s]
    tot = sum(w)
    out = [sum(w[j] / tot * vals[j][c] for j in range(len(vals))) for c in range(len(vals[0]))]
    return out, m + math.log(tot)


def brute_prefill(q, k, v, scale, causal):
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                o[b, h, i], lse[b, h, i] = brute_attention_row(
                    q[b, h, i].tolist(), k[b, g].tolist(), v[b, g].tolist(), scale,
                    i if causal else None)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 4, 2, 5, 3), (1, 3, 3, 6, 2), (1, 4, 1, 4, 3)])
def test_prefill_matches_brute_force(shape, causal):
    B, Hq, Hkv, T, d = shape
    q = RNG.standard_normal((B, Hq, T, d))
    k = RNG.standard_normal((B, Hkv, T, d))
    v = RNG.standard_normal((B, Hkv, T, d))
    scale = 0.37
    o, lse = oracle.prefill(q, k, v, scale, causal=causal)
    ob, lb = brute_prefill(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# hand-worked examples (exact rationals), tests/golden/hand_worked.json
# ----------------------------------------------------------------------------

def test_hand_worked_golden():
    cases = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))["cases"]
    for c in cases:
        qr = np.array(c["q_rows"], dtype=np.float64)
        T, d = qr.shape
        q = qr.reshape(1, 1, T, d)
        k = np.array(c["k"], dtype=np.float64).reshape(1, 1, T, d)
        v = np.array(c["v"], dtype=np.float64).reshape(1, 1, T, -1)
        o, lse = oracle.prefill(q, k, v, c["scale"], causal=True)
        np.testing.assert_allclose(o[0, 0], np.array(c["o"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], np.array(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])


# ----------------------------------------------------------------------------
# invariants and closed forms
# ----------------------------------------------------------------------------

def test_weights_are_a_causal_stochastic_matrix():
    # With V = identity (d = T) the output row i IS the weight row i:
    # non-negative, summing to 1, zero for keys after the query.
    T = 9
    q = RNG.standard_normal((1, 1, T, 4))
    k = RNG.standard_normal((1, 1, T, 4))
    v = np.eye(T).reshape(1, 1, T, T)
    o, _ = oracle.prefill(q, k, v, 0.8, causal=True)
    W = o[0, 0]
    assert np.all(W >= 0)
    np.testing.assert_allclose(W.sum(axis=1), np.ones(T), rtol=0, atol=1e-12)
    assert np.all(np.triu(W, 1) == 0)
    assert np.all(np.diag(W) > 0)


@pytest.mark.parametrize("causal", [True, False])
def test_zero_query_closed_form(causal):
    # q = 0: every visible score is 0, so the weights are uniform over the
    # visible keys: o_i = mean(v_0..v_i) (causal) and lse_i = ln(i + 1).
    T, d = 12, 5
    q = np.zeros((1, 2, T, d))
    k = RNG.standard_normal((1, 2, T, d))
    v = RNG.standard_normal((1, 2, T, d))
    o, lse = oracle.prefill(q, k, v, 1.3, causal=causal)
    for h in range(2):
        for i in range(T):
            n = i + 1 if causal else T
            np.testing.assert_allclose(o[0, h, i], v[0, h, :n].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[0, h, i] - math.log(n)) < 1e-13


def test_constant_v_gives_constant_output():
    T, d = 10, 6
    q = RNG.standard_normal((1, 2, T, d)) * 3
    k = RNG.standard_normal((1, 2, T, d)) * 3
    row = RNG.standard_normal(d)
    v = np.broadcast_to(row, (1, 2, T, d)).copy()
    o, _ = oracle.prefill(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=0, atol=1e-13)


def test_single_key_output_is_v0():
    q = RNG.standard_normal((2, 3, 1, 7))
    k = RNG.standard_normal((2, 3, 1, 7))
    v = RNG.standard_normal((2, 3, 1, 7))
    for causal in (True, False):
        o, lse = oracle.prefill(q, k, v, 0.25, causal=causal)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse, 0.25 * np.sum(q * k, axis=-1), rtol=0, atol=1e-14)


def test_causality_later_tokens_do_not_matter():
    T, d = 16, 4
    q = RNG.standard_normal((1, 2, T, d))
    k = RNG.standard_normal((1, 2, T, d))
    v = RNG.standard_normal((1, 2, T, d))
    o, lse = oracle.prefill(q, k, v, 0.6, causal=True)
    for i in (0, 5, 14):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, :, i + 1:] += 100.0
        k2[:, :, i + 1:] -= 50.0
        v2[:, :, i + 1:] *= -7.0
        o2, lse2 = oracle.prefill(q2, k2, v2, 0.6, causal=True)
        np.testing.assert_array_equal(o2[:, :, :i + 1], o[:, :, :i + 1])
        np.testing.assert_array_equal(lse2[:, :, :i + 1], lse[:, :, :i + 1])
        assert not np.allclose(o2[:, :, i + 1:], o[:, :, i + 1:])


def test_scale_moves_between_q_and_scale():
    T, d = 8, 4
    q = RNG.standard_normal((1, 1, T, d))
    k = RNG.standard_normal((1, 1, T, d))
    v = RNG.standard_normal((1, 1, T, d))
    o1, l1 = oracle.prefill(q, k, v, 0.5, causal=True)
    o2, l2 = oracle.prefill(q * 4.0, k, v, 0.125, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    # and the scale really enters: a different scale changes the result
    o3, _ = oracle.prefill(q, k, v, 1.0, causal=True)
    assert not np.allclose(o1, o3)


def test_gqa_equals_mha_on_repeated_kv():
    B, Hq, Hkv, T, d = 2, 6, 2, 7, 3
    q = RNG.standard_normal((B, Hq, T, d))
    k = RNG.standard_normal((B, Hkv, T, d))
    v = RNG.standard_normal((B, Hkv, T, d))
    o, lse = oracle.prefill(q, k, v, 0.7, causal=True)
    G = Hq // Hkv
    o2, lse2 = oracle.prefill(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.7, causal=True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_fp64(causal):
    # The library special case: PyTorch's scaled_dot_product_attention (the
    # op the pages name) on the CPU in float64, GQA expanded explicitly.
    B, Hq, Hkv, T, d = 2, 4, 2, 33, 16
    q = RNG.standard_normal((B, Hq, T, d))
    k = RNG.standard_normal((B, Hkv, T, d))
    v = RNG.standard_normal((B, Hkv, T, d))
    o, _ = oracle.prefill(q, k, v, 0.2, causal=causal)
    G = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, G, axis=1)),
        torch.from_numpy(np.repeat(v, G, axis=1)), is_causal=causal, scale=0.2).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    T, d = 40, 8
    q = RNG.standard_normal((1, 2, T, d))
    k = RNG.standard_normal((1, 1, T, d))
    v = RNG.standard_normal((1, 1, T, d))
    o, lse = oracle.prefill(q, k, v, 0.3, causal=True)
    rows = [0, 3, 17, 39]
    os_, ls_ = oracle.prefill(q, k, v, 0.3, causal=True, rows=rows, heads=[1])
    np.testing.assert_allclose(os_[0, 1], o[0, 1, rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ls_[0, 1], lse[0, 1, rows], rtol=0, atol=1e-13)
    assert np.all(np.isnan(os_[0, 0]))


def test_row_blocking_does_not_change_rows():
    # more rows than one internal row block
    T, d = 2048 + 37, 4
    q = RNG.standard_normal((1, 1, T, d))
    k = RNG.standard_normal((1, 1, T, d))
    v = RNG.standard_normal((1, 1, T, d))
    o, _ = oracle.prefill(q, k, v, 0.5, causal=True)
    rows = [0, 2047, 2048, T - 1]
    for i in rows:
        ob, _ = brute_attention_row(q[0, 0, i].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.5, i)
        np.testing.assert_allclose(o[0, 0, i], ob, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# paged KV cache ("Fast attention kernels and operator fusion", section on
# FlashAttention-style and paged attention)
# ----------------------------------------------------------------------------

def brute_gather(cache, table_row, L, bs=16):
    out = []
    for p in range(L):
        blk = int(table_row[p // bs])
        out.append(cache[blk, :, p % bs, :])
    return np.array(out).reshape(L, cache.shape[1], cache.shape[3])


def small_batch(seed, seq_lens, q_lens=None, Hq=4, Hkv=2, d=8):
    return inputs.paged_inputs(len(seq_lens), Hq, Hkv, d, seq_lens=seq_lens, q_lens=q_lens,
                               dtype=torch.float32, seed=seed)


def test_gather_matches_brute_force():
    b = small_batch(1, [1, 15, 16, 17, 40])
    kc = b["k_cache"].double().numpy()
    for n, L in enumerate(b["seq_lens_host"]):
        got = oracle.gather_paged_kv(kc, b["block_table"][n].numpy(), L)
        np.testing.assert_array_equal(got, brute_gather(kc, b["block_table"][n].numpy(), L))
        assert np.all(np.isfinite(got))  # never touches poisoned slots


def test_paged_decode_brute_force_mixed_lengths():
    seq_lens = [5, 16, 17, 33]
    q_lens = [1, 3, 1, 4]
    b = small_batch(2, seq_lens, q_lens, Hq=6, Hkv=2, d=3)
    o, lse = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 0.9, query_start_loc=b["query_start_loc"])
    q = b["q"].double().numpy()
    kc, vc = b["k_cache"].double().numpy(), b["v_cache"].double().numpy()
    qsl = b["query_start_loc"].numpy()
    G = 3
    for n, L in enumerate(seq_lens):
        K = brute_gather(kc, b["block_table"][n].numpy(), L)
        V = brute_gather(vc, b["block_table"][n].numpy(), L)
        for t in range(qsl[n], qsl[n + 1]):
            pos = L - (qsl[n + 1] - t)  # absolute position of this query
            for h in range(6):
                ob, lb = brute_attention_row(q[t, h].tolist(), K[:, h // G].tolist(),
                                             V[:, h // G].tolist(), 0.9, pos)
                np.testing.assert_allclose(o[t, h], ob, rtol=0, atol=1e-12)
                assert abs(lse[t, h] - lb) < 1e-12


def test_paged_decode_equals_last_row_of_contiguous_prefill():
    seq_lens = [1, 16, 31, 64, 100]
    b = small_batch(3, seq_lens, Hq=4, Hkv=2, d=8)
    o, lse = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 0.35)
    kc, vc = b["k_cache"].double().numpy(), b["v_cache"].double().numpy()
    for n, L in enumerate(seq_lens):
        K = oracle.gather_paged_kv(kc, b["block_table"][n].numpy(), L).transpose(1, 0, 2)[None]
        V = oracle.gather_paged_kv(vc, b["block_table"][n].numpy(), L).transpose(1, 0, 2)[None]
        Q = np.zeros((1, 4, L, 8))
        Q[0, :, L - 1] = b["q"][n].double().numpy()
        op, lp = oracle.prefill(Q, K, V, 0.35, causal=True, rows=[L - 1])
        np.testing.assert_allclose(o[n], op[0, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[n], lp[0, :, 0], rtol=0, atol=1e-12)


def test_paged_chunk_equals_prefill_rows_with_context():
    # A chunk of q_len queries after ctx cached tokens equals rows ctx..L-1 of
    # the full causal prefill of the whole sequence (bottom-right alignment).
    L, q_len = 45, 13
    b = small_batch(4, [L], [q_len], Hq=2, Hkv=1, d=5)
    o, _ = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                               b["seq_lens"], 0.4, query_start_loc=b["query_start_loc"])
    K = oracle.gather_paged_kv(b["k_cache"], b["block_table"][0].numpy(), L).transpose(1, 0, 2)[None]
    V = oracle.gather_paged_kv(b["v_cache"], b["block_table"][0].numpy(), L).transpose(1, 0, 2)[None]
    Q = RNG.standard_normal((1, 2, L, 5))
    Q[0, :, L - q_len:] = b["q"].double().numpy().transpose(1, 0, 2)
    op, _ = oracle.prefill(Q, K, V, 0.4, causal=True)
    np.testing.assert_allclose(o.transpose(1, 0, 2), op[0, :, L - q_len:], rtol=0, atol=1e-12)


def test_block_permutation_is_invisible():
    b = small_batch(5, [3, 16, 47, 80])
    o, lse = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 0.5)
    k2, v2, t2 = inputs.permute_blocks(b, seed=99)
    assert not torch.equal(t2, b["block_table"])
    o2, lse2 = oracle.decode_paged(b["q"], k2, v2, t2, b["seq_lens"], 0.5)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_unreferenced_storage_is_never_read():
    # paged_inputs poisons spare blocks and the tail slots of last blocks with NaN
    b = small_batch(6, [7, 16, 23, 50])
    assert torch.isnan(b["k_cache"]).any()
    o, lse = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 0.5)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_empty_sequence_gives_zero_and_minus_inf():
    b = small_batch(7, [0, 5])
    o, lse = oracle.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 0.5)
    np.testing.assert_array_equal(o[0], np.zeros_like(o[0]))
    assert np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(o[1]))


# ---- paged cache append -------------------------------------------------

def test_kv_append_hand_worked_golden():
    # tests/golden/kv_append_hand.json: every write worked out by hand
    cases = json.load(open(os.path.join(HERE, "golden", "kv_append_hand.json")))["cases"]
    for c in cases:
        shape = (c["num_blocks"], c["Hkv"], 16, c["d"])
        k0, v0 = np.zeros(shape), np.zeros(shape)
        qsl = c["query_start_loc"]
        kc, vc = oracle.kv_append(np.array(c["k_new"], dtype=float),
                                  np.array(c["v_new"], dtype=float), k0, v0,
                                  np.array(c["block_table"]), np.array(c["seq_lens"]),
                                  None if qsl is None else np.array(qsl))
        ek, ev = np.zeros(shape), np.zeros(shape)
        for w in c["writes"]:
            ek[w["block"], w["head"], w["slot"]] = w["k"]
            ev[w["block"], w["head"], w["slot"]] = w["v"]
        assert np.array_equal(kc, ek), c["name"]
        assert np.array_equal(vc, ev), c["name"]
        assert not np.any(k0) and not np.any(v0)  # inputs untouched


def test_kv_append_then_gather_returns_the_sequence():
    # appending every token of a sequence (q_len = L) into a cache with a
    # random table, then gathering positions 0..L-1, gives the rows back in
    # order; the gather is the decode oracle's own, written separately
    rng = np.random.default_rng(40)
    for L in (1, 15, 16, 17, 50):
        nb = -(-L // 16)
        num_blocks = nb + 3
        table = rng.permutation(num_blocks)[:nb].reshape(1, nb)
        k_new = rng.standard_normal((L, 2, 4))
        v_new = rng.standard_normal((L, 2, 4))
        kc0 = rng.standard_normal((num_blocks, 2, 16, 4))
        vc0 = rng.standard_normal((num_blocks, 2, 16, 4))
        kc, vc = oracle.kv_append(k_new, v_new, kc0, vc0, table, np.array([L]), np.array([0, L]))
        assert np.array_equal(oracle.gather_paged_kv(kc, table[0], L), k_new)
        assert np.array_equal(oracle.gather_paged_kv(vc, table[0], L), v_new)


def test_kv_append_touches_only_the_new_slots():
    # slots other than the new tokens' keep their values (decode step after a
    # chunk: positions written earlier are not disturbed)
    rng = np.random.default_rng(41)
    num_blocks, Hkv, d = 12, 2, 3
    kc0 = rng.standard_normal((num_blocks, Hkv, 16, d))
    vc0 = rng.standard_normal((num_blocks, Hkv, 16, d))
    table = np.array([[4, 7, 1], [9, 0, 11]])
    lens = np.array([40, 20])
    qsl = np.array([0, 5, 6])  # 5 new rows for seq 0 (positions 35..39), 1 for seq 1 (19)
    k_new = rng.standard_normal((6, Hkv, d))
    v_new = rng.standard_normal((6, Hkv, d))
    kc, vc = oracle.kv_append(k_new, v_new, kc0, vc0, table, lens, qsl)
    written = {(1, s) for s in range(3, 8)} | {(0, 3)}  # (block, slot): 35..39 -> block 1, 19 -> block 0
    for b in range(num_blocks):
        for s in range(16):
            if (b, s) not in written:
                assert np.array_equal(kc[b, :, s], kc0[b, :, s]) and np.array_equal(vc[b, :, s], vc0[b, :, s])
    assert np.array_equal(kc[1, :, 3:8], k_new[:5].transpose(1, 0, 2))
    assert np.array_equal(vc[0, :, 3], v_new[5])


def test_kv_append_keeps_bf16_bits():
    # bf16 tensors are copied through their bit patterns, NaN payloads included
    import torch

    k_new = torch.tensor([[[1.5, -0.0]]], dtype=torch.bfloat16)
    v_new = torch.tensor([[[float("nan"), 3.0]]], dtype=torch.bfloat16)
    kc0 = torch.zeros(2, 1, 16, 2, dtype=torch.bfloat16)
    kc, vc = oracle.kv_append(k_new, v_new, kc0, kc0.clone(), torch.tensor([[1]]),
                              torch.tensor([3]))
    assert kc.dtype == np.int16
    assert list(kc[1, 0, 2]) == list(k_new.view(torch.int16).numpy()[0, 0])
    assert list(vc[1, 0, 2]) == list(v_new.view(torch.int16).numpy()[0, 0])
    assert not np.any(kc[0]) and not np.any(kc[1, 0, :2])


# ---- residual add + RMSNorm ---------------------------------------------

def test_add_rmsnorm_hand_worked_golden():
    # tests/golden/add_rmsnorm_hand.json: every value worked out by hand
    cases = json.load(open(os.path.join(HERE, "golden", "add_rmsnorm_hand.json")))["cases"]
    for c in cases:
        y, h = oracle.add_rmsnorm(np.array(c["x"]), np.array(c["residual"]), np.array(c["weight"]),
                                  c["eps"])
        np.testing.assert_allclose(h, np.array(c["h"]), rtol=0, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(y, np.array(c["y"]), rtol=1e-14, atol=1e-15, err_msg=c["name"])


def test_add_rmsnorm_unit_rms_and_scale_invariance():
    # with eps = 0 and unit weight every output row has mean square exactly 1,
    # and scaling both inputs by alpha leaves y unchanged
    x = RNG.standard_normal((5, 37))
    r = RNG.standard_normal((5, 37))
    y, h = oracle.add_rmsnorm(x, r, np.ones(37), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    y2, _ = oracle.add_rmsnorm(3.5 * x, 3.5 * r, np.ones(37), 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(h, x + r)


def test_add_rmsnorm_weight_multiplies_columns():
    x = RNG.standard_normal((3, 16))
    r = RNG.standard_normal((3, 16))
    w = RNG.standard_normal(16)
    y1, _ = oracle.add_rmsnorm(x, r, np.ones(16), 1e-5)
    yw, _ = oracle.add_rmsnorm(x, r, w, 1e-5)
    np.testing.assert_allclose(yw, y1 * w, rtol=1e-14, atol=1e-15)


def test_add_rmsnorm_matches_torch_rms_norm_fp64():
    # library special case: torch.nn.functional.rms_norm on the sum, in fp64
    x = torch.randn(4, 64, dtype=torch.float64)
    r = torch.randn(4, 64, dtype=torch.float64)
    w = torch.randn(64, dtype=torch.float64)
    y, _ = oracle.add_rmsnorm(x, r, w, 1e-6)
    ref = torch.nn.functional.rms_norm(x + r, (64,), weight=w, eps=1e-6)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)
