"""GPU parity of attn_kv_append (new tokens' K/V written into the paged cache
through the block table) against the oracle. A byte copy: every comparison
is bit for bit, on the raw 16-bit patterns of the whole cache (NaN-poisoned
spare blocks and tail slots included)."""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs
from parity import assert_close, assert_lse_close, ref_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    return t.detach().cpu().view(torch.int16).numpy()


def gpu_append(b, k_new, v_new, with_qsl=True):
    d = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in b.items()}
    kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
    attn.kv_append(k_new.to(DEV), v_new.to(DEV), kc, vc, d["block_table"], d["seq_lens"],
                   max_query_len=max(1, b["max_query_len"]),
                   query_start_loc=d["query_start_loc"] if with_qsl else None)
    torch.cuda.synchronize()
    return kc, vc


@pytest.mark.parametrize("Hkv,d,seq_lens,q_lens,seed", [
    (2, 128, [300, 5, 129, 1000, 64, 17, 700, 2], [45, 1, 129, 1, 2, 17, 300, 1], 80),
    (1, 64, [16, 17, 33, 1], [16, 1, 33, 1], 81),          # block-aligned, whole-sequence chunks
    (8, 128, [40, 100, 3], [0, 70, 3], 82),                # a sequence with no new rows
    (4, 64, [5000, 31], [1000, 31], 83),                   # runs of 32 across many blocks
])
def test_append_matches_oracle(Hkv, d, seq_lens, q_lens, seed):
    print(f"[append] Hkv={Hkv} d={d} seed={seed}", flush=True)
    b = inputs.paged_inputs(len(seq_lens), 2 * Hkv, Hkv, d, seq_lens=seq_lens, q_lens=q_lens,
                            seed=seed)
    k_new, v_new = inputs.new_kv_rows(sum(q_lens), Hkv, d, seed + 100)
    kc, vc = gpu_append(b, k_new, v_new)
    rk, rv = oracle.kv_append(k_new, v_new, b["k_cache"], b["v_cache"], b["block_table"],
                              b["seq_lens"], b["query_start_loc"])
    assert np.array_equal(bits(kc), rk)
    assert np.array_equal(bits(vc), rv)


def test_append_one_row_per_sequence_without_qsl():
    print("[append] decode step, no query_start_loc", flush=True)
    b = inputs.paged_inputs(64, 12, 2, 128, seq_len_range=(1, 600), seed=84)
    k_new, v_new = inputs.new_kv_rows(64, 2, 128, 184)
    kc, vc = gpu_append(b, k_new, v_new, with_qsl=False)
    rk, rv = oracle.kv_append(k_new, v_new, b["k_cache"], b["v_cache"], b["block_table"],
                              b["seq_lens"])
    assert np.array_equal(bits(kc), rk)
    assert np.array_equal(bits(vc), rv)


def test_append_many_sequences_and_unclaimed_rows():
    # 5000 sequences (more than the workgroup stages in LDS: the sequence of
    # each row is then searched in global memory), mixed row counts, and two
    # extra rows past query_start_loc[num_seqs] that belong to no sequence and
    # must not be written anywhere
    print("[append] 5000 sequences + unclaimed rows", flush=True)
    rng = np.random.default_rng(87)
    q_lens = [int(x) for x in rng.integers(0, 3, 5000)]
    seq_lens = [int(q + x) for q, x in zip(q_lens, rng.integers(0, 40, 5000))]
    seq_lens = [max(1, L) for L in seq_lens]
    b = inputs.paged_inputs(5000, 2, 1, 64, seq_lens=seq_lens, q_lens=q_lens, seed=87)
    rows = sum(q_lens)
    k_new, v_new = inputs.new_kv_rows(rows + 2, 1, 64, 187)
    d = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in b.items()}
    kc, vc = d["k_cache"].clone(), d["v_cache"].clone()
    attn.kv_append(k_new.to(DEV), v_new.to(DEV), kc, vc, d["block_table"], d["seq_lens"],
                   max_query_len=max(1, b["max_query_len"]), query_start_loc=d["query_start_loc"])
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(k_new[:rows], v_new[:rows], b["k_cache"], b["v_cache"],
                              b["block_table"], b["seq_lens"], b["query_start_loc"])
    assert np.array_equal(bits(kc), rk)
    assert np.array_equal(bits(vc), rv)


def test_append_then_decode_step():
    # one decode step as a serving loop runs it: write the new token's K/V,
    # then attend over the whole cache; against the oracle's append + decode
    print("[append] append then decode", flush=True)
    b = inputs.paged_inputs(16, 8, 2, 128, seq_len_range=(1, 900), seed=85)
    k_new, v_new = inputs.new_kv_rows(16, 2, 128, 185)
    kc, vc = gpu_append(b, k_new, v_new, with_qsl=False)
    q = b["q"].to(DEV)
    lse = torch.full(tuple(q.shape[:2]), float("nan"), device=DEV)
    o = attn.decode_paged(q, kc, vc, b["block_table"].to(DEV), b["seq_lens"].to(DEV),
                          max_seq_len=b["max_seq_len"], lse=lse)
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(k_new, v_new, b["k_cache"], b["v_cache"], b["block_table"],
                              b["seq_lens"])
    rk = torch.from_numpy(rk).view(torch.bfloat16)
    rv = torch.from_numpy(rv).view(torch.bfloat16)
    ro, rl, rb = ref_decode(b["q"], rk, rv, b["block_table"], b["seq_lens"],
                                 1.0 / math.sqrt(128))
    assert_close(o, ro, torch.bfloat16, "append + decode")
    assert_lse_close(lse, rl, rb, "append + decode")


def test_append_full_size_mixed_batch_sampled():
    # the mixed-batch shape: 8 chunks of 512 new tokens + 256 decodes with
    # lengths uniform in [1024, 32768], Hkv=8, d=128, one ~17.9 GB pool on the
    # GPU, appended in the launch configuration the benchmark times. The
    # blocks of every chunk and of 16 decode sequences (shortest, longest and
    # 14 seeded) are compared with the oracle bit for bit, whole blocks
    # (untouched slots included).
    print("[append] full-size mixed batch", flush=True)
    b = inputs.mixed_batch_inputs(8, 512, 256, (1024, 32768), 32, 8, 128, seed=5, device=DEV)
    num_tokens = b["q"].shape[0]
    k_new, v_new = inputs.new_kv_rows(num_tokens, 8, 128, 105, device=DEV)
    lens = b["seq_lens_host"]
    dec = list(range(8, 264))
    rng = np.random.default_rng(6)
    pick = {min(dec, key=lambda n: lens[n]), max(dec, key=lambda n: lens[n])}
    pick |= set(int(x) for x in rng.choice(dec, 14, replace=False))
    seqs = list(range(8)) + sorted(pick)
    kc0, vc0, table, sl, _, qsl = inputs.compact_sequences(b, seqs)
    qsl_full = b["query_start_loc"].cpu()
    rows = torch.cat([torch.arange(int(qsl_full[n]), int(qsl_full[n + 1])) for n in seqs])
    kn, vn = k_new[rows.to(DEV)].cpu(), v_new[rows.to(DEV)].cpu()
    attn.kv_append(k_new, v_new, b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                   max_query_len=b["max_query_len"], query_start_loc=b["query_start_loc"])
    torch.cuda.synchronize()
    kc1, vc1, _, _, _, _ = inputs.compact_sequences(b, seqs)
    rk, rv = oracle.kv_append(kn, vn, kc0, vc0, table, sl, qsl)
    assert np.array_equal(bits(kc1), rk)
    assert np.array_equal(bits(vc1), rv)
    del b, k_new, v_new
    torch.cuda.empty_cache()


def test_append_rejects_bad_requests_on_the_host():
    b = inputs.paged_inputs(2, 4, 2, 128, seq_lens=[10, 20], seed=86)
    d = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in b.items()}
    k_new, v_new = inputs.new_kv_rows(2, 2, 128, 186, device=DEV)
    with pytest.raises(attn.AttnError) as e:
        attn.kv_append(k_new.float(), v_new.float(), d["k_cache"].float(), d["v_cache"].float(),
                       d["block_table"], d["seq_lens"])
    assert e.value.name == "ATTN_ERR_UNSUPPORTED"
    with pytest.raises(attn.AttnError) as e:  # two rows per sequence need query_start_loc
        attn.kv_append(k_new, v_new, d["k_cache"], d["v_cache"], d["block_table"],
                       d["seq_lens"], max_query_len=2)
    assert e.value.name == "ATTN_ERR_SHAPE"
