"""GPU parity of attn_decode_paged on mixed batches: chunked-prefill sequences
(q_len >= 2, K/V tiles gathered through the block table) next to single-token
decodes, against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs
from parity import assert_close, assert_lse_close, ref_decode, ref_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(b, partition_size=0):
    d = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in b.items()}
    lse = torch.full(tuple(d["q"].shape[:2]), float("nan"), device=DEV)
    o = attn.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                          max_seq_len=b["max_seq_len"], max_query_len=b["max_query_len"],
                          query_start_loc=d["query_start_loc"], partition_size=partition_size,
                          lse=lse)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("seed", [70, 71])
def test_small_mixed_with_context(seed):
    # chunks with prior context (ctx = L - q_len > 0), ragged chunk lengths,
    # next to decodes
    seq_lens = [300, 5, 129, 1000, 64, 17, 700, 2]
    q_lens = [45, 1, 129, 1, 2, 17, 300, 1]
    print(f"[mixed] small seed={seed}", flush=True)
    b = inputs.paged_inputs(len(seq_lens), 8, 2, 128, seq_lens=seq_lens, q_lens=q_lens, seed=seed)
    o, lse = run(b)
    ro, rl, rb = ref_decode(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 1.0 / math.sqrt(128),
                                 query_start_loc=b["query_start_loc"])
    assert_close(o, ro, torch.bfloat16, "mixed")
    assert_lse_close(lse, rl, rb, "mixed")


def test_growing_scores_paged_chunks_and_decodes():
    # Positive queries and keys that drift toward them with their position
    # (about 8.5 log2 units per 64 positions): the running max moves on most
    # tiles of the chunk kernel and most blocks of the split-KV decode, in
    # rows that see context and rows that do not.
    seq_lens = [900, 1500, 257, 2000]
    q_lens = [200, 1, 64, 1]
    d, Hq, Hkv = 128, 8, 2
    print("[mixed] growing scores", flush=True)
    b = inputs.paged_inputs(len(seq_lens), Hq, Hkv, d, seq_lens=seq_lens, q_lens=q_lens,
                            seed=77, poison=False)
    g = torch.Generator().manual_seed(78)
    b["q"] = (torch.randn(b["q"].shape, generator=g).abs() + 0.5).to(torch.bfloat16)
    a = 4.54 / math.sqrt(d)
    kc = b["k_cache"].to(torch.float32)
    for n, L in enumerate(seq_lens):
        for p in range(L):
            blk = int(b["block_table"][n, p // 16])
            kc[blk, :, p % 16, :] = 0.1 * kc[blk, :, p % 16, :] + a * (p / 64.0)
    b["k_cache"] = kc.to(torch.bfloat16)
    o, lse = run(b)
    ro, rl, rb = ref_decode(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                        1.0 / math.sqrt(d), query_start_loc=b["query_start_loc"])
    assert_close(o, ro, torch.bfloat16, "growing scores, paged")
    assert_lse_close(lse, rl, rb, "growing scores, paged")


def test_mixed_d64_gqa4():
    seq_lens = [128, 40, 513]
    q_lens = [128, 1, 200]
    b = inputs.paged_inputs(3, 16, 4, 64, seq_lens=seq_lens, q_lens=q_lens, seed=72)
    o, lse = run(b)
    ro, rl, rb = ref_decode(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                                 b["seq_lens"], 1.0 / math.sqrt(64),
                                 query_start_loc=b["query_start_loc"])
    assert_close(o, ro, torch.bfloat16, "mixed d64")
    assert_lse_close(lse, rl, rb, "mixed d64")


def test_chunk_rows_match_contiguous_prefill():
    # A chunk with context equals the last q_len rows of the contiguous causal
    # prefill over the whole sequence (both on the GPU, within tolerance).
    L, q_len = 640, 200
    b = inputs.paged_inputs(1, 4, 2, 128, seq_lens=[L], q_lens=[q_len], seed=73)
    o, _ = run(b)
    K = oracle.gather_paged_kv(b["k_cache"], b["block_table"][0].numpy(), L)
    V = oracle.gather_paged_kv(b["v_cache"], b["block_table"][0].numpy(), L)
    Kt = torch.from_numpy(K).permute(1, 0, 2)[None].to(torch.bfloat16).contiguous()
    Vt = torch.from_numpy(V).permute(1, 0, 2)[None].to(torch.bfloat16).contiguous()
    Q = torch.zeros(1, 4, L, 128, dtype=torch.bfloat16)
    Q[0, :, L - q_len:] = b["q"].permute(1, 0, 2)
    op = attn.prefill(Q.to(DEV), Kt.to(DEV), Vt.to(DEV), causal=True)
    torch.cuda.synchronize()
    a = o.float().cpu().permute(1, 0, 2)
    c = op[0, :, L - q_len:].float().cpu()
    assert (a - c).abs().max().item() <= 2e-2


def test_mixed_many_sequences_direct_grid():
    # more sequences than the chunk planner handles (2048): the chunk
    # path then launches one workgroup per (query tile, sequence, head) of the
    # host bound, and workgroups of single-token sequences exit at once
    print("[mixed] 2100 sequences, chunks every 100th", flush=True)
    rng = np.random.default_rng(73)
    q_lens = [1] * 2100
    for n in range(0, 2100, 100):
        q_lens[n] = int(rng.integers(2, 300))
    seq_lens = [q + int(rng.integers(0, 200)) for q in q_lens]
    b = inputs.paged_inputs(2100, 4, 2, 64, seq_lens=seq_lens, q_lens=q_lens, seed=73)
    o, lse = run(b)
    chunks = list(range(0, 2100, 100))
    dec = sorted(set(int(x) for x in rng.choice(2100, 40, replace=False)) - set(chunks))
    seqs = chunks + dec
    kc, vc, table, sl, q, qsl_c = inputs.compact_sequences(b, seqs)
    ro, rl, rb = ref_decode(q, kc, vc, table, sl, 1.0 / math.sqrt(64), query_start_loc=qsl_c)
    qsl = b["query_start_loc"]
    rows = torch.cat([torch.arange(int(qsl[n]), int(qsl[n + 1])) for n in seqs])
    assert_close(o[rows.to(DEV)], ro, torch.bfloat16, "2100 sequences")
    assert_lse_close(lse[rows.to(DEV)], rl, rb, "2100 sequences")


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 4, 1)])
def test_mixed_many_chunk_sequences_unsorted(d, Hq, Hkv):
    # 200 chunk sequences (more than the 128 that the chunk planner orders by
    # size) among 800 sequences (within the 2048 it plans): the plan then
    # lists the chunk sequences in batch order. Chunks and
    # decodes interleave in the batch, chunks have ragged lengths and prior
    # context; every chunk and 40 decodes are checked against the oracle.
    print(f"[mixed] 800 sequences, 200 chunks, d={d}", flush=True)
    rng = np.random.default_rng(74 + d)
    n = 800
    chunk_ids = sorted(int(x) for x in rng.choice(n, 200, replace=False))
    q_lens = [1] * n
    for c in chunk_ids:
        q_lens[c] = int(rng.integers(2, 301))
    seq_lens = [q + int(rng.integers(0, 201)) for q in q_lens]
    b = inputs.paged_inputs(n, Hq, Hkv, d, seq_lens=seq_lens, q_lens=q_lens, seed=74 + d)
    o, lse = run(b)
    dec = sorted(set(int(x) for x in rng.choice(n, 60, replace=False)) - set(chunk_ids))[:40]
    seqs = chunk_ids + dec
    kc, vc, table, sl, q, qsl_c = inputs.compact_sequences(b, seqs)
    ro, rl, rb = ref_decode(q, kc, vc, table, sl, 1.0 / math.sqrt(d), query_start_loc=qsl_c)
    qsl = b["query_start_loc"]
    rows = torch.cat([torch.arange(int(qsl[m]), int(qsl[m + 1])) for m in seqs])
    assert_close(o[rows.to(DEV)], ro, torch.bfloat16, "200 chunk sequences")
    assert_lse_close(lse[rows.to(DEV)], rl, rb, "200 chunk sequences")


def test_many_chunk_sequences_unsorted_with_split_rows():
    # 150 chunk sequences (more than the 128 the planner orders, so batch
    # order) among 600, three of them after about 9000 cached tokens: those
    # rows are split along the keys while the plan keeps batch order. Every
    # chunk and 30 decodes are checked against the oracle.
    print("[mixed] 600 sequences, 150 chunks, 3 split", flush=True)
    rng = np.random.default_rng(77)
    n = 600
    chunk_ids = sorted(int(x) for x in rng.choice(n, 150, replace=False))
    q_lens = [1] * n
    for c in chunk_ids:
        q_lens[c] = int(rng.integers(2, 65))
    seq_lens = [q + int(rng.integers(0, 301)) for q in q_lens]
    long_ids = chunk_ids[10::50]
    for c in long_ids:
        seq_lens[c] = q_lens[c] + 9000 + int(rng.integers(0, 200))
    b = inputs.paged_inputs(n, 8, 2, 128, seq_lens=seq_lens, q_lens=q_lens, seed=77)
    # room for key pieces only when some sequence may pass 4096 keys
    assert attn.paged_workspace_size(n, sum(q_lens), 8, 2, 128, max(seq_lens), max(q_lens)) > \
        attn.paged_workspace_size(n, sum(q_lens), 8, 2, 128, 4096, max(q_lens)) + \
        attn.decode_paged_workspace_size(n, 8, 2, 128, max(seq_lens)) - \
        attn.decode_paged_workspace_size(n, 8, 2, 128, 4096)
    o, lse = run(b)
    dec = sorted(set(int(x) for x in rng.choice(n, 50, replace=False)) - set(chunk_ids))[:30]
    seqs = chunk_ids + dec
    kc, vc, table, sl, q, qsl_c = inputs.compact_sequences(b, seqs)
    ro, rl, rb = ref_decode(q, kc, vc, table, sl, 1.0 / math.sqrt(128), query_start_loc=qsl_c)
    qsl = b["query_start_loc"]
    rows = torch.cat([torch.arange(int(qsl[m]), int(qsl[m + 1])) for m in seqs])
    assert_close(o[rows.to(DEV)], ro, torch.bfloat16, "150 chunk sequences, 3 split")
    assert_lse_close(lse[rows.to(DEV)], rl, rb, "150 chunk sequences, 3 split")


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 8, 2), (64, 4, 1), (128, 16, 1), (64, 8, 8)])
def test_chunk_rows_split_along_the_keys(d, Hq, Hkv):
    # chunk rows whose keys span more than one 4096-key piece (each query
    # tile's key range is split evenly, the pieces run in parallel and are
    # merged by log-sum-exp): 9000 keys (3 pieces), 5000 (2), 4200 with 200
    # new rows (their two query tiles, of 65 and 66 key tiles, split in 2),
    # next to decodes and a short chunk that is not split
    seq_lens = [9000, 300, 5000, 4200, 6000, 700]
    q_lens = [300, 1, 64, 200, 1, 129]
    print(f"[mixed] chunk rows split along the keys d={d} Hq={Hq} Hkv={Hkv}", flush=True)
    b = inputs.paged_inputs(len(seq_lens), Hq, Hkv, d, seq_lens=seq_lens, q_lens=q_lens,
                            seed=79 + d)
    assert attn.paged_workspace_size(len(seq_lens), sum(q_lens), Hq, Hkv, d, max(seq_lens),
                                     max(q_lens)) > \
        attn.decode_paged_workspace_size(len(seq_lens), Hq, Hkv, d, max(seq_lens))
    o, lse = run(b)
    ro, rl, rb = ref_decode(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                            1.0 / math.sqrt(d), query_start_loc=b["query_start_loc"])
    assert_close(o, ro, torch.bfloat16, "split chunk rows")
    assert_lse_close(lse, rl, rb, "split chunk rows")


def test_split_chunk_rows_match_unsplit_batch():
    # the same chunk computed in a batch of more than 2048 sequences (whose
    # chunk rows are not split) and in a small batch (split): equal within
    # the rounding of the merge (each piece rounds its weights to bf16
    # against its own max; bound derived as for the split-KV decode)
    L, q_len, Hq, Hkv, d = 8200, 100, 4, 2, 128
    small = inputs.paged_inputs(1, Hq, Hkv, d, seq_lens=[L], q_lens=[q_len], seed=81)
    o_split, _ = run(small)
    n = 2049
    big_lens = [L] + [1] * (n - 1)
    big_q = [q_len] + [1] * (n - 1)
    big = inputs.paged_inputs(n, Hq, Hkv, d, seq_lens=big_lens, q_lens=big_q, seed=82)
    # put the small batch's sequence into the big pool: same K/V, same q
    t = big["block_table"][0, :-(-L // 16)].long()
    big["k_cache"][t] = small["k_cache"][small["block_table"][0, :-(-L // 16)].long()]
    big["v_cache"][t] = small["v_cache"][small["block_table"][0, :-(-L // 16)].long()]
    big["q"][:q_len] = small["q"]
    o_whole, _ = run(big)
    a_ = o_split.float().cpu().double().numpy()
    c_ = o_whole[:q_len].float().cpu().double().numpy()
    V = oracle.gather_paged_kv(small["v_cache"], small["block_table"][0].numpy(), L)
    vmax = np.repeat(np.abs(V).max(axis=0), Hq // Hkv, axis=0)[None]  # [1, Hq, d]
    bound = (2.0 ** -8) * (np.abs(a_) + np.abs(c_)) * (1 + 2.0 ** -7) + (2.0 ** -7 + 2.0 ** -12) * vmax
    assert (np.abs(a_ - c_) <= bound).all()


def test_config_mixed_batch_full_size_sampled():
    # 8 chunks of 512 new tokens + 256 decodes with lengths uniform in
    # [1024, 32768], Hq=32, Hkv=8, d=128, one shuffled pool (~17.9 GB) drawn
    # on the GPU; the call is the one the benchmark times. The oracle checks
    # every chunk and 16 decode sequences including the shortest and longest.
    print("[mixed] full-size batch", flush=True)
    b = inputs.mixed_batch_inputs(8, 512, 256, (1024, 32768), 32, 8, 128, seed=5, device=DEV)
    o = torch.empty_like(b["q"])
    lse = torch.full(tuple(b["q"].shape[:2]), float("nan"), device=DEV)
    attn.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                      max_seq_len=b["max_seq_len"], max_query_len=b["max_query_len"],
                      query_start_loc=b["query_start_loc"], o=o, lse=lse)
    torch.cuda.synchronize()
    lens = b["seq_lens_host"]
    dec = list(range(8, 264))
    rng = np.random.default_rng(5)
    pick = {min(dec, key=lambda n: lens[n]), max(dec, key=lambda n: lens[n])}
    pick |= set(int(x) for x in rng.choice(dec, 14, replace=False))
    seqs = list(range(8)) + sorted(pick)
    kc, vc, table, sl, q, qsl = inputs.compact_sequences(b, seqs)
    ro, rl, rb = ref_decode(q, kc, vc, table, sl, 1.0 / math.sqrt(128), query_start_loc=qsl)
    qsl_full = b["query_start_loc"].cpu()
    rows = torch.cat([torch.arange(int(qsl_full[n]), int(qsl_full[n + 1])) for n in seqs])
    assert_close(o[rows.to(DEV)], ro, torch.bfloat16, "full-size mixed")
    assert_lse_close(lse[rows.to(DEV)], rl, rb, "full-size mixed")
    del b
    torch.cuda.empty_cache()


def test_config_mixed_batch_with_context_full_size_sampled():
    # the mixed batch with prior context: 8 chunks of 512 new tokens whose
    # sequences are 1024..32768 long (so each chunk follows up to 32256 cached
    # tokens), next to 256 decodes, Hq=32, Hkv=8, d=128, one shuffled pool on
    # the GPU, in the launch configuration the benchmark times. The oracle
    # checks 8 rows of every chunk (first, last, the rest seeded) against the
    # contiguous causal prefill of the gathered sequence at those rows, and 16
    # decode sequences including the shortest and longest.
    print("[mixed] full-size batch with context", flush=True)
    b = inputs.mixed_batch_inputs(8, 512, 256, (1024, 32768), 32, 8, 128, seed=7, device=DEV,
                                  chunk_len_range=(1024, 32768))
    o = torch.empty_like(b["q"])
    lse = torch.full(tuple(b["q"].shape[:2]), float("nan"), device=DEV)
    attn.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                      max_seq_len=b["max_seq_len"], max_query_len=b["max_query_len"],
                      query_start_loc=b["query_start_loc"], o=o, lse=lse)
    torch.cuda.synchronize()
    lens = b["seq_lens_host"]
    qsl = b["query_start_loc"].cpu()
    rng = np.random.default_rng(7)
    scale = 1.0 / math.sqrt(128)
    for n in range(8):
        L = lens[n]
        ctx = L - 512
        picks = sorted({0, 511} | set(int(x) for x in rng.choice(512, 6, replace=False)))
        kc, vc, table, sl, q, _ = inputs.compact_sequences(b, [n])
        K = oracle.gather_paged_kv(kc, table[0].numpy(), L).transpose(1, 0, 2)[None]
        V = oracle.gather_paged_kv(vc, table[0].numpy(), L).transpose(1, 0, 2)[None]
        Q = np.zeros((1, 32, L, 128))
        Q[0, :, ctx:] = q.double().numpy().transpose(1, 0, 2)
        ro, rl, rb = ref_prefill(Q, K, V, scale, causal=True, rows=[ctx + i for i in picks])
        rows = torch.tensor([int(qsl[n]) + i for i in picks])
        got = o[rows.to(DEV)].transpose(0, 1)  # [Hq, rows, d]
        assert_close(got, ro[0], torch.bfloat16, f"chunk {n} (context {ctx})")
        assert_lse_close(lse[rows.to(DEV)].transpose(0, 1), rl[0], rb[0], f"chunk {n} lse")
    dec = list(range(8, 264))
    pick = {min(dec, key=lambda n: lens[n]), max(dec, key=lambda n: lens[n])}
    pick |= set(int(x) for x in rng.choice(dec, 14, replace=False))
    seqs = sorted(pick)
    kc, vc, table, sl, q, qsl_c = inputs.compact_sequences(b, seqs)
    ro, rl, rb = ref_decode(q, kc, vc, table, sl, scale, query_start_loc=qsl_c)
    rows = torch.tensor([int(qsl[n]) for n in seqs])
    assert_close(o[rows.to(DEV)], ro, torch.bfloat16, "decodes next to context chunks")
    assert_lse_close(lse[rows.to(DEV)], rl, rb, "decodes next to context chunks")
    del b
    torch.cuda.empty_cache()
