"""attn_decode_paged_noalloc (through the C ABI) against attn_decode_paged:
same kernels, so the same partition size must give the same bits; both are
also held to the oracle. Two calls in a row, the second with a smaller
batch, so the fixed scratch array is reused with the first call's contents
still in it. No allocation may happen during the calls."""

import math

import pytest
import torch

import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs
from parity import assert_close, assert_lse_close, ref_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(b):
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in b.items()}


def both(b, with_qsl, partition_size=0):
    d = to_dev(b)
    kw = dict(max_seq_len=b["max_seq_len"], max_query_len=b["max_query_len"],
              query_start_loc=d["query_start_loc"] if with_qsl else None,
              partition_size=partition_size)
    o_ref = torch.empty_like(d["q"])
    lse_ref = torch.full(tuple(d["q"].shape[:2]), float("nan"), device=DEV)
    attn.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                      o=o_ref, lse=lse_ref, **kw)
    o = torch.full_like(d["q"], float("nan"))
    lse = torch.full(tuple(d["q"].shape[:2]), float("nan"), device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    attn.decode_paged_noalloc(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                              d["seq_lens"], o, lse=lse, **kw)
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    assert after == before, "the no-allocation call allocated through torch"
    return o, lse, o_ref, lse_ref


def check(b, with_qsl, what, partition_size=0):
    print(f"[noalloc] {what}", flush=True)
    o, lse, o_ref, lse_ref = both(b, with_qsl, partition_size)
    assert torch.equal(o, o_ref), f"{what}: output differs from attn_decode_paged"
    assert torch.equal(lse, lse_ref), f"{what}: lse differs from attn_decode_paged"
    ro, rl, rb = ref_decode(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                            1.0 / math.sqrt(b["q"].shape[-1]),
                            query_start_loc=b["query_start_loc"] if with_qsl else None)
    assert_close(o, ro, torch.bfloat16, what)
    assert_lse_close(lse, rl, rb, what)


def test_noalloc_matches_workspace_entry_point_twice():
    # first: the 64-sequence decode batch (Hq=12, Hkv=2, d=128, lengths
    # uniform in [256, 4096]), split into partitions and merged
    big = inputs.paged_inputs(64, 12, 2, 128, seq_len_range=(256, 4096), seed=4)
    check(big, False, "64 sequences")
    # second, smaller, right after: a mixed batch with chunks and decodes,
    # d = 64, small partitions (many partials in the reused array)
    seq_lens = [300, 5, 129, 1000, 64, 17, 700, 2]
    q_lens = [45, 1, 129, 1, 2, 17, 300, 1]
    small = inputs.paged_inputs(len(seq_lens), 8, 2, 64, seq_lens=seq_lens, q_lens=q_lens,
                                seed=70)
    check(small, True, "mixed batch after the large one", partition_size=32)


def test_noalloc_split_chunk_rows():
    # chunk rows whose keys are split into pieces (9000 and 5000 keys) next to
    # a decode: the chunk rows' work plan and the pieces' partial results
    # live in the fixed array too, after the calls above left it dirty
    seq_lens = [9000, 40, 5000]
    q_lens = [300, 1, 64]
    b = inputs.paged_inputs(len(seq_lens), 8, 2, 128, seq_lens=seq_lens, q_lens=q_lens, seed=72)
    assert attn.paged_workspace_size(3, sum(q_lens), 8, 2, 128, max(seq_lens), max(q_lens)) < \
        attn.DECODE_NOALLOC_SCRATCH_BYTES
    check(b, True, "split chunk rows")


def test_noalloc_rejects_requests_beyond_the_array():
    # 2000 sequences of up to 32768 tokens in 16-token partitions need far
    # more than the fixed array: rejected on the host, nothing launched
    n, Hq, Hkv, d, max_len = 2000, 32, 8, 128, 32768
    need = attn.decode_paged_workspace_size(n, Hq, Hkv, d, max_len, 16)
    assert need > attn.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(n, Hq, d, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, Hkv, 16, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    table = torch.zeros(n, max_len // 16, dtype=torch.int32, device=DEV)
    lens = torch.ones(n, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    with pytest.raises(attn.AttnError) as e:
        attn.decode_paged_noalloc(q, kc, vc, table, lens, o, max_seq_len=max_len,
                                  partition_size=16)
    assert e.value.name == "ATTN_ERR_SCRATCH"
