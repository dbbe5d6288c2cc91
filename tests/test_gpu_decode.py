"""GPU parity of attn_decode_paged (one query per sequence) against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import inputs
from parity import assert_close, assert_lse_close, ref_decode, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(b):
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in b.items()}


def run(b, partition_size=0, with_qsl=False, want_lse=True):
    d = to_dev(b)
    lse = torch.full(tuple(d["q"].shape[:2]), float("nan"), device=DEV) if want_lse else None
    o = attn.decode_paged(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                          max_seq_len=max(1, b["max_seq_len"]), max_query_len=b["max_query_len"],
                          query_start_loc=d["query_start_loc"] if with_qsl else None,
                          partition_size=partition_size, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def reference(b):
    return ref_decode(b["q"], b["k_cache"], b["v_cache"], b["block_table"],
                      b["seq_lens"], 1.0 / math.sqrt(b["q"].shape[-1]))


def check(b, partition_size=0, with_qsl=False, what=""):
    o, lse = run(b, partition_size, with_qsl)
    ro, rl, bound = reference(b)
    assert_close(o, ro, torch.bfloat16, what)
    assert_lse_close(lse, rl, bound, what)
    return o, lse


def test_config_decode_64_seqs():
    # 64 sequences, Hq=12, Hkv=2, d=128, lengths uniform in [256, 4096]
    print("[decode] 64 seqs Hq=12 Hkv=2", flush=True)
    b = inputs.paged_inputs(64, 12, 2, 128, seq_len_range=(256, 4096), seed=4)
    check(b, what="64 seqs")


EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1000, 4095, 4096,
             4097]


@pytest.mark.parametrize("P", [0, 16, 32, 256, 512, 4096])
def test_edge_lengths_all_partition_sizes(P):
    print(f"[decode] edge lengths P={P}", flush=True)
    b = inputs.paged_inputs(len(EDGE_LENS), 8, 2, 128, seq_lens=EDGE_LENS, seed=40 + P)
    check(b, partition_size=P, what=f"P={P}")


@pytest.mark.parametrize("G", [1, 4, 6, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_group_sizes(G, d):
    print(f"[decode] G={G} d={d}", flush=True)
    b = inputs.paged_inputs(7, 2 * G, 2, d, seq_len_range=(1, 700), seed=50 + G + d)
    check(b, what=f"G={G} d={d}")


def max_abs_v(b):
    """Per (sequence, query head, d): the largest |v| over the sequence's keys."""
    Hq, Hkv = b["q"].shape[1], b["v_cache"].shape[1]
    out = []
    for n, L in enumerate(b["seq_lens_host"]):
        V = np.abs(oracle.gather_paged_kv(b["v_cache"], b["block_table"][n].numpy(), L))
        out.append(np.repeat(V.max(axis=0), Hq // Hkv, axis=0))  # [Hq, d]
    return np.stack(out)


def test_partition_size_invariance():
    b = inputs.paged_inputs(9, 12, 2, 128, seq_len_range=(1, 2000), seed=60)
    outs = [run(b, P) for P in (16, 32, 256, 512, 2048)]
    base_o, base_l = outs[-1]  # one partition per sequence: the unsplit case
    vmax = max_abs_v(b)
    nblk = np.array([-(-L // 16) for L in b["seq_lens_host"]], dtype=np.float64)[:, None]
    for o, l in outs[:-1]:
        # The merge identity is exact. Each path rounds its softmax weights to
        # bf16 (relative u = 2^-8 each, against its own partition's max), so
        # its fp32 result lies within u * sum_j p_j |v_j| / l <= u * max_j |v_j|
        # of the same exact value, and both results are rounded to bf16
        # (within u of their magnitude). fp32 sums, the merge and the scale
        # by 1/l add a few 1e-6 relative, inside the 2^-12 allowance.
        a, c = to64(o), to64(base_o)
        bound = (2.0 ** -8) * (np.abs(a) + np.abs(c)) * (1 + 2.0 ** -7) + \
            (2.0 ** -7 + 2.0 ** -12) * vmax
        assert (np.abs(a - c) <= bound).all()
        # lse: the scores are the same on every path (no reference max seeds
        # them in decode); the row sums are fp32 chains of at most L/16 + 64
        # additions, plus the merge's exp2/log2 and the final ln2 scaling
        la, lc = to64(l), to64(base_l)
        lbound = 2 * (nblk + 64) * 2.0 ** -23 + np.abs(lc) * 2.0 ** -22
        assert (np.abs(la - lc) <= lbound).all()


def test_block_permutation_is_bitwise_invisible():
    b = inputs.paged_inputs(12, 8, 2, 128, seq_len_range=(1, 900), seed=61)
    o1, l1 = run(b)
    k2, v2, t2 = inputs.permute_blocks(b, seed=62)
    b2 = dict(b, k_cache=k2, v_cache=v2, block_table=t2)
    o2, l2 = run(b2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_poisoned_storage_and_padded_table():
    # spare blocks and tail slots hold NaN; table slots past the length are -1
    b = inputs.paged_inputs(6, 4, 1, 128, seq_lens=[3, 17, 33, 100, 250, 16], seed=63,
                            spare_frac=0.5, max_blocks_per_seq=40)
    assert torch.isnan(b["k_cache"]).any() and (b["block_table"] == -1).any()
    check(b, what="poisoned")


def test_empty_sequence():
    b = inputs.paged_inputs(3, 4, 2, 128, seq_lens=[0, 5, 40], seed=64)
    o, lse = run(b)
    assert torch.equal(o[0].float(), torch.zeros_like(o[0].float()))
    assert torch.isinf(lse[0]).all() and (lse[0] < 0).all()
    ro, _, _ = reference(b)
    assert_close(o[1:], ro[1:], torch.bfloat16, "empty neighbours")


def test_deterministic():
    b = inputs.paged_inputs(16, 12, 2, 128, seq_len_range=(1, 3000), seed=65)
    o1, l1 = run(b)
    o2, l2 = run(b)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_query_start_loc_all_ones_same_as_null():
    b = inputs.paged_inputs(10, 8, 2, 128, seq_len_range=(1, 600), seed=66)
    o1, l1 = run(b)
    o2, l2 = run(b, with_qsl=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_workspace_too_small_is_an_error():
    b = to_dev(inputs.paged_inputs(4, 8, 2, 128, seq_len_range=(1, 100), seed=67))
    ws = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(attn.AttnError) as e:
        attn.decode_paged(b["q"], b["k_cache"], b["v_cache"], b["block_table"], b["seq_lens"],
                          max_seq_len=b["max_seq_len"], workspace=ws)
    assert e.value.status == -5



def test_workspace_reuse_across_calls():
    # One workspace serves several calls with different batches, filled with
    # garbage first: its contents need no initialisation.
    nseq, Hq, Hkv, d, max_len = 12, 8, 2, 128, 2000
    ws = torch.full((attn.decode_paged_workspace_size(nseq, Hq, Hkv, d, max_len, 128),), 0xAB,
                    dtype=torch.uint8, device=DEV)
    for seed in (80, 81, 82):
        b = inputs.paged_inputs(nseq, Hq, Hkv, d, seq_len_range=(1, max_len), seed=seed,
                                max_blocks_per_seq=-(-max_len // 16))
        bd = to_dev(b)
        o = attn.decode_paged(bd["q"], bd["k_cache"], bd["v_cache"], bd["block_table"],
                              bd["seq_lens"], max_seq_len=max_len, partition_size=128,
                              workspace=ws)
        torch.cuda.synchronize()
        ro, _, _ = reference(b)
        assert_close(o, ro, torch.bfloat16, f"reuse seed={seed}")


def test_large_batch_partition_major_path():
    # More than 1024 sequences: workgroups use the partition-major order
    # instead of the packed item list; mix of lengths including empty.
    n = 1100
    lens = [((i * 37) % 300) for i in range(n)]
    b = inputs.paged_inputs(n, 4, 2, 64, seq_lens=lens, seed=90)
    for P in (0, 64):
        o, lse = run(b, partition_size=P)
        ro, rl, bound = reference(b)
        assert_close(o, ro, torch.bfloat16, f"1100 seqs P={P}")
        assert_lse_close(lse, rl, bound, f"1100 seqs P={P}")
