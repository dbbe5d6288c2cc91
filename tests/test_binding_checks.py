"""The Python binding rejects, on the host and before any library or device
call, tensors that the C ABI cannot see are wrong: the wrong device, element
type, layout or shape. These run on the CPU: every case raises ValueError
before a pointer is handed over (and the last case of each entry point,
correct in every other way, is rejected for being on the CPU)."""

import pytest
import torch

import transformer_attention_tiled_amd as attn

bf16, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64


def t(*shape, dtype=bf16):
    return torch.zeros(*shape, dtype=dtype)


def prefill_args(**kw):
    a = dict(q=t(1, 4, 8, 64), k=t(1, 2, 8, 64), v=t(1, 2, 8, 64), o=None, lse=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,msg", [
    (dict(q=t(4, 8, 64)), "dimensions"),
    (dict(k=t(1, 2, 9, 64)), "shape"),                 # k shorter/longer than q
    (dict(k=t(2, 2, 8, 64)), "shape"),                 # batch mismatch
    (dict(k=t(1, 2, 8, 128)), "shape"),                # head size mismatch
    (dict(k=t(1, 2, 8, 64, dtype=f32)), "bfloat16"),   # k dtype differs from q
    (dict(v=t(1, 2, 8, 32)), "shape"),
    (dict(v=t(1, 2, 64, 8).transpose(2, 3)), "contiguous"),
    (dict(o=t(1, 4, 8, 64, dtype=f32)), "bfloat16"),
    (dict(o=t(1, 4, 7, 64)), "shape"),
    (dict(lse=t(1, 4, 8)), "float32"),                 # a bf16 lse would be overrun by fp32 writes
    (dict(lse=t(1, 4, 7, dtype=f32)), "shape"),
    (dict(q=t(1, 4, 64, 8).transpose(2, 3)), "contiguous"),
    (dict(), "GPU"),                                   # everything right, but on the CPU
])
def test_prefill_rejects(kw, msg):
    a = prefill_args(**kw)
    with pytest.raises(ValueError, match=msg):
        attn.prefill(a["q"], a["k"], a["v"], a["o"], lse=a["lse"])


def paged_args(**kw):
    a = dict(q=t(3, 4, 128), k_cache=t(10, 2, 16, 128), v_cache=t(10, 2, 16, 128),
             block_table=t(3, 4, dtype=i32), seq_lens=t(3, dtype=i32), query_start_loc=None,
             o=None, lse=None, workspace=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,msg", [
    (dict(q=t(3, 4, 2, 64)), "dimensions"),
    (dict(k_cache=t(10, 2, 16, 64), v_cache=t(10, 2, 16, 64)), "head size"),
    (dict(v_cache=t(11, 2, 16, 128)), "shape"),
    (dict(k_cache=t(10, 2, 16, 128, dtype=f32)), "bfloat16"),
    (dict(block_table=t(3, 4, dtype=i64)), "int32"),      # would be read as the wrong entries
    (dict(seq_lens=t(3, dtype=i64)), "int32"),
    (dict(block_table=t(2, 4, dtype=i32)), "rows"),
    (dict(block_table=t(4, 3, dtype=i32).t()), "contiguous"),
    (dict(query_start_loc=t(3, dtype=i32)), "shape"),     # needs num_seqs + 1 entries
    (dict(query_start_loc=t(4, dtype=i64)), "int32"),
    (dict(o=t(3, 4, 64)), "shape"),
    (dict(lse=t(3, 4)), "float32"),
    (dict(lse=t(4, 3, dtype=f32)), "shape"),
    (dict(workspace=t(64, 2, dtype=torch.uint8).t()), "contiguous"),
    (dict(), "GPU"),
])
def test_decode_paged_rejects(kw, msg):
    a = paged_args(**kw)
    with pytest.raises(ValueError, match=msg):
        attn.decode_paged(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"],
                          max_seq_len=64, query_start_loc=a["query_start_loc"], o=a["o"],
                          lse=a["lse"], workspace=a["workspace"])


def append_args(**kw):
    a = dict(k_new=t(3, 2, 128), v_new=t(3, 2, 128), k_cache=t(10, 2, 16, 128),
             v_cache=t(10, 2, 16, 128), block_table=t(3, 4, dtype=i32), seq_lens=t(3, dtype=i32),
             query_start_loc=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,msg", [
    (dict(v_new=t(3, 2, 64)), "shape"),
    (dict(k_cache=t(10, 4, 16, 128), v_cache=t(10, 4, 16, 128)), "Hkv"),
    (dict(v_cache=t(10, 2, 16, 128, dtype=f32)), "bfloat16"),
    (dict(block_table=t(3, 4, dtype=i64)), "int32"),
    (dict(seq_lens=t(3, 1, dtype=i32)), "dimensions"),
    (dict(query_start_loc=t(4, dtype=i64)), "int32"),
    (dict(), "GPU"),
])
def test_kv_append_rejects(kw, msg):
    a = append_args(**kw)
    with pytest.raises(ValueError, match=msg):
        attn.kv_append(a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["block_table"],
                       a["seq_lens"], query_start_loc=a["query_start_loc"])


@pytest.mark.parametrize("kw,msg", [
    (dict(residual=t(4, 32)), "shape"),
    (dict(weight=t(65)), "shape"),
    (dict(weight=t(64, dtype=f32)), "bfloat16"),
    (dict(out=t(4, 64, dtype=f32)), "bfloat16"),
    (dict(residual_out=t(64, 4).t()), "contiguous"),
    (dict(), "GPU"),
])
def test_add_rmsnorm_rejects(kw, msg):
    a = dict(x=t(4, 64), residual=t(4, 64), weight=t(64), out=None, residual_out=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        attn.add_rmsnorm(a["x"], a["residual"], a["weight"], 1e-6, out=a["out"],
                         residual_out=a["residual_out"])
