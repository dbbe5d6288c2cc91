"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad requests on the host before any HIP call (so these run without a
GPU; no test here launches a kernel)."""

import ctypes
import os
import re

import pytest

import transformer_attention_tiled_amd as attn
from transformer_attention_tiled_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1

# Fake device addresses: never dereferenced, because validation fails first.
P = 0x100000
P2 = 0x900000
P3 = 0x1100000
P4 = 0x1900000


@pytest.fixture(scope="module")
def lib():
    return attn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_prefill", "attn_decode_paged", "attn_status_string",
            "attn_decode_paged_workspace_size", "attn_decode_paged_partition_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH):
        s = attn.status_string(code)
        assert s and s != "unknown status"
    assert attn.status_string(12345) == "unknown status"


def prefill(lib, q=P, k=P2, v=P3, o=P4, B=1, Hq=2, Hkv=2, T=16, d=64, scale=0.125, causal=1,
            dtype=BF16, lse=None):
    return lib.attn_prefill(q, k, v, o, B, Hq, Hkv, T, d, ctypes.c_float(scale), causal, dtype,
                            lse, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(B=0), SHAPE), (dict(T=0), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=0), SHAPE),
    (dict(Hq=6, Hkv=4), SHAPE), (dict(causal=2), SHAPE),
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(dtype=7), UNSUP),
    (dict(scale=0.0), UNSUP), (dict(scale=-1.0), UNSUP), (dict(scale=float("nan")), UNSUP),
    (dict(scale=float("inf")), UNSUP),
    (dict(q=P + 8), ALIGN), (dict(o=P4 + 4), ALIGN), (dict(lse=P + 2), ALIGN),
    (dict(o=P), SHAPE),            # output overlaps q
    (dict(lse=P4 + 64), SHAPE),    # lse overlaps o
    (dict(B=2**20, Hq=2**20, Hkv=2**20, T=2**20), SHAPE),  # byte counts overflow int64
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(lib, **kw) == code


def decode(lib, q=P, kc=P2, vc=P3, table=P4, seq_lens=P4 + 0x10000, qsl=None, o=P4 + 0x20000,
           num_seqs=4, num_tokens=4, Hq=8, Hkv=2, d=128, block_size=16, mbps=8, max_seq_len=128,
           max_query_len=1, num_blocks=64, scale=0.1, dtype=BF16, partition_size=0, lse=None,
           ws=0x4000000, ws_bytes=1 << 30):
    return lib.attn_decode_paged(q, kc, vc, table, seq_lens, qsl, o, num_seqs, num_tokens, Hq,
                                 Hkv, d, block_size, mbps, max_seq_len, max_query_len, num_blocks,
                                 ctypes.c_float(scale), dtype, partition_size, lse, ws, ws_bytes,
                                 None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL), (dict(table=None), NULL),
    (dict(seq_lens=None), NULL), (dict(o=None), NULL),
    (dict(dtype=F32), UNSUP), (dict(d=80), UNSUP), (dict(block_size=32), UNSUP),
    (dict(partition_size=4096 + 16), UNSUP),
    (dict(Hq=34, Hkv=2), UNSUP), (dict(scale=0.0), UNSUP),
    (dict(num_seqs=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(max_seq_len=0), SHAPE),
    (dict(mbps=7), SHAPE), (dict(num_blocks=0), SHAPE), (dict(max_query_len=2), SHAPE),
    (dict(num_tokens=3), SHAPE), (dict(partition_size=8), SHAPE), (dict(partition_size=-16), SHAPE),
    (dict(max_query_len=200, qsl=P4 + 0x30000, num_tokens=300), SHAPE),
    (dict(q=P + 4), ALIGN), (dict(table=P4 + 2), ALIGN), (dict(ws=0x4000000 + 16), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS),
    (dict(o=P), SHAPE),                                  # o overlaps q
    (dict(o=P4), SHAPE),                                 # o overlaps the block table
    (dict(lse=P4 + 0x10000), SHAPE),                     # lse overlaps seq_lens
    (dict(lse=P4 + 0x20000), SHAPE),                     # lse overlaps o
    (dict(ws=P2), SHAPE),                                # workspace overlaps the K cache
    (dict(ws=P4 + 0x10000), SHAPE),                      # workspace overlaps seq_lens
    (dict(ws=P4 + 0x20000), SHAPE),                      # workspace overlaps o
    (dict(qsl=P4 + 0x20000, max_query_len=2), SHAPE),    # o overlaps query_start_loc
    (dict(num_blocks=2**60), SHAPE),                     # cache bytes overflow int64
    (dict(num_seqs=2**31 - 1, num_tokens=2**31 - 1, mbps=2**31 - 1, ws_bytes=2**60),
     SHAPE),                                             # block-table bytes overflow int64
    (dict(num_seqs=2**31 - 1, num_tokens=2**31 - 1, Hq=2**30, Hkv=2**30,
          max_seq_len=2**31 - 16, mbps=2**27, ws_bytes=2**63), SHAPE),  # policy estimate
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


def test_workspace_size_and_partition_policy():
    # pure host functions
    P_auto = attn.decode_paged_partition_size(64, 2, 4096)
    assert P_auto > 0 and P_auto % 16 == 0
    assert attn.decode_paged_partition_size(0, 2, 4096) == 0
    # sizes whose estimate or byte counts overflow int64 are out of range
    assert attn.decode_paged_partition_size(2**31 - 1, 2**30, 2**31 - 1) == 0
    assert attn.decode_paged_workspace_size(2**31 - 1, 2**30, 2**30, 128, 2**31 - 1, 0) == 0
    assert attn.decode_paged_workspace_size(2**31 - 1, 2**31 - 1, 1, 128, 2**31 - 1, 16) == 0
    ws = attn.decode_paged_workspace_size(64, 12, 2, 128, 4096, 256)
    parts = 4096 // 256
    rows = 64 * 12 * parts
    # partial outputs, then partial lse
    expect = -(-rows * 128 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert ws == expect
    assert attn.decode_paged_workspace_size(64, 12, 2, 128, 4096, 4096 + 16) == 0  # too long
    for args in ((64, 2, 4096), (1, 1, 1), (256, 8, 32768), (3, 2, 100000)):
        P = attn.decode_paged_partition_size(*args)
        assert 16 <= P <= 4096 and P % 16 == 0
    assert attn.decode_paged_workspace_size(64, 12, 2, 128, 4096, 8) == 0    # not a multiple of 16
    assert attn.decode_paged_workspace_size(64, 12, 2, 96, 4096, 0) == 0     # d unsupported
    # automatic partition length: the workspace query and the launch agree
    assert (attn.decode_paged_workspace_size(64, 12, 2, 128, 4096, 0)
            == attn.decode_paged_workspace_size(64, 12, 2, 128, 4096, P_auto))


def test_binding_raises_attn_error_with_code(lib):
    e = _binding.AttnError(SHAPE, "attn_prefill")
    assert e.status == SHAPE and "ATTN_ERR_SHAPE" in str(e)


def append(lib, kn=P, vn=P2, kc=P3, vc=P4, table=P4 + 0x40000000, seq_lens=P4 + 0x40010000,
           qsl=None, num_seqs=4, num_tokens=4, Hkv=2, d=128, block_size=16, mbps=8,
           max_query_len=1, num_blocks=64, dtype=BF16):
    return lib.attn_kv_append(kn, vn, kc, vc, table, seq_lens, qsl, num_seqs, num_tokens, Hkv, d,
                              block_size, mbps, max_query_len, num_blocks, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), NULL), (dict(vn=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL),
    (dict(table=None), NULL), (dict(seq_lens=None), NULL),
    (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP), (dict(block_size=32), UNSUP),
    (dict(num_seqs=0), SHAPE), (dict(num_tokens=0), SHAPE), (dict(Hkv=0), SHAPE),
    (dict(num_blocks=0), SHAPE), (dict(mbps=0), SHAPE), (dict(max_query_len=0), SHAPE),
    (dict(max_query_len=2), SHAPE),             # several rows per sequence need query_start_loc
    (dict(num_tokens=3), SHAPE),                # fewer rows than sequences
    (dict(max_query_len=5, qsl=P4 + 0x40020000), SHAPE),  # bound above num_tokens
    (dict(kn=P + 8), ALIGN), (dict(kc=P3 + 4), ALIGN), (dict(table=P4 + 0x40000002), ALIGN),
    (dict(kn=P3), SHAPE),                       # new rows overlap the K cache
    (dict(vc=P3 + 0x1000), SHAPE),              # the two caches overlap
    (dict(table=P3 + 0x1000), SHAPE),           # the block table lies inside the K cache
    (dict(seq_lens=P4 + 0x100), SHAPE),         # seq_lens lies inside the V cache
    (dict(qsl=P3 + 0x2000), SHAPE),             # query_start_loc lies inside the K cache
    (dict(num_blocks=2**60), SHAPE),            # cache bytes overflow int64
])
def test_kv_append_rejects(lib, kw, code):
    assert append(lib, **kw) == code


def add_rmsnorm(lib, x=P, r=P2, w=P3, out=P4, rout=P4 + 0x10000000, rows=4, hidden=4096,
                eps=1e-6, dtype=BF16):
    return lib.attn_add_rmsnorm(x, r, w, out, rout, rows, hidden, ctypes.c_float(eps), dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(r=None), NULL), (dict(w=None), NULL), (dict(out=None), NULL),
    (dict(rout=None), NULL),
    (dict(dtype=F32), UNSUP), (dict(hidden=16384 + 8), UNSUP), (dict(eps=-1.0), UNSUP),
    (dict(eps=float("nan")), UNSUP),
    (dict(rows=0), SHAPE), (dict(hidden=0), SHAPE), (dict(hidden=100), SHAPE),
    (dict(x=P + 8), ALIGN), (dict(w=P3 + 4), ALIGN), (dict(rout=P4 + 0x10000002), ALIGN),
    (dict(out=P), SHAPE),                  # output overlaps x
    (dict(rout=P), SHAPE),                 # residual output overlaps x
    (dict(rout=P2 + 0x100), SHAPE),        # partial overlap with residual (only exact in place is allowed)
])
def test_add_rmsnorm_rejects(lib, kw, code):
    assert add_rmsnorm(lib, **kw) == code


def decode_noalloc(lib, q=P, kc=P2, vc=P3, table=P4, seq_lens=P4 + 0x40000000, qsl=None,
                   o=P4 + 0x50000000, num_seqs=4, num_tokens=4, Hq=8, Hkv=2, d=128,
                   block_size=16, mbps=8, max_seq_len=128, max_query_len=1, num_blocks=64,
                   scale=0.088, dtype=BF16, partition_size=0, lse=None):
    return lib.attn_decode_paged_noalloc(q, kc, vc, table, seq_lens, qsl, o, num_seqs,
                                         num_tokens, Hq, Hkv, d, block_size, mbps, max_seq_len,
                                         max_query_len, num_blocks, ctypes.c_float(scale), dtype,
                                         partition_size, lse, None)


SCRATCH = -7


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(table=None), NULL),
    (dict(dtype=F32), UNSUP), (dict(d=96), UNSUP), (dict(block_size=8), UNSUP),
    (dict(Hq=7), SHAPE), (dict(max_seq_len=0), SHAPE), (dict(mbps=7), SHAPE),
    (dict(q=P + 8), ALIGN),
    (dict(o=P), SHAPE),                                  # output over q
    # 2000 sequences of 32768 tokens in 16-token partitions: far beyond the
    # fixed array, refused before the array's address is even looked up
    (dict(num_seqs=2000, num_tokens=2000, Hq=32, Hkv=8, mbps=2048, max_seq_len=32768,
          partition_size=16, seq_lens=P4 + 0x60000000, o=P4 + 0x70000000), SCRATCH),
])
def test_decode_noalloc_rejects_on_the_host(lib, kw, code):
    assert decode_noalloc(lib, **kw) == code


def test_noalloc_limit_matches_header(lib):
    text = open(HEADER).read()
    assert "ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert attn.DECODE_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert attn.status_string(SCRATCH) != "unknown status"


def test_paged_workspace_size_adds_chunk_plan_and_pieces(lib):
    dec = attn.decode_paged_workspace_size(264, 32, 8, 128, 32768, 0)
    # one query per sequence: the same as the decode-only size
    assert attn.paged_workspace_size(264, 264, 32, 8, 128, 32768, 1, 0) == dec

    def plan(num_seqs, num_tokens, Hq, Hkv, split):
        # head groups: Hkv per chunk query tile (at most min(num_seqs,
        # num_tokens / 2) + ceil(num_tokens / 256) of them) and per extra key
        # piece (at most ceil(256 / Hq) per KV head); 16 bytes each after a
        # 16-byte header, rounded up to 256 bytes
        cap = Hkv * (min(num_seqs, num_tokens // 2) + -(-num_tokens // 256)
                     + (-(-256 // Hq) if split else 0))
        return -(-(16 + 16 * cap) // 256) * 256

    # chunk rows and keys beyond one 4096-key piece: the plan, then room for
    # the pieces' fp32 partial outputs and lse, [num_tokens][Hq][pieces][d + 1]
    full = attn.paged_workspace_size(264, 4352, 32, 8, 128, 32768, 512, 0)
    pieces = 32768 // 4096
    rows = 4352 * 32 * pieces
    assert full == dec + plan(264, 4352, 32, 8, True) + -(-rows * 128 * 4 // 256) * 256 + \
        -(-rows * 4 // 256) * 256
    # keys within one piece: the plan only
    assert attn.paged_workspace_size(264, 4352, 32, 8, 128, 4096, 512, 0) == \
        attn.decode_paged_workspace_size(264, 32, 8, 128, 4096, 0) + plan(264, 4352, 32, 8, False)
    # a batch beyond 2048 sequences: nothing extra (one workgroup per possible
    # chunk query tile and head, no plan and no split)
    assert attn.paged_workspace_size(2049, 4352, 32, 8, 128, 32768, 512, 0) == \
        attn.decode_paged_workspace_size(2049, 32, 8, 128, 32768, 0)
    assert attn.paged_workspace_size(264, 0, 32, 8, 128, 32768, 512, 0) == 0
    assert attn.paged_workspace_size(264, 4352, 12, 5, 128, 32768, 512, 0) == 0  # Hq % Hkv
