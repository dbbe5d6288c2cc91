"""The chunk rows' work plan fits the room the host reserves for it.

attn_paged_workspace_size reserves, for a batch with chunk rows (q_len >= 2)
of at most 2048 sequences, 16 bytes per head group after a 16-byte header,
for a bound on the number of head groups computed from host arguments only.
The planning kernel fills that list from the device's seq_lens and
query_start_loc. Here the number of head groups it lists is re-derived in
Python from the same rule (256-row query tiles, 64-key tiles, pieces of at
least 64 tiles sized by the chunk work's share per compute unit of 256) for
many random batches, and checked against the reserved room. Host logic only:
no device call."""

import random

import pytest

import transformer_attention_tiled_amd as attn

PPBM, BN, PLAN_WGS, MIN_PIECE = 256, 64, 256, 64


def tiles_of(L, q_len, qt):
    last_q = min((qt + 1) * PPBM, q_len)
    return (min(L, L - q_len + last_q) + BN - 1) // BN


def head_groups(seqs, Hq, Hkv, chunk_pieces):
    chunk = [(L, q) for L, q in seqs if q >= 2]
    items = [(L, q, qt) for L, q in chunk for qt in range(-(-q // PPBM))]
    if chunk_pieces > 1:
        tot = sum(tiles_of(L, q, qt) for L, q, qt in items)
        target = max(MIN_PIECE, (tot * Hq + PLAN_WGS - 1) // PLAN_WGS)
    else:
        target = None
    n = 0
    for L, q, qt in items:
        t = tiles_of(L, q, qt)
        pieces = 1 if target is None else min(chunk_pieces, max(1, (t - 1) // target + 1))
        n += Hkv * pieces
    return n


def plan_room(num_seqs, num_tokens, Hq, Hkv, max_seq_len, max_query_len):
    # the plan is what attn_paged_workspace_size adds to the decode partials
    # and (when max_seq_len > 4096) the pieces' partial results
    full = attn.paged_workspace_size(num_seqs, num_tokens, Hq, Hkv, 128, max_seq_len,
                                     max_query_len)
    dec = attn.decode_paged_workspace_size(num_seqs, Hq, Hkv, 128, max_seq_len)
    pieces = -(-max_seq_len // 4096)
    part = 0
    if pieces >= 2:
        rows = num_tokens * Hq * pieces
        part = -(-rows * 128 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    plan_bytes = full - dec - part
    assert plan_bytes > 0 and plan_bytes % 256 == 0
    return (plan_bytes - 16) // 16, pieces if pieces >= 2 else 1


@pytest.mark.parametrize("seed", range(6))
def test_plan_fits_the_reserved_room(seed):
    rng = random.Random(seed)
    worst = 0.0
    for _ in range(400):
        ns = rng.randint(1, 80)
        Hkv = rng.choice([1, 2, 8])
        Hq = Hkv * rng.choice([1, 4, 6, 16])
        seqs = []
        for _ in range(ns):
            q = rng.choice([0, 1, 1, 2, 3, 17, 255, 256, 257, 512, 1000, 3000])
            L = q + rng.choice([0, 7, 4000, 4096, 30000, rng.randint(0, 70000)])
            seqs.append((L, q))
        num_tokens = sum(q for _, q in seqs)
        max_q = max(q for _, q in seqs)
        if num_tokens < 1 or max_q < 2:
            continue
        max_len = max(L for L, _ in seqs)
        room, chunk_pieces = plan_room(ns, num_tokens, Hq, Hkv, max_len, max_q)
        need = head_groups(seqs, Hq, Hkv, chunk_pieces)
        assert need <= room, (ns, Hq, Hkv, need, room)
        worst = max(worst, need / room)
    assert worst > 0.3  # the bound is not vacuous on these batches


def test_single_long_chunk_is_split_and_fits():
    # one 512-row chunk after 32 256 cached tokens, Hq = 32, Hkv = 8: its two
    # query tiles have 508 and 512 key tiles, so the share per compute unit
    # is ceil(1020 * 32 / 256) = 128 tiles and each tile splits into 4 pieces
    seqs = [(32768, 512)]
    room, pieces = plan_room(1, 512, 32, 8, 32768, 512)
    assert tiles_of(32768, 512, 0) == 508 and tiles_of(32768, 512, 1) == 512
    need = head_groups(seqs, 32, 8, pieces)
    assert need == 8 * 2 * 4 and need <= room
