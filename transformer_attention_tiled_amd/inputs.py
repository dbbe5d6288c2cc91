"""Seeded synthetic inputs for attention prefill and paged decode.

This module only draws random numbers and lays out index structures; it holds
none of the attention arithmetic. Both the HIP path and the CPU oracle consume
what it returns, so neither depends on the other.

Recipe (the same for every consumer):

* Values: i.i.d. N(0, 1) drawn in fp32 by ``torch.randn`` with a
  ``torch.Generator`` seeded with ``seed``, then rounded to the element type
  (bf16 by round-to-nearest-even). Large paged pools may be drawn directly on
  the GPU with a CUDA generator (``device="cuda"``); that stream differs from
  the CPU one but is just as fixed by the seed.
* Prefill draw order: q, k, v.
* Paged draw order: seq_lens (uniform integers in [lo, hi]), a random
  permutation of all physical blocks, then q, k_cache, v_cache.
* Physical pool: sum over sequences of ceil(L_n / 16) blocks plus
  ``spare_frac`` spare blocks, shuffled; sequence n takes the next
  ceil(L_n / 16) entries of the permutation as its table row; unused table
  slots hold -1. With ``poison=True`` the spare blocks and every cache slot
  past a sequence's length hold NaN, so any read of data the method must not
  touch shows up in the result.
"""

import math

import torch

BLOCK_SIZE = 16


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def prefill_inputs(B, Hq, Hkv, T, d, dtype=torch.bfloat16, seed=0, device="cpu"):
    """q [B,Hq,T,d], k and v [B,Hkv,T,d], i.i.d. N(0,1) rounded to ``dtype``."""
    g = _gen(seed, device)
    q = torch.randn(B, Hq, T, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    k = torch.randn(B, Hkv, T, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    v = torch.randn(B, Hkv, T, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    return q, k, v


def paged_inputs(num_seqs, Hq, Hkv, d, seq_len_range=None, seq_lens=None, q_lens=None,
                 dtype=torch.bfloat16, seed=0, spare_frac=0.05, poison=True,
                 device="cpu", max_blocks_per_seq=None):
    """A paged batch.

    Either ``seq_len_range=(lo, hi)`` (drawn) or ``seq_lens`` (given) fixes the
    lengths. ``q_lens`` (default all 1) gives the query tokens per sequence;
    query_start_loc is their running sum.

    Returns a dict with q [num_tokens,Hq,d], k_cache/v_cache
    [num_blocks,Hkv,16,d], block_table int32 [num_seqs,max_blocks_per_seq],
    seq_lens int32, query_start_loc int32 [num_seqs+1], and the host-side
    bounds max_seq_len, max_query_len, max_blocks_per_seq, num_blocks.
    """
    g = _gen(seed, device)
    if seq_lens is None:
        lo, hi = seq_len_range
        lens = torch.randint(lo, hi + 1, (num_seqs,), generator=g, device=device)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int64, device=device)
    lens_host = [int(x) for x in lens.cpu().tolist()]
    if q_lens is None:
        q_lens = [1] * num_seqs
    q_lens = [int(x) for x in q_lens]
    nblk = [math.ceil(L / BLOCK_SIZE) for L in lens_host]
    used = sum(nblk)
    num_blocks = max(1, used + int(math.ceil(used * spare_frac)))
    perm = torch.randperm(num_blocks, generator=g, device=device).cpu()
    mbps = max(1, max(nblk) if nblk else 1)
    if max_blocks_per_seq is not None:
        mbps = max(mbps, int(max_blocks_per_seq))
    table = torch.full((num_seqs, mbps), -1, dtype=torch.int32)
    off = 0
    for n, nb in enumerate(nblk):
        table[n, :nb] = perm[off:off + nb].to(torch.int32)
        off += nb
    num_tokens = sum(q_lens)
    q = torch.randn(num_tokens, Hq, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    k_cache = _randn_big((num_blocks, Hkv, BLOCK_SIZE, d), g, device, dtype)
    v_cache = _randn_big((num_blocks, Hkv, BLOCK_SIZE, d), g, device, dtype)
    if poison:
        spare = perm[off:].to(device)
        if spare.numel():
            k_cache[spare] = float("nan")
            v_cache[spare] = float("nan")
        for n, L in enumerate(lens_host):
            if L % BLOCK_SIZE:
                last = int(table[n, nblk[n] - 1])
                k_cache[last, :, L % BLOCK_SIZE:, :] = float("nan")
                v_cache[last, :, L % BLOCK_SIZE:, :] = float("nan")
    qsl = torch.zeros(num_seqs + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    return {
        "q": q,
        "k_cache": k_cache,
        "v_cache": v_cache,
        "block_table": table.to(device),
        "seq_lens": torch.tensor(lens_host, dtype=torch.int32, device=device),
        "query_start_loc": qsl.to(device),
        "max_seq_len": max(lens_host) if lens_host else 0,
        "max_query_len": max(q_lens) if q_lens else 0,
        "max_blocks_per_seq": mbps,
        "num_blocks": num_blocks,
        "q_lens": q_lens,
        "seq_lens_host": lens_host,
    }


def _randn_big(shape, g, device, dtype):
    """N(0,1) in ``dtype``, drawn in fp32 chunks so that huge pools fit in memory."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    rows_per_chunk = max(1, (1 << 26) // max(1, flat.shape[1]))
    for r0 in range(0, shape[0], rows_per_chunk):
        r1 = min(shape[0], r0 + rows_per_chunk)
        flat[r0:r1] = torch.randn(r1 - r0, flat.shape[1], generator=g, device=device,
                                  dtype=torch.float32).to(dtype)
    return out


def permute_blocks(batch, seed):
    """The same logical batch with its physical blocks shuffled again.

    Returns new (k_cache, v_cache, block_table): physical block p moves to
    position pi[p], and the table is rewritten so that every logical position
    still names the same values.
    """
    g = _gen(seed, "cpu")
    nb = batch["k_cache"].shape[0]
    pi = torch.randperm(nb, generator=g)
    inv = torch.empty_like(pi)
    inv[pi] = torch.arange(nb)
    dev = batch["k_cache"].device
    k_new = torch.empty_like(batch["k_cache"])
    v_new = torch.empty_like(batch["v_cache"])
    k_new[pi.to(dev)] = batch["k_cache"]
    v_new[pi.to(dev)] = batch["v_cache"]
    t = batch["block_table"].cpu().to(torch.int64)
    t_new = torch.where(t >= 0, pi[t.clamp(min=0)], t).to(torch.int32)
    return k_new, v_new, t_new.to(batch["block_table"].device)


def mixed_batch_inputs(n_chunks=8, chunk_len=512, n_decode=256, decode_len_range=(1024, 32768),
                       Hq=32, Hkv=8, d=128, seed=5, device="cpu", poison=False,
                       chunk_len_range=None):
    """Mixed paged batch: ``n_chunks`` prefill chunks of ``chunk_len`` new
    tokens followed by ``n_decode`` single-token decodes whose lengths are
    uniform integers in ``decode_len_range`` (drawn on the CPU from ``seed``).
    The chunks have no prior context (their sequences are ``chunk_len``
    long), unless ``chunk_len_range`` is given: then each chunk's sequence
    length is a uniform integer in that range (drawn after the decode
    lengths), so the chunk follows L - chunk_len cached tokens. The K/V of
    every token, new ones included, is already in the pool. One shuffled pool
    holds every sequence; on ``device="cuda"`` the values are drawn there.
    """
    g = torch.Generator().manual_seed(int(seed))
    lo, hi = decode_len_range
    dec_lens = torch.randint(lo, hi + 1, (n_decode,), generator=g).tolist()
    if chunk_len_range is None:
        chunk_lens = [chunk_len] * n_chunks
    else:
        clo, chi = chunk_len_range
        chunk_lens = torch.randint(max(clo, chunk_len), chi + 1, (n_chunks,), generator=g).tolist()
    seq_lens = chunk_lens + dec_lens
    q_lens = [chunk_len] * n_chunks + [1] * n_decode
    return paged_inputs(n_chunks + n_decode, Hq, Hkv, d, seq_lens=seq_lens, q_lens=q_lens,
                        seed=seed, device=device, poison=poison)


def new_kv_rows(num_tokens, Hkv, d, seed, dtype=torch.bfloat16, device="cpu"):
    """Keys and values of new tokens for a cache append: k_new, v_new
    [num_tokens, Hkv, d], i.i.d. N(0,1) rounded to ``dtype`` (draw order k, v)."""
    g = _gen(seed, device)
    k = torch.randn(num_tokens, Hkv, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    v = torch.randn(num_tokens, Hkv, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    return k, v


def norm_inputs(rows, hidden, seed, dtype=torch.bfloat16, device="cpu"):
    """Inputs of the residual-add + RMSNorm fusion: x and residual [rows, hidden]
    i.i.d. N(0,1), weight [hidden] = 1 + 0.1 N(0,1), each rounded to ``dtype``
    (draw order x, residual, weight)."""
    g = _gen(seed, device)
    x = torch.randn(rows, hidden, generator=g, device=device, dtype=torch.float32).to(dtype)
    r = torch.randn(rows, hidden, generator=g, device=device, dtype=torch.float32).to(dtype)
    w = (1.0 + 0.1 * torch.randn(hidden, generator=g, device=device, dtype=torch.float32)).to(dtype)
    return x, r, w


def compact_sequences(batch, seqs):
    """CPU copy of just the physical blocks that the given sequences use.

    Returns (k_cache, v_cache, block_table, seq_lens, q, query_start_loc) on
    the CPU for the sub-batch ``seqs`` (in that order), with the table
    rewritten onto the compact pool. Only data movement: nothing is computed.
    """
    table = batch["block_table"].cpu()
    lens = batch["seq_lens"].cpu()
    qsl = batch["query_start_loc"].cpu()
    used, rows = [], []
    for n in seqs:
        nb = math.ceil(int(lens[n]) / BLOCK_SIZE)
        rows.append((len(used), nb))
        used.extend(int(x) for x in table[n, :nb])
    idx = torch.tensor(used, dtype=torch.int64)
    dev = batch["k_cache"].device
    k = batch["k_cache"][idx.to(dev)].cpu()
    v = batch["v_cache"][idx.to(dev)].cpu()
    width = max(nb for _, nb in rows)
    new_table = torch.full((len(seqs), max(1, width)), -1, dtype=torch.int32)
    for i, (start, nb) in enumerate(rows):
        new_table[i, :nb] = torch.arange(start, start + nb, dtype=torch.int32)
    q_parts, new_qsl = [], [0]
    for n in seqs:
        t0, t1 = int(qsl[n]), int(qsl[n + 1])
        q_parts.append(batch["q"][t0:t1].cpu())
        new_qsl.append(new_qsl[-1] + (t1 - t0))
    return (k, v, new_table, lens[list(seqs)].to(torch.int32), torch.cat(q_parts),
            torch.tensor(new_qsl, dtype=torch.int32))
