"""Plain fp64 attention on the CPU (numpy). Test infrastructure only.

Definitions followed (page titles and sections of the source pages):

* Naive causal attention, "Hugging Face attention profiling guide", second
  paragraph: S = Q @ K^T, then the scaling, then the causal mask
  (masked_fill with -inf where the key lies after the query), then a row
  softmax, then the product with V.
* The score matrix has T x T entries per head, "Fast attention kernels and
  operator fusion", section "FlashAttention-style attention and paged
  attention". The oracle materialises it on purpose (in row blocks, so that
  long sequences fit in memory); the row blocking does not reorder any
  arithmetic within a row.
* Paged KV cache, same page and section: storage in fixed 16-token blocks and
  a block table from logical block to physical block; every logical position
  p is translated to (block_table[n, p // block_size], p % block_size).

Readings of points the pages leave open (each is listed with its reason in
the design notes of the repository):

* The scale is an explicit argument (the pages name the scaling step without
  a value; the configurations use 1/sqrt(d)).
* Grouped-query heads: query head h reads KV head h // (Hq // Hkv).
* When a query block is shorter than the key range (chunked prefill, decode),
  the mask is aligned bottom-right: the query at absolute position t sees
  keys 0..t.
* seq_lens counts the cached tokens including the current query's own K/V.
* A query row that sees no key yields output 0 and lse = -inf.

Inputs are converted to float64 exactly (bf16 and fp32 values are exactly
representable), so the oracle sees the very values the GPU sees.
"""

import numpy as np

_ROW_BLOCK = 2048


def _as_f64(x):
    """Exact conversion to a float64 numpy array (accepts numpy or torch CPU tensors)."""
    if hasattr(x, "detach"):  # torch tensor: upcast on the torch side (bf16 has no numpy dtype)
        x = x.detach().to("cpu")
        import torch  # local import: only needed for torch inputs

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _softmax_rows_times_v(S, V):
    """Row softmax of the (already scaled and masked) scores S, then @ V.

    Returns (O, lse). Rows whose entries are all -inf give O = 0 and lse = -inf.
    """
    m = S.max(axis=1, initial=-np.inf)  # a row with no key at all has max -inf
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    P = np.exp(S - m_safe[:, None])  # exp(-inf) = 0 for masked entries
    l = P.sum(axis=1)
    O = np.zeros((S.shape[0], V.shape[1]), dtype=np.float64)
    O[finite] = (P[finite] / l[finite, None]) @ V
    lse = np.full(S.shape[0], -np.inf)
    lse[finite] = m[finite] + np.log(l[finite])
    return O, lse


def _attend(q_rows, K, V, scale, key_limit):
    """Attention of query rows against keys 0..len(K)-1.

    q_rows: [R, d]; K, V: [L, d]; key_limit: None (no mask) or int array [R]
    giving, per row, the last key index the row may see (the causal mask).
    """
    S = scale * (q_rows @ K.T)  # scores, then the scaling step
    if key_limit is not None:
        j = np.arange(K.shape[0])[None, :]
        S = np.where(j > key_limit[:, None], -np.inf, S)  # masked_fill(-inf) for keys after the query
    return _softmax_rows_times_v(S, V)


def prefill(q, k, v, scale, causal=True, rows=None, heads=None):
    """Scaled dot-product attention over contiguous q, k, v.

    q: [B, Hq, T, d]; k, v: [B, Hkv, T, d]. Query head h uses KV head
    h // (Hq // Hkv). With causal=True, query i sees keys 0..i.

    rows: optional sorted list of query indices to evaluate (default: all);
    heads: optional list of query heads to evaluate (default: all).
    Returns (o, lse) with o: [B, Hq, R, d] and lse: [B, Hq, R] (R = len(rows)),
    float64. Heads not evaluated are left as NaN.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    dv = v.shape[-1]  # value width (equal to d in every configuration)
    o = np.full((B, Hq, len(rows), dv), np.nan)
    lse = np.full((B, Hq, len(rows)), np.nan)
    for b in range(B):
        for h in heads:
            g = h // G
            for r0 in range(0, len(rows), _ROW_BLOCK):
                rr = rows[r0:r0 + _ROW_BLOCK]
                # a causal row i only needs keys 0..i; taking the prefix changes nothing
                kv_len = int(rr.max()) + 1 if causal else T
                ob, lb = _attend(q[b, h, rr], k[b, g, :kv_len], v[b, g, :kv_len], scale,
                                 rr if causal else None)
                o[b, h, r0:r0 + len(rr)] = ob
                lse[b, h, r0:r0 + len(rr)] = lb
    return o, lse


def gather_paged_kv(cache, block_table_row, seq_len, block_size=16):
    """Contiguous [seq_len, Hkv, d] view of one sequence of a paged cache.

    cache: [num_blocks, Hkv, block_size, d]. Logical position p lives in
    physical block block_table_row[p // block_size], slot p % block_size.
    """
    table = np.asarray(block_table_row, dtype=np.int64)
    p = np.arange(int(seq_len))
    phys = table[p // block_size]
    slot = p % block_size
    if hasattr(cache, "detach"):  # torch tensor: pick the rows first, then convert them
        import torch  # local import: only needed for torch inputs

        rows = cache.detach()[torch.from_numpy(phys), :, torch.from_numpy(slot), :]
        return _as_f64(rows)  # [L, Hkv, d]
    return np.asarray(cache)[phys, :, slot, :].astype(np.float64)  # [L, Hkv, d]


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale,
                 query_start_loc=None, block_size=16, seqs=None):
    """Attention of the batch's query tokens against a paged KV cache.

    q: [num_tokens, Hq, d]; k_cache, v_cache: [num_blocks, Hkv, block_size, d];
    block_table: int [num_seqs, max_blocks_per_seq]; seq_lens: int [num_seqs].
    query_start_loc: int [num_seqs + 1] (None: one query per sequence). The
    queries of sequence n are the last q_len = qsl[n+1] - qsl[n] positions
    L - q_len .. L - 1 of that sequence (L = seq_lens[n]); the query at
    position t sees keys 0..t.

    seqs: optional list of sequences to evaluate (others' rows stay NaN).
    Returns (o, lse): o [num_tokens, Hq, d], lse [num_tokens, Hq], float64.
    """
    q = _as_f64(q)
    num_tokens, Hq, d = q.shape
    block_table = np.asarray(block_table, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    num_seqs = seq_lens.shape[0]
    if query_start_loc is None:
        qsl = np.arange(num_seqs + 1)
    else:
        qsl = np.asarray(query_start_loc, dtype=np.int64)
    Hkv = k_cache.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.full((num_tokens, Hq, v_cache.shape[-1]), np.nan)
    lse = np.full((num_tokens, Hq), np.nan)
    seqs = range(num_seqs) if seqs is None else seqs
    for n in seqs:
        L = int(seq_lens[n])
        t0, t1 = int(qsl[n]), int(qsl[n + 1])
        q_len = t1 - t0
        if q_len == 0:
            continue
        K = gather_paged_kv(k_cache, block_table[n], L, block_size)
        V = gather_paged_kv(v_cache, block_table[n], L, block_size)
        pos = L - q_len + np.arange(q_len)  # absolute positions of the queries
        for h in range(Hq):
            g = h // G
            ob, lb = _attend(q[t0:t1, h], K[:, g], V[:, g], scale, pos)
            o[t0:t1, h] = ob
            lse[t0:t1, h] = lb
    return o, lse


def _raw(x):
    """Element values as a numpy array, bit for bit (bf16 tensors through
    their 16-bit patterns, which numpy has no float type for)."""
    if hasattr(x, "detach"):
        import torch  # local import: only needed for torch inputs

        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        return x.numpy()
    return np.asarray(x)


def kv_append(k_new, v_new, k_cache, v_cache, block_table, seq_lens, query_start_loc=None,
              block_size=16):
    """Paged caches after the new tokens' keys and values are written.

    Definition ("Fast attention kernels and operator fusion", section
    "FlashAttention-style attention and paged attention", second paragraph):
    the cache grows by the new tokens; a paged cache holds keys and values in
    fixed-size blocks and a block table maps every logical position to its
    physical block. Sequence n's new rows qsl[n] .. qsl[n+1]-1 of k_new /
    v_new ([num_tokens, Hkv, d]) are its last q_len positions L - q_len ..
    L - 1 (L = seq_lens[n], which counts them); position t is slot
    t % block_size of block block_table[n, t // block_size]. query_start_loc
    None means one new row per sequence (row n).

    Returns (k_cache, v_cache) as new numpy arrays holding the raw element
    values (int16 bit patterns for bf16 tensors); the inputs are untouched.
    """
    kn, vn = _raw(k_new), _raw(v_new)
    kc, vc = _raw(k_cache).copy(), _raw(v_cache).copy()
    table = np.asarray(_raw(block_table), dtype=np.int64)
    lens = np.asarray(_raw(seq_lens), dtype=np.int64)
    num_seqs = lens.shape[0]
    qsl = (np.arange(num_seqs + 1) if query_start_loc is None
           else np.asarray(_raw(query_start_loc), dtype=np.int64))
    for n in range(num_seqs):
        t0, t1 = int(qsl[n]), int(qsl[n + 1])
        q_len = t1 - t0
        for i in range(q_len):
            t = int(lens[n]) - q_len + i  # logical position of new row t0 + i
            blk = int(table[n, t // block_size])
            kc[blk, :, t % block_size, :] = kn[t0 + i]
            vc[blk, :, t % block_size, :] = vn[t0 + i]
    return kc, vc


def add_rmsnorm(x, residual, weight, eps):
    """Residual addition followed by RMS normalisation, row by row, in fp64.

    The pages name "a residual connection added, then an RMSNorm" as a common
    fusion ("Fast attention kernels and operator fusion", section "Operator
    fusion", second paragraph) without writing it out; this is the usual
    definition, over the last axis (``hidden``):

        h = x + residual
        y = h / sqrt(mean(h * h) + eps) * weight

    x, residual: [..., hidden]; weight: [hidden]. Returns (y, h) in float64
    (h is the new residual stream).
    """
    h = _as_f64(x) + _as_f64(residual)
    w = _as_f64(weight)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    y = h / np.sqrt(ms + float(eps)) * w
    return y, h
