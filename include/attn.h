/*
 * attn.h — C ABI of libattn.so: fused scaled-dot-product attention on AMD
 * Instinct MI355X (gfx950).
 *
 * Two operations, as the source pages state the problem, the cache append
 * that feeds the second (attn_kv_append) and the residual-add + RMSNorm
 * fusion the same page names (attn_add_rmsnorm), both below:
 *
 *  - attn_prefill: causal (or full) attention over contiguous Q, K, V,
 *    computed block by block so that the T x T score matrix never reaches
 *    HBM: per block of keys the kernel forms part of the scores, updates the
 *    running softmax statistics and accumulates the output in on-chip
 *    memory. ("Fast attention kernels and operator fusion", the-ai.news,
 *    section "FlashAttention-style attention and paged attention", first
 *    paragraph.) The result is the naive definition — Q K^T, scaling, causal
 *    mask, row softmax, product with V ("Hugging Face attention profiling
 *    guide", aiexpert.news, second paragraph) — up to rounding order.
 *
 *  - attn_decode_paged: attention of the batch's new query tokens against a
 *    paged KV cache of fixed 16-token blocks, every logical position being
 *    translated through a block table (same page and section, second and
 *    third paragraphs: fixed-size blocks, a table from logical positions to
 *    physical blocks, block_size = 16).
 *
 * Conventions shared by all entry points
 *  - Every pointer is caller-owned DEVICE memory (except where noted). The
 *    library never allocates, frees or keeps a pointer after returning.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without waiting. There is no host synchronisation
 *    and no device-to-host read, and launch shapes depend on host arguments
 *    only, so the calls may be captured in a HIP graph (the pages' reason for
 *    graph replay: fixed shapes and fixed addresses, "Fast attention kernels
 *    and operator fusion", section "Fusion and CUDA Graphs with
 *    torch.compile").
 *  - Arguments are validated on the host BEFORE any HIP call. An invalid or
 *    unsupported request returns a negative status and launches nothing: the
 *    library never falls back to another algorithm (the pages warn that a
 *    silent fallback to an unfused path is the hardest risk to see,
 *    "Hugging Face attention profiling guide", last paragraph).
 *  - Sizes whose byte counts or grids do not fit in int64 (or in the launch
 *    limits) return ATTN_ERR_SHAPE.
 *  - A launch failure reported by the HIP runtime returns ATTN_ERR_LAUNCH.
 *  - bf16 is IEEE bfloat16 (the upper 16 bits of an fp32). Products are
 *    accumulated in fp32. The bf16 paths fold the softmax scale into the
 *    query: each element of q is multiplied by scale * log2(e) (fp32) and
 *    rounded to bf16 once (round-to-nearest-even: a relative error of at
 *    most 2^-8 per element of q), so a score q.k moves by at most
 *    2^-8 * scale * sum_i |q_i k_i| and lse by at most the largest such move
 *    over the keys the row sees. The softmax weights are rounded to bf16
 *    (round-to-nearest-even) before the product with V, their row sum is
 *    taken in fp32 from the unrounded weights, and outputs are rounded to
 *    the output type at the end. The fp32 prefill path rounds nothing.
 *  - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *  - `scale` multiplies the scores before the softmax; it must be finite and
 *    > 0 (use 1/sqrt(d) for the usual scaling).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  ATTN_ERR_UNSUPPORTED = -3, /* valid request outside the supported set */
  ATTN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  ATTN_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  ATTN_ERR_LAUNCH = -6,      /* the HIP runtime rejected a launch */
  ATTN_ERR_SCRATCH = -7      /* the no-allocation variant's fixed scratch is too small */
};

/*
 * attn_prefill — o = softmax(scale * q k^T [+ causal mask]) v, per (batch,
 * query head).
 *
 * Layout (row-major, contiguous, element type `dtype`):
 *   q, o : [B][Hq][T][d]
 *   k, v : [B][Hkv][T][d]
 *   lse  : [B][Hq][T] fp32, optional (NULL = not written):
 *          lse = log(sum_j exp(scale * q.k_j)) over the keys the row sees.
 * causal = 1: query i sees keys 0..i; causal = 0: all T keys.
 * Supported: d in {64, 128}; dtype ATTN_BF16 (MFMA path) or ATTN_F32;
 * Hq % Hkv == 0; B, Hq, Hkv, T >= 1; q, k, v, o 16-byte aligned; lse 4-byte
 * aligned. q/k/v must not overlap o or lse.
 * Returns ATTN_OK or a negative status; on error nothing is launched.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o,
                 int B, int Hq, int Hkv, int T, int d, float scale, int causal,
                 attn_dtype dtype, float* lse, void* stream);

/*
 * attn_decode_paged_partition_size — the KV partition length (tokens) that
 * attn_decode_paged uses for these arguments when it is passed
 * partition_size = 0. A pure function of its arguments. Returns 0 if the
 * arguments are out of range.
 */
int attn_decode_paged_partition_size(int num_seqs, int Hkv, int max_seq_len);

/*
 * attn_decode_paged_workspace_size — bytes of device workspace that
 * attn_decode_paged needs for the same arguments (partition_size as passed
 * to attn_decode_paged, 0 = automatic). Returns 0 if the arguments are out
 * of range. The workspace holds the fp32 split-KV partial results; its
 * contents need no initialisation and are garbage after the call. Calls that
 * run at the same time must not share a workspace.
 */
size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int Hkv, int d,
                                        int max_seq_len, int partition_size);

/*
 * attn_paged_workspace_size — bytes of device workspace that
 * attn_decode_paged (and attn_decode_paged_noalloc, from its fixed array)
 * needs for a batch that may hold sequences with several query tokens:
 * num_tokens and max_query_len as passed to attn_decode_paged. Besides the
 * split-KV partials it holds, for batches of up to 2048 sequences with
 * max_query_len >= 2, the work plan of the chunk rows (a few bytes per chunk
 * query tile and KV head) and, when max_seq_len > 4096, the partial results
 * of their key pieces: where the chunk rows alone would leave compute units
 * idle, a chunk row's keys are split into pieces of at least 4096 keys,
 * processed in parallel and merged by log-sum-exp, so that one long row does
 * not hold a compute unit alone. With max_query_len == 1 it equals
 * attn_decode_paged_workspace_size. Returns 0 if the arguments are out of
 * range. Same contents rules as above.
 */
size_t attn_paged_workspace_size(int num_seqs, int num_tokens, int Hq, int Hkv, int d,
                                 int max_seq_len, int max_query_len, int partition_size);

/*
 * attn_decode_paged — attention of the batch's query tokens against a paged
 * KV cache.
 *
 * Layout:
 *   q, o         : [num_tokens][Hq][d] bf16, token-major
 *   k_cache,
 *   v_cache      : [num_blocks][Hkv][block_size][d] bf16 (one (block, head)
 *                  is block_size * d contiguous elements)
 *   block_table  : int32 [num_seqs][max_blocks_per_seq]; entry b of row n is
 *                  the physical block holding logical positions
 *                  16b .. 16b+15 of sequence n
 *   seq_lens     : int32 [num_seqs]; L_n = number of cached positions of
 *                  sequence n, including the K/V of its current query tokens
 *   query_start_loc : int32 [num_seqs + 1] or NULL. Sequence n owns query
 *                  rows qsl[n] .. qsl[n+1]-1 of q/o (q_len_n of them), which
 *                  are its LAST q_len_n positions L_n - q_len_n .. L_n - 1;
 *                  the query at position t sees keys 0..t. NULL means one
 *                  query per sequence (row n) that sees all L_n keys.
 *   lse          : [num_tokens][Hq] fp32, optional (NULL = not written).
 *   workspace    : device memory of at least
 *                  attn_paged_workspace_size(num_seqs, num_tokens, Hq, Hkv,
 *                  d, max_seq_len, max_query_len, partition_size) bytes
 *                  (which is attn_decode_paged_workspace_size(...) when
 *                  max_query_len == 1), 256-byte aligned.
 * Host-side bounds (the caller knows them; nothing is read back):
 *   max_seq_len   >= every L_n;  max_query_len >= every q_len_n (1 when
 *   query_start_loc is NULL);  max_blocks_per_seq >= ceil(max_seq_len/16).
 * Sequences with q_len_n == 1 take the split-KV decode path (partitions of
 * partition_size tokens, 0 = automatic, else a positive multiple of 16, then
 * a log-sum-exp merge); sequences with q_len_n >= 2 take the tiled prefill
 * path reading K/V tiles through the block table; when the batch has at
 * most 2048 sequences, a 256-row query tile's keys may be split into pieces
 * of at least 4096 keys merged by log-sum-exp (see attn_paged_workspace_size).
 * partition_size is at most 4096 (larger: ATTN_ERR_UNSUPPORTED).
 * Preconditions not checked on the device: table entries for logical blocks
 * < ceil(L_n/16) lie in [0, num_blocks); 0 <= L_n <= max_seq_len;
 * q_len_n <= L_n; query_start_loc is non-decreasing with qsl[num_seqs] <=
 * num_tokens. Table entries past ceil(L_n/16) are never read and may hold
 * anything (e.g. -1); cache slots at positions >= L_n are never read. A row
 * that sees no key (L_n = 0) gets o = 0 and lse = -inf.
 * Supported: d in {64, 128}; dtype ATTN_BF16; block_size == 16;
 * Hq % Hkv == 0 and Hq / Hkv <= 16.
 * What the call writes (o, lse, the first
 * attn_paged_workspace_size(...) bytes of workspace) must not overlap
 * any input (q, the caches, block_table, seq_lens, query_start_loc) or
 * another output: ATTN_ERR_SHAPE.
 * Returns ATTN_OK or a negative status; on error nothing is launched.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* query_start_loc, void* o,
                      int num_seqs, int num_tokens, int Hq, int Hkv, int d,
                      int block_size, int max_blocks_per_seq, int max_seq_len,
                      int max_query_len, int64_t num_blocks, float scale,
                      attn_dtype dtype, int partition_size, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc — attn_decode_paged for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. It allocates nothing and takes no
 * workspace argument: the split-KV partials live in a fixed array inside the
 * library, ATTN_DECODE_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the
 * library's first use on that GPU until the process ends. Arguments,
 * layouts, results and errors are those of attn_decode_paged (same kernels,
 * bitwise the same output for the same partition size), plus:
 *   - ATTN_ERR_SCRATCH when the request needs more than the fixed array
 *     (attn_paged_workspace_size(...) > ATTN_DECODE_NOALLOC_SCRATCH_BYTES);
 *     nothing is launched then.
 *   - ATTN_ERR_LAUNCH if the array's device address cannot be obtained.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and must not be made.
 * Calls on the same stream are ordered and safe.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* query_start_loc, void* o,
                              int num_seqs, int num_tokens, int Hq, int Hkv, int d,
                              int block_size, int max_blocks_per_seq, int max_seq_len,
                              int max_query_len, int64_t num_blocks, float scale,
                              attn_dtype dtype, int partition_size, float* lse, void* stream);

/*
 * attn_kv_append — write the new tokens' keys and values into a paged KV
 * cache, the step before attn_decode_paged reads them. A paged cache keeps
 * keys and values in fixed-size blocks and translates each logical position
 * through a block table; the cache grows by the new tokens of every step
 * ("Fast attention kernels and operator fusion", the-ai.news, section
 * "FlashAttention-style attention and paged attention", second paragraph).
 *
 * Layout:
 *   k_new, v_new : [num_tokens][Hkv][d] bf16, token-major (the rows of the
 *                  new tokens, in the order of query_start_loc)
 *   k_cache,
 *   v_cache      : [num_blocks][Hkv][block_size][d] bf16, written in place
 *   block_table, seq_lens, query_start_loc : exactly as in
 *                  attn_decode_paged: sequence n owns rows qsl[n] ..
 *                  qsl[n+1]-1 of k_new/v_new (q_len_n rows, NULL = one row
 *                  per sequence, row n), which are its last positions
 *                  L_n - q_len_n .. L_n - 1 (seq_lens counts them already).
 * Effect: for every new row i of sequence n, at position t:
 *   k_cache[block_table[n][t/16]][h][t%16][:] = k_new[i][h][:] for all h,
 *   and the same for v. Nothing else in the caches is written.
 * Preconditions not checked on the device: q_len_n <= L_n <= 16 *
 * max_blocks_per_seq; the table entries of the written positions lie in
 * [0, num_blocks); no two new rows
 * map to the same cache slot (otherwise which one lands is unspecified).
 * Supported: d in {64, 128}; dtype ATTN_BF16; block_size == 16. Pointers of
 * k_new, v_new and the caches 16-byte aligned; the new rows must not overlap
 * the caches, the two caches must not overlap each other, block_table,
 * seq_lens or query_start_loc (ATTN_ERR_SHAPE). max_query_len >= every
 * q_len_n (1 when query_start_loc is NULL).
 * Returns ATTN_OK or a negative status; on error nothing is launched.
 */
int attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens,
                   const int32_t* query_start_loc, int num_seqs, int num_tokens, int Hkv, int d,
                   int block_size, int max_blocks_per_seq, int max_query_len, int64_t num_blocks,
                   attn_dtype dtype, void* stream);

/*
 * attn_add_rmsnorm — residual addition fused with RMS normalisation, the
 * fusion the pages name next to attention: unfused, the sum is written to
 * HBM and read back by the norm ("Fast attention kernels and operator
 * fusion", the-ai.news, section "Operator fusion", second paragraph). Per
 * row of `hidden` elements:
 *   residual_out = x + residual
 *   out          = (x + residual) / sqrt(mean((x + residual)^2) + eps) * weight
 * computed in fp32 from the bf16 inputs; both results rounded to bf16 (RNE).
 *
 * Layout (row-major, bf16): x, residual, out, residual_out: [rows][hidden];
 * weight: [hidden]. residual_out may be residual itself (the residual stream
 * updated in place); no other pair may overlap.
 * Supported: dtype ATTN_BF16; hidden a multiple of 8 and at most 16384;
 * eps finite and >= 0; all pointers 16-byte aligned.
 * Returns ATTN_OK or a negative status; on error nothing is launched.
 */
int attn_add_rmsnorm(const void* x, const void* residual, const void* weight, void* out,
                     void* residual_out, int rows, int hidden, float eps, attn_dtype dtype,
                     void* stream);

/* attn_status_string — static, human-readable text for a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
