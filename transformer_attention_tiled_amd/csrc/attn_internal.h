// Internal interface between the C ABI (attn_api.cpp) and the kernel
// launchers. Arguments reaching a launcher have been validated already.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/attn.h"
#include "paged_index.h"

namespace attn {

// Contiguous prefill: q,o [B][Hq][T][d], k,v [B][Hkv][T][d].
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // [B][Hq][T] or nullptr
  int B, Hq, Hkv, T, d;
  float scale;
  int causal;
};

// Paged batch: q,o [num_tokens][Hq][d]; caches [num_blocks][Hkv][16][d].
struct PagedArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;  // [num_seqs][max_blocks_per_seq]
  const int32_t* seq_lens;     // [num_seqs]
  const int32_t* qsl;          // [num_seqs + 1] or nullptr (one query per sequence)
  void* o;
  float* lse;  // [num_tokens][Hq] or nullptr
  int num_seqs, num_tokens, Hq, Hkv, d;
  int max_blocks_per_seq, max_seq_len, max_query_len;
  int64_t num_blocks;
  float scale;
  int partition_size;  // resolved (> 0, multiple of 16)
  int max_parts;       // ceil(max_seq_len / partition_size)
  float* ws_o;         // split-KV partial outputs [num_seqs][Hq][max_parts][d]
  float* ws_lse;       // split-KV partial log2-sum-exp [num_seqs][Hq][max_parts]
  // chunk rows (q_len >= 2) split along the keys into pieces of at least
  // kChunkPieceTiles key tiles: at most chunk_pieces per query tile (1: not
  // split; then chunk_o / chunk_lse are unused)
  int chunk_pieces;
  float* chunk_o;      // piece partial outputs [num_tokens][Hq][chunk_pieces][d]
  float* chunk_lse;    // piece partial log2-sum-exp [num_tokens][Hq][chunk_pieces]
  // the chunk rows' work plan (batches of up to kPagedMaxSeqs sequences, else
  // nullptr): [0] head groups listed, [1] key tiles per piece, from int 4 on
  // one int4 {sequence, piece, query tile, KV head} per head group
  int* chunk_plan;
  int plan_cap;        // head groups the plan has room for
};

// Chunk rows are split along the keys in pieces of at least this many 64-key
// tiles (4096 keys), by the planned chunk kernel (batches of up to
// kPagedMaxSeqs sequences); the workspace holds ceil(max_seq_len / 4096)
// pieces per row.
constexpr int kChunkPieceTiles = 64;
constexpr int kPagedMaxSeqs = 2048;
// The piece length is the chunk work's share per compute unit of a chip of
// this many; the plan's length bound uses it.
constexpr int kPlanWGs = 256;

// Head groups (G = Hq / Hkv units sharing keys) the plan of a paged call can
// list: Hkv per (chunk query tile, piece). A chunk sequence has at least 2 of
// the num_tokens query rows and at most ceil(q_len / 256) <= q_len / 256 + 1
// query tiles; the pieces add at most kPlanWGs / Hq per KV head (the piece
// length is at least the chunk key tiles times Hq over kPlanWGs, and an item
// of t tiles has at most t / length + 1 pieces).
inline int64_t plan_head_groups(int64_t num_seqs, int64_t num_tokens, int Hq, int Hkv,
                                bool split) {
  const int64_t tiles = std::min(num_seqs, num_tokens / 2) + (num_tokens + 255) / 256;
  const int64_t extra = split ? (kPlanWGs + Hq - 1) / Hq : 0;
  return (int64_t)Hkv * (tiles + extra);
}

// Append to a paged cache: k_new,v_new [num_tokens][Hkv][d] written into
// caches [num_blocks][Hkv][16][d] at the positions the block table gives.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;  // [num_seqs][max_blocks_per_seq]
  const int32_t* seq_lens;     // [num_seqs]
  const int32_t* qsl;          // [num_seqs + 1] or nullptr (one new token per sequence)
  int num_seqs, num_tokens, Hkv, d;
  int max_blocks_per_seq, max_query_len;
};

// Residual add + RMSNorm over rows of `hidden` elements.
struct NormArgs {
  const void* x;         // [rows][hidden]
  const void* residual;  // [rows][hidden]
  const void* weight;    // [hidden]
  void* out;             // [rows][hidden]: RMSNorm(x + residual) * weight
  void* residual_out;    // [rows][hidden]: x + residual (may be `residual` itself)
  int rows, hidden;
  float eps;
};
constexpr int kNormMaxHidden = 8 * 256 * 8;  // 8 chunks of 16 bytes per thread

constexpr int kBlockSize = 16;
constexpr int kMaxPartition = 4096;  // tokens per split-KV partition, at most

// Compute units of the current device (queried once per device and cached).
int device_cu_count();

// Host-side policy shared by the workspace query and the launch.
int decode_partition_size(int num_seqs, int Hkv, int max_seq_len);

// One attn_decode_paged request as the caller made it (before validation).
struct DecodeRequest {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  void* o;
  float* lse;
  int num_seqs, num_tokens, Hq, Hkv, d, block_size, max_blocks_per_seq, max_seq_len,
      max_query_len;
  int64_t num_blocks;
  float scale;
  attn_dtype dtype;
  int partition_size;
};

// Bytes of the fixed device array behind attn_decode_paged_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// Supplies the device address of the library's scratch array on the current
// device (ATTN_OK) or a failure status. Called only after validation passed.
typedef int (*ScratchProvider)(void** ptr);

// Validate a paged request, then launch it with the caller's workspace, or
// with the scratch array when `scratch` is not null.
int decode_paged_run(const DecodeRequest& r, void* workspace, size_t workspace_bytes,
                     ScratchProvider scratch, void* stream);

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_paged_prefill_bf16(const PagedArgs& a, hipStream_t s);  // q_len >= 2 sequences
hipError_t launch_paged_decode_bf16(const PagedArgs& a, hipStream_t s);   // q_len == 1 sequences
constexpr int kAppendRows = 8;  // new rows per workgroup of the append kernel
inline int append_grid(int num_tokens) { return (num_tokens + kAppendRows - 1) / kAppendRows; }
hipError_t launch_kv_append_bf16(const AppendArgs& a, hipStream_t s);
hipError_t launch_add_rmsnorm_bf16(const NormArgs& a, hipStream_t s);

}  // namespace attn
