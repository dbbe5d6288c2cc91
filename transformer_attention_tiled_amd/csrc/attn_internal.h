// Internal interface between the C ABI (attn_api.cpp) and the kernel
// launchers. Arguments reaching a launcher have been validated already.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
};

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
