// Address arithmetic of the paged KV cache, shared by the kernels and a CPU
// test (no HIP dependency, so the host compiler can check it directly).
//
// A cache is [num_blocks][Hkv][16][d]: block-table entry `entry` (an int32 in
// [0, num_blocks)) names the physical block, and (block, KV head g) starts
// ((int64) entry * Hkv + g) * 16 * d elements into the cache. The entry is
// widened to 64 bits before any product, so offsets past 2^31 elements (a
// cache beyond 4 GiB of bf16) stay exact; an entry is never sign-extended
// from a narrower or unsigned value.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

namespace attn {

ATTN_HD inline int64_t paged_block_index(int32_t entry) { return (int64_t)entry; }

// Element offset of (block named by `entry`, KV head g) in a [num_blocks][Hkv][16][d] cache.
ATTN_HD inline int64_t paged_kv_offset(int32_t entry, int g, int Hkv, int d) {
  return (paged_block_index(entry) * Hkv + g) * 16 * (int64_t)d;
}

}  // namespace attn
