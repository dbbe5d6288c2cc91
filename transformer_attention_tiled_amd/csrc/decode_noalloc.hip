// attn_decode_paged_noalloc: the paged call with its split-KV scratch in a
// fixed device array of the library, for callers that cannot allocate (see
// include/attn.h). Same validation and kernels as attn_decode_paged.

#include <hip/hip_runtime.h>

#include <atomic>

#include "attn_internal.h"

namespace attn {

static_assert(kNoAllocScratchBytes == ATTN_DECODE_NOALLOC_SCRATCH_BYTES,
              "the header's limit and the array agree");

// Zero-initialised when the library's code object is loaded on a device;
// each device holds its own copy. Host code never passes this name to a
// kernel or a copy: it is a host-side stand-in, not a device address.
// `scratch_ptr` below holds the device address, per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current (hipGetSymbolAddress; no allocation).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_ERR_LAUNCH;
    // concurrent first calls on one device look up the same address
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

extern "C" int attn_decode_paged_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    const int32_t* seq_lens, const int32_t* query_start_loc, void* o, int num_seqs,
    int num_tokens, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
    int max_seq_len, int max_query_len, int64_t num_blocks, float scale, attn_dtype dtype,
    int partition_size, float* lse, void* stream) {
  attn::DecodeRequest r{q, k_cache, v_cache, block_table, seq_lens, query_start_loc, o, lse,
                        num_seqs, num_tokens, Hq, Hkv, d, block_size, max_blocks_per_seq,
                        max_seq_len, max_query_len, num_blocks, scale, dtype, partition_size};
  return attn::decode_paged_run(r, nullptr, 0, attn::current_scratch, stream);
}
