// Stand-ins for the device side of libattn.so, so that the host code of the
// C ABI (attn_api.cpp: validation, workspace layout, argument marshalling)
// can be built by a host compiler alone, with sanitizers, and run where no
// GPU exists. The launchers record what they were given instead of launching;
// the HIP device queries report no device, as on a machine without a GPU.
// Test infrastructure only: nothing here is linked into libattn.so.

#include <hip/hip_runtime.h>

#include "attn_internal.h"
#include "host_stubs.h"

StubRecord g_stub;

extern "C" hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
extern "C" hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) {
  return hipErrorNoDevice;
}

namespace attn {

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t) {
  g_stub.prefill = a;
  g_stub.prefill_bf16 += 1;
  return hipSuccess;
}
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t) {
  g_stub.prefill = a;
  g_stub.prefill_f32 += 1;
  return hipSuccess;
}
hipError_t launch_paged_prefill_bf16(const PagedArgs& a, hipStream_t) {
  g_stub.paged = a;
  g_stub.paged_prefill += 1;
  return hipSuccess;
}
hipError_t launch_paged_decode_bf16(const PagedArgs& a, hipStream_t) {
  g_stub.paged = a;
  g_stub.paged_decode += 1;
  return hipSuccess;
}
hipError_t launch_kv_append_bf16(const AppendArgs& a, hipStream_t) {
  g_stub.append = a;
  g_stub.append_calls += 1;
  return hipSuccess;
}
hipError_t launch_add_rmsnorm_bf16(const NormArgs& a, hipStream_t) {
  g_stub.norm = a;
  g_stub.norm_calls += 1;
  return hipSuccess;
}

}  // namespace attn

// The no-allocation entry point with a stand-in for the device array's
// address (the real one lives in a HIP source with the array itself).
static int stub_scratch(void** p) {
  *p = reinterpret_cast<void*>(kStubScratchAddress);
  g_stub.scratch_lookups += 1;
  return ATTN_OK;
}

extern "C" int attn_decode_paged_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
    const int32_t* seq_lens, const int32_t* query_start_loc, void* o, int num_seqs,
    int num_tokens, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
    int max_seq_len, int max_query_len, int64_t num_blocks, float scale, attn_dtype dtype,
    int partition_size, float* lse, void* stream) {
  attn::DecodeRequest r{q, k_cache, v_cache, block_table, seq_lens, query_start_loc, o, lse,
                        num_seqs, num_tokens, Hq, Hkv, d, block_size, max_blocks_per_seq,
                        max_seq_len, max_query_len, num_blocks, scale, dtype, partition_size};
  return attn::decode_paged_run(r, nullptr, 0, stub_scratch, stream);
}
