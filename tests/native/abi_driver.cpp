// Host-only check of the C ABI (include/attn.h) under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with bad requests
// (each must return its status and launch nothing) and with good ones (the
// stand-in launchers of host_stubs.cpp record the arguments the kernels would
// receive, which are checked here). Also checks the paged cache's address
// arithmetic (paged_index.h) at block-table entries where a 32-bit product
// would wrap. Prints "ALL OK" and exits 0 when every check passes.
// Test infrastructure only.

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"
#include "attn_internal.h"
#include "host_stubs.h"
#include "paged_index.h"

static int failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);           \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

// Fake device addresses: never dereferenced (the stand-ins do not launch).
static void* A(uintptr_t x) { return reinterpret_cast<void*>(x); }
static const uintptr_t Q = 0x100000, K = 0x10000000, V = 0x20000000, O = 0x30000000,
                       L = 0x40000000, T = 0x50000000, S = 0x50100000, QSL = 0x50200000,
                       W = 0x60000000;

static void check_prefill() {
  const StubRecord before = g_stub;
  // bad requests: nothing is launched
  CHECK(attn_prefill(nullptr, A(K), A(V), A(O), 1, 2, 2, 16, 64, 0.125f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_NULL);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1, 3, 2, 16, 64, 0.125f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_SHAPE);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1, 2, 2, 16, 96, 0.125f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_UNSUPPORTED);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1, 2, 2, 16, 64, -1.f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_UNSUPPORTED);
  CHECK(attn_prefill(A(Q + 8), A(K), A(V), A(O), 1, 2, 2, 16, 64, 0.125f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_ALIGN);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(Q), 1, 2, 2, 16, 64, 0.125f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_SHAPE);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1 << 20, 1 << 20, 1 << 20, 1 << 20, 128, 0.1f, 1, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_SHAPE);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1, 2, 2, 16, 64, 0.125f, 2, ATTN_BF16, nullptr, nullptr) == ATTN_ERR_SHAPE);
  CHECK(g_stub.prefill_bf16 == before.prefill_bf16 && g_stub.prefill_f32 == before.prefill_f32);
  // good requests reach the launcher with their arguments
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1, 32, 8, 16384, 128, 0.088f, 1, ATTN_BF16,
                     (float*)A(L), nullptr) == ATTN_OK);
  CHECK(g_stub.prefill_bf16 == before.prefill_bf16 + 1);
  CHECK(g_stub.prefill.q == A(Q) && g_stub.prefill.o == A(O) && g_stub.prefill.lse == A(L));
  CHECK(g_stub.prefill.Hq == 32 && g_stub.prefill.Hkv == 8 && g_stub.prefill.T == 16384 &&
        g_stub.prefill.d == 128 && g_stub.prefill.causal == 1);
  CHECK(attn_prefill(A(Q), A(K), A(V), A(O), 1, 2, 2, 128, 64, 0.125f, 0, ATTN_F32, nullptr,
                     nullptr) == ATTN_OK);
  CHECK(g_stub.prefill_f32 == before.prefill_f32 + 1 && g_stub.prefill.causal == 0);
}

static int decode(const void* ws, size_t ws_bytes, int num_seqs, int num_tokens, int Hq, int Hkv,
                  int max_seq_len, int max_query_len, const int32_t* qsl, int P,
                  const void* o = A(O)) {
  return attn_decode_paged(A(Q), A(K), A(V), (const int32_t*)A(T), (const int32_t*)A(S), qsl,
                           (void*)o, num_seqs, num_tokens, Hq, Hkv, 128, 16,
                           (max_seq_len + 15) / 16, max_seq_len, max_query_len, 1 << 10,
                           0.088f, ATTN_BF16, P, nullptr, (void*)ws, ws_bytes, nullptr);
}

static void check_decode() {
  const StubRecord before = g_stub;
  const size_t need = attn_decode_paged_workspace_size(64, 12, 2, 128, 4096, 0);
  CHECK(need > 0);
  CHECK(decode(A(W), need - 1, 64, 64, 12, 2, 4096, 1, nullptr, 0) == ATTN_ERR_WORKSPACE);
  CHECK(decode(nullptr, need, 64, 64, 12, 2, 4096, 1, nullptr, 0) == ATTN_ERR_WORKSPACE);
  CHECK(decode(A(W + 16), need, 64, 64, 12, 2, 4096, 1, nullptr, 0) == ATTN_ERR_ALIGN);
  CHECK(decode(A(W), need, 64, 64, 12, 2, 4096, 2, nullptr, 0) == ATTN_ERR_SHAPE);
  CHECK(decode(A(W), need, 64, 64, 12, 2, 4096, 1, nullptr, 24) == ATTN_ERR_SHAPE);
  CHECK(decode(A(W), need, 64, 64, 12, 2, 4096, 1, nullptr, 8192) == ATTN_ERR_UNSUPPORTED);
  CHECK(decode(A(W), need, 64, 64, 12, 2, 4096, 1, nullptr, 0, A(Q)) == ATTN_ERR_SHAPE);
  CHECK(decode(A(T), need, 64, 64, 12, 2, 4096, 1, nullptr, 0) == ATTN_ERR_SHAPE);  // ws over table
  CHECK(decode(A(W), need, 0x7fffffff, 0x7fffffff, 1 << 30, 1 << 30, 0x7ffffff0, 1, nullptr, 0) ==
        ATTN_ERR_SHAPE);
  CHECK(g_stub.paged_decode == before.paged_decode && g_stub.paged_prefill == before.paged_prefill);
  // good: one query per sequence, automatic partitions
  CHECK(decode(A(W), need, 64, 64, 12, 2, 4096, 1, nullptr, 0) == ATTN_OK);
  CHECK(g_stub.paged_decode == before.paged_decode + 1 && g_stub.paged_prefill == before.paged_prefill);
  const attn::PagedArgs& p = g_stub.paged;
  CHECK(p.partition_size == attn_decode_paged_partition_size(64, 2, 4096));
  CHECK(p.max_parts == (4096 + p.partition_size - 1) / p.partition_size);
  CHECK((void*)p.ws_o == A(W));
  const size_t o_bytes = ((size_t)64 * 12 * p.max_parts * 128 * 4 + 255) / 256 * 256;
  CHECK((uintptr_t)p.ws_lse == W + o_bytes);
  CHECK(o_bytes + ((size_t)64 * 12 * p.max_parts * 4 + 255) / 256 * 256 == need);
  // good: a mixed batch with chunks takes the chunk launcher too, with its
  // work plan after the decode partials (no key pieces: 700 keys fit one)
  const size_t dec2 = attn_decode_paged_workspace_size(8, 8, 2, 128, 700, 32);
  const size_t need2 = attn_paged_workspace_size(8, 500, 8, 2, 128, 700, 300, 32);
  const int64_t cap2 = attn::plan_head_groups(8, 500, 8, 2, false);
  CHECK(cap2 == 2 * (8 + 2));
  CHECK(need2 == dec2 + (16 + 16 * cap2 + 255) / 256 * 256);
  CHECK(decode(A(W), dec2, 8, 500, 8, 2, 700, 300, (const int32_t*)A(QSL), 32) ==
        ATTN_ERR_WORKSPACE);
  CHECK(decode(A(W), need2, 8, 500, 8, 2, 700, 300, (const int32_t*)A(QSL), 32) == ATTN_OK);
  CHECK(g_stub.paged_prefill == before.paged_prefill + 1 &&
        g_stub.paged_decode == before.paged_decode + 2);
  CHECK(g_stub.paged.qsl == A(QSL) && g_stub.paged.max_query_len == 300 &&
        g_stub.paged.partition_size == 32);
  CHECK((uintptr_t)g_stub.paged.chunk_plan == W + dec2 && g_stub.paged.plan_cap == cap2);
  CHECK(g_stub.paged.chunk_pieces == 1 && g_stub.paged.chunk_o == nullptr);
}

static void check_noalloc() {
  const StubRecord before = g_stub;
  auto call = [](int num_seqs, int Hq, int Hkv, int max_seq_len, int P, const void* q) {
    return attn_decode_paged_noalloc(q, A(K), A(V), (const int32_t*)A(T), (const int32_t*)A(S),
                                     nullptr, A(O), num_seqs, num_seqs, Hq, Hkv, 128, 16,
                                     (max_seq_len + 15) / 16, max_seq_len, 1, 1 << 10, 0.088f,
                                     ATTN_BF16, P, nullptr, nullptr);
  };
  CHECK(call(64, 12, 2, 4096, 0, nullptr) == ATTN_ERR_NULL);
  CHECK(call(2000, 32, 8, 32768, 16, A(Q)) == ATTN_ERR_SCRATCH);  // far beyond the array
  CHECK(g_stub.scratch_lookups == before.scratch_lookups);           // refused before the lookup
  CHECK(call(64, 12, 2, 4096, 0, A(Q)) == ATTN_OK);
  CHECK(g_stub.scratch_lookups == before.scratch_lookups + 1);
  CHECK((uintptr_t)g_stub.paged.ws_o == kStubScratchAddress);
}

static void check_append_and_norm() {
  const StubRecord before = g_stub;
  CHECK(attn_kv_append(A(Q), A(Q + 0x8000), A(K), A(V), (const int32_t*)A(T), (const int32_t*)A(S),
                       nullptr, 4, 3, 2, 128, 16, 8, 1, 64, ATTN_BF16, nullptr) == ATTN_ERR_SHAPE);
  CHECK(attn_kv_append(A(Q), A(Q + 0x8000), A(K), A(K + 0x100), (const int32_t*)A(T),
                       (const int32_t*)A(S), nullptr, 4, 4, 2, 128, 16, 8, 1, 64, ATTN_BF16,
                       nullptr) == ATTN_ERR_SHAPE);
  CHECK(attn_kv_append(A(Q), A(Q + 0x8000), A(K), A(V), (const int32_t*)A(T), (const int32_t*)A(S),
                       nullptr, 4, 4, 2, 128, 16, 8, 1, 64, ATTN_BF16, nullptr) == ATTN_OK);
  CHECK(g_stub.append_calls == before.append_calls + 1 && g_stub.append.Hkv == 2 &&
        g_stub.append.num_tokens == 4);
  CHECK(attn_add_rmsnorm(A(Q), A(K), A(V), A(O), A(O), 4, 4096, 1e-6f, ATTN_BF16, nullptr) ==
        ATTN_ERR_SHAPE);
  CHECK(attn_add_rmsnorm(A(Q), A(K), A(V), A(O), A(K), 4, 4096, 1e-6f, ATTN_BF16, nullptr) ==
        ATTN_OK);  // residual updated in place
  CHECK(g_stub.norm_calls == before.norm_calls + 1 && g_stub.norm.residual_out == A(K));
}

static void check_paged_offsets() {
  // (block, head g) of a [num_blocks][Hkv][16][d] cache starts
  // ((entry * Hkv) + g) * 16 * d elements in; computed here in 128-bit
  // arithmetic and compared with the helper the kernels use.
  const int Hkv = 8, d = 128;
  const int64_t block_elems = (int64_t)Hkv * 16 * d;
  const int32_t wrap = (int32_t)(((int64_t)1 << 31) / (block_elems * 2)) + 1;  // bytes past 2^31
  const int32_t entries[] = {0, 1, 1023, wrap - 1, wrap, 270000, 0x7fffffff};
  for (int32_t e : entries) {
    for (int g : {0, 3, Hkv - 1}) {
      const __int128 expect = ((__int128)e * Hkv + g) * 16 * d;
      CHECK((__int128)attn::paged_kv_offset(e, g, Hkv, d) == expect);
      CHECK(attn::paged_kv_offset(e, g, Hkv, d) >= 0);
    }
  }
  // a byte offset formed in a 32-bit int would wrap negative at `wrap` (the
  // checks above can see that slip)
  const int32_t narrow = (int32_t)((uint32_t)wrap * (uint32_t)Hkv * 16u * (uint32_t)d * 2u);
  CHECK(narrow < 0 && (int64_t)narrow != attn::paged_kv_offset(wrap, 0, Hkv, d) * 2);
}

int main() {
  check_prefill();
  check_decode();
  check_noalloc();
  check_append_and_norm();
  check_paged_offsets();
  if (failures == 0) std::printf("ALL OK\n");
  return failures == 0 ? 0 : 1;
}
