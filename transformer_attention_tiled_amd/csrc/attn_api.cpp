// C ABI of libattn.so (declared in include/attn.h): host-side validation,
// then launch on the caller's stream. Every check runs before the first HIP
// call, so an invalid request launches nothing and touches no device state;
// no request is ever re-routed to another algorithm (the pages name a silent
// fallback to an unfused path as the integration risk that only a profiler
// reveals: "Hugging Face attention profiling guide", aiexpert.news, last
// paragraph).

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

constexpr int64_t kMaxGrid = 0x7fffffff;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int d) { return d == 64 || d == 128; }

bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Product of sizes in int64, or false if it overflows (absurd arguments are
// rejected before any size derived from them is used).
bool mul(std::initializer_list<int64_t> f, int64_t* out) {
  int64_t p = 1;
  for (int64_t x : f)
    if (x < 0 || __builtin_mul_overflow(p, x, &p)) return false;
  *out = p;
  return true;
}

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (a == nullptr || b == nullptr) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// The partition policy estimates the work as num_seqs * Hkv * (max_seq_len /
// 2 + 1) in int64; sizes beyond that range are rejected.
bool policy_in_range(int num_seqs, int Hkv, int max_seq_len) {
  int64_t est;
  return mul({num_seqs, Hkv, (int64_t)max_seq_len / 2 + 1, 2}, &est);
}

// Bytes of the paged-call workspace: the decode partitions' partial outputs
// and lse, then for batches with chunk rows (q_len >= 2) of up to
// kPagedMaxSeqs sequences the chunk rows' work plan and (when their keys may
// span several pieces) the pieces' partial outputs and lse.
struct WsLayout {
  int partition_size = 0;
  int max_parts = 0;
  size_t o_bytes = 0;
  size_t l_bytes = 0;
  int plan_cap = 0;
  size_t plan_bytes = 0;
  int chunk_pieces = 1;
  size_t co_bytes = 0;
  size_t cl_bytes = 0;
  size_t total = 0;
};

bool ws_layout(int num_seqs, int num_tokens, int Hq, int Hkv, int d, int max_seq_len,
               int max_query_len, int partition_size, WsLayout* w) {
  if (num_seqs < 1 || num_tokens < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_seq_len < 1 ||
      max_query_len < 1 || !supported_d(d))
    return false;
  if (partition_size < 0 || partition_size % attn::kBlockSize != 0 ||
      partition_size > attn::kMaxPartition)
    return false;
  if (!policy_in_range(num_seqs, Hkv, max_seq_len)) return false;
  const int P = partition_size > 0 ? partition_size
                                   : attn::decode_partition_size(num_seqs, Hkv, max_seq_len);
  if (P <= 0) return false;
  const int64_t parts = ((int64_t)max_seq_len + P - 1) / P;
  int64_t rows, ob;
  if (!mul({num_seqs, Hq, parts}, &rows) || !mul({rows, d, 4}, &ob) || ob > (INT64_MAX >> 2))
    return false;
  const int64_t o_bytes = (ob + 255) / 256 * 256;
  const int64_t l_bytes = (rows * 4 + 255) / 256 * 256;
  int64_t co_bytes = 0, cl_bytes = 0, plan_bytes = 0, cap = 0;
  int pieces = 1;
  if (max_query_len >= 2 && num_seqs <= attn::kPagedMaxSeqs) {
    const int64_t piece_keys = 64LL * attn::kChunkPieceTiles;
    const int64_t np = ((int64_t)max_seq_len + piece_keys - 1) / piece_keys;
    if (np >= 2) {
      int64_t crows, cob;
      if (!mul({num_tokens, Hq, np}, &crows) || !mul({crows, d, 4}, &cob) ||
          cob > (INT64_MAX >> 3))
        return false;
      co_bytes = (cob + 255) / 256 * 256;
      cl_bytes = (crows * 4 + 255) / 256 * 256;
      pieces = (int)np;
    }
    cap = attn::plan_head_groups(num_seqs, num_tokens, Hq, Hkv, pieces > 1);
    // the planned grid has ceil(cap / 8) * 8 * (Hq / Hkv) workgroups
    if (cap > INT32_MAX / 8 || (cap + 7) / 8 * 8 * (Hq / Hkv) > INT32_MAX) return false;
    plan_bytes = (16 + 16 * cap + 255) / 256 * 256;
  }
  w->partition_size = P;
  w->max_parts = (int)parts;
  w->o_bytes = (size_t)o_bytes;
  w->l_bytes = (size_t)l_bytes;
  w->plan_cap = (int)cap;
  w->plan_bytes = (size_t)plan_bytes;
  w->chunk_pieces = pieces;
  w->co_bytes = (size_t)co_bytes;
  w->cl_bytes = (size_t)cl_bytes;
  w->total = (size_t)(o_bytes + l_bytes + plan_bytes + co_bytes + cl_bytes);
  return true;
}

}  // namespace

namespace attn {

int decode_partition_size(int num_seqs, int Hkv, int max_seq_len) {
  if (num_seqs < 1 || Hkv < 1 || max_seq_len < 1) return 0;
  // One wave per partition, up to six resident per CU, all resident from the
  // start. Aim for about 608 partitions (2.4 per CU of 256): on MI355X fewer,
  // longer partitions beat more, shorter ones until about that point (64
  // sequences, Hkv 2, lengths up to 4096: 37.0-37.5 us at 416..464-token
  // partitions, 40.8 us at 272, 39.6 us at 512). The mean length is
  // estimated as half the maximum; partitions stay between 256 and 4096
  // tokens, in whole 16-token blocks.
  constexpr int64_t kTargetParts = 608;
  const int64_t units = (int64_t)num_seqs * Hkv;
  int64_t P = (units * ((int64_t)max_seq_len / 2 + 1) + kTargetParts - 1) / kTargetParts;
  if (P < 256) P = 256;
  if (P > kMaxPartition) P = kMaxPartition;
  P = (P + 15) / 16 * 16;
  return (int)P;
}

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  // 0: not queried yet; threads that race both store the same value
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cu = cached[dev].load(std::memory_order_relaxed);
  if (cu == 0) {
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0)
      cu = 256;
    cached[dev].store(cu, std::memory_order_relaxed);
  }
  return cu;
}

// Validation, then launch, of one paged call. The workspace is either the
// caller's (workspace, workspace_bytes) or, when `scratch` is given, asked
// of it only after every check has passed, so that a rejected request makes
// no HIP call at all.
int decode_paged_run(const DecodeRequest& r, void* workspace, size_t workspace_bytes,
                     ScratchProvider scratch, void* stream) {
  const void *q = r.q, *k_cache = r.k_cache, *v_cache = r.v_cache;
  const int32_t *block_table = r.block_table, *seq_lens = r.seq_lens,
                *query_start_loc = r.query_start_loc;
  void* o = r.o;
  float* lse = r.lse;
  const int num_seqs = r.num_seqs, num_tokens = r.num_tokens, Hq = r.Hq, Hkv = r.Hkv, d = r.d;
  const int max_blocks_per_seq = r.max_blocks_per_seq, max_seq_len = r.max_seq_len,
            max_query_len = r.max_query_len, partition_size = r.partition_size;
  const int64_t num_blocks = r.num_blocks;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || o == nullptr)
    return ATTN_ERR_NULL;
  if (r.dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (num_seqs < 1 || num_tokens < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!supported_d(d) || r.block_size != kBlockSize || Hq / Hkv > 16 || !good_scale(r.scale))
    return ATTN_ERR_UNSUPPORTED;
  if (max_seq_len < 1 || num_blocks < 1 || max_query_len < 1 || max_query_len > max_seq_len ||
      max_query_len > num_tokens)
    return ATTN_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq < ((int64_t)max_seq_len + kBlockSize - 1) / kBlockSize)
    return ATTN_ERR_SHAPE;
  if (query_start_loc == nullptr && (max_query_len != 1 || num_tokens < num_seqs))
    return ATTN_ERR_SHAPE;
  if (partition_size < 0 || partition_size % kBlockSize != 0) return ATTN_ERR_SHAPE;
  if (partition_size > kMaxPartition) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(query_start_loc, 4) ||
      !aligned(lse, 4) || !aligned(workspace, 256))
    return ATTN_ERR_ALIGN;
  WsLayout w;
  if (!ws_layout(num_seqs, num_tokens, Hq, Hkv, d, max_seq_len, max_query_len, partition_size,
                 &w))
    return ATTN_ERR_SHAPE;
  if (scratch == nullptr && (workspace == nullptr || workspace_bytes < w.total))
    return ATTN_ERR_WORKSPACE;
  if (scratch != nullptr && w.total > kNoAllocScratchBytes) return ATTN_ERR_SCRATCH;
  int64_t qb, cb, tb, lb;
  if (!mul({num_tokens, Hq, d, 2}, &qb) || !mul({num_blocks, Hkv, kBlockSize, d, 2}, &cb) ||
      !mul({num_seqs, max_blocks_per_seq, 4}, &tb) || !mul({num_tokens, Hq, 4}, &lb))
    return ATTN_ERR_SHAPE;
  {
    // what the call writes (o, lse, the workspace) overlaps nothing it reads
    // and no other output (the library's own scratch array is a separate
    // allocation and overlaps nothing of the caller's)
    const void* in[] = {q, k_cache, v_cache, block_table, seq_lens, query_start_loc};
    const int64_t in_bytes[] = {qb, cb, cb, tb, (int64_t)num_seqs * 4,
                                (int64_t)(num_seqs + 1) * 4};
    const void* out[] = {o, lse, scratch != nullptr ? nullptr : workspace};
    const int64_t out_bytes[] = {qb, lb, (int64_t)w.total};
    for (int i = 0; i < 3; ++i) {
      for (int j = 0; j < 6; ++j)
        if (overlap(out[i], out_bytes[i], in[j], in_bytes[j])) return ATTN_ERR_SHAPE;
      for (int j = i + 1; j < 3; ++j)
        if (overlap(out[i], out_bytes[i], out[j], out_bytes[j])) return ATTN_ERR_SHAPE;
    }
  }
  int64_t g1, g2;
  const int64_t n_qt = ((int64_t)max_query_len + 255) / 256;  // 256-row query tiles
  if (!mul({w.max_parts, Hkv, num_seqs}, &g1) || g1 > kMaxGrid ||
      !mul({n_qt, num_seqs, Hq}, &g2) || g2 > kMaxGrid)
    return ATTN_ERR_SHAPE;

  // every check has passed: only now may the scratch provider touch HIP
  if (scratch != nullptr) {
    const int st = scratch(&workspace);
    if (st != ATTN_OK) return st;
  }
  PagedArgs a;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_table = block_table; a.seq_lens = seq_lens; a.qsl = query_start_loc;
  a.o = o; a.lse = lse;
  a.num_seqs = num_seqs; a.num_tokens = num_tokens; a.Hq = Hq; a.Hkv = Hkv; a.d = d;
  a.max_blocks_per_seq = max_blocks_per_seq; a.max_seq_len = max_seq_len;
  a.max_query_len = max_query_len; a.num_blocks = num_blocks; a.scale = r.scale;
  a.partition_size = w.partition_size; a.max_parts = w.max_parts;
  char* ws = static_cast<char*>(workspace);
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_lse = reinterpret_cast<float*>(ws + w.o_bytes);
  char* chunk = ws + w.o_bytes + w.l_bytes;
  a.chunk_plan = w.plan_cap > 0 ? reinterpret_cast<int*>(chunk) : nullptr;
  a.plan_cap = w.plan_cap;
  a.chunk_pieces = w.chunk_pieces;
  a.chunk_o = w.chunk_pieces > 1 ? reinterpret_cast<float*>(chunk + w.plan_bytes) : nullptr;
  a.chunk_lse =
      w.chunk_pieces > 1 ? reinterpret_cast<float*>(chunk + w.plan_bytes + w.co_bytes) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (max_query_len >= 2) {
    if (launch_paged_prefill_bf16(a, s) != hipSuccess) return ATTN_ERR_LAUNCH;
  }
  if (launch_paged_decode_bf16(a, s) != hipSuccess) return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case ATTN_ERR_UNSUPPORTED: return "request outside the supported set (d, dtype, block size, GQA ratio, scale)";
    case ATTN_ERR_ALIGN: return "a pointer is not aligned as required";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case ATTN_ERR_SCRATCH:
      return "the request needs more scratch memory than the fixed no-allocation array holds";
    default: return "unknown status";
  }
}

int attn_prefill(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                 int T, int d, float scale, int causal, attn_dtype dtype, float* lse,
                 void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (!supported_d(d) || !good_scale(scale)) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return ATTN_ERR_ALIGN;
  const int64_t esize = dtype == ATTN_BF16 ? 2 : 4;
  int64_t qbytes, kvbytes, lbytes;
  if (!mul({B, Hq, T, d, esize}, &qbytes) || !mul({B, Hkv, T, d, esize}, &kvbytes) ||
      !mul({B, Hq, T, 4}, &lbytes))
    return ATTN_ERR_SHAPE;
  if (overlap(o, qbytes, q, qbytes) || overlap(o, qbytes, k, kvbytes) ||
      overlap(o, qbytes, v, kvbytes) || overlap(lse, lbytes, q, qbytes) ||
      overlap(lse, lbytes, k, kvbytes) || overlap(lse, lbytes, v, kvbytes) ||
      overlap(lse, lbytes, o, qbytes))
    return ATTN_ERR_SHAPE;
  // query tiles of 64 (fp32) or 256 (bf16) rows, all in one grid dimension;
  // the bound takes the smaller tile
  int64_t grid;
  if (!mul({((int64_t)T + 63) / 64, B, Hq}, &grid) || grid > kMaxGrid) return ATTN_ERR_SHAPE;

  attn::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.T = T; a.d = d;
  a.scale = scale; a.causal = causal;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == ATTN_BF16 ? attn::launch_prefill_bf16(a, s)
                                          : attn::launch_prefill_f32(a, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int attn_decode_paged_partition_size(int num_seqs, int Hkv, int max_seq_len) {
  if (!policy_in_range(num_seqs, Hkv, max_seq_len)) return 0;
  return attn::decode_partition_size(num_seqs, Hkv, max_seq_len);
}

size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int Hkv, int d, int max_seq_len,
                                        int partition_size) {
  WsLayout w;
  if (!ws_layout(num_seqs, num_seqs, Hq, Hkv, d, max_seq_len, 1, partition_size, &w)) return 0;
  return w.total;
}

size_t attn_paged_workspace_size(int num_seqs, int num_tokens, int Hq, int Hkv, int d,
                                 int max_seq_len, int max_query_len, int partition_size) {
  WsLayout w;
  if (!ws_layout(num_seqs, num_tokens, Hq, Hkv, d, max_seq_len, max_query_len, partition_size,
                 &w))
    return 0;
  return w.total;
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* query_start_loc, void* o, int num_seqs, int num_tokens,
                      int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
                      int max_seq_len, int max_query_len, int64_t num_blocks, float scale,
                      attn_dtype dtype, int partition_size, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  attn::DecodeRequest r{q, k_cache, v_cache, block_table, seq_lens, query_start_loc, o, lse,
                        num_seqs, num_tokens, Hq, Hkv, d, block_size, max_blocks_per_seq,
                        max_seq_len, max_query_len, num_blocks, scale, dtype, partition_size};
  return attn::decode_paged_run(r, workspace, workspace_bytes, nullptr, stream);
}

int attn_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens,
                   const int32_t* query_start_loc, int num_seqs, int num_tokens, int Hkv, int d,
                   int block_size, int max_blocks_per_seq, int max_query_len, int64_t num_blocks,
                   attn_dtype dtype, void* stream) {
  if (k_new == nullptr || v_new == nullptr || k_cache == nullptr || v_cache == nullptr ||
      block_table == nullptr || seq_lens == nullptr)
    return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (num_seqs < 1 || num_tokens < 1 || Hkv < 1 || num_blocks < 1 || max_blocks_per_seq < 1 ||
      max_query_len < 1 || max_query_len > num_tokens)
    return ATTN_ERR_SHAPE;
  if (!supported_d(d) || block_size != attn::kBlockSize) return ATTN_ERR_UNSUPPORTED;
  if (query_start_loc == nullptr && (max_query_len != 1 || num_tokens < num_seqs))
    return ATTN_ERR_SHAPE;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(query_start_loc, 4))
    return ATTN_ERR_ALIGN;
  int64_t nbytes, cbytes, tbytes;
  if (!mul({num_tokens, Hkv, d, 2}, &nbytes) ||
      !mul({num_blocks, Hkv, attn::kBlockSize, d, 2}, &cbytes) ||
      !mul({num_seqs, max_blocks_per_seq, 4}, &tbytes))
    return ATTN_ERR_SHAPE;
  const int64_t sbytes = (int64_t)num_seqs * 4, qslbytes = (int64_t)(num_seqs + 1) * 4;
  if (overlap(k_cache, cbytes, v_cache, cbytes) || overlap(k_new, nbytes, k_cache, cbytes) ||
      overlap(k_new, nbytes, v_cache, cbytes) || overlap(v_new, nbytes, k_cache, cbytes) ||
      overlap(v_new, nbytes, v_cache, cbytes))
    return ATTN_ERR_SHAPE;
  // the caches (written) overlap none of the metadata the call reads
  for (const void* c : {(const void*)k_cache, (const void*)v_cache})
    if (overlap(c, cbytes, block_table, tbytes) || overlap(c, cbytes, seq_lens, sbytes) ||
        overlap(c, cbytes, query_start_loc, qslbytes))
      return ATTN_ERR_SHAPE;
  if ((int64_t)attn::append_grid(num_tokens) > kMaxGrid) return ATTN_ERR_SHAPE;

  attn::AppendArgs a;
  a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
  a.block_table = block_table; a.seq_lens = seq_lens; a.qsl = query_start_loc;
  a.num_seqs = num_seqs; a.num_tokens = num_tokens; a.Hkv = Hkv; a.d = d;
  a.max_blocks_per_seq = max_blocks_per_seq; a.max_query_len = max_query_len;
  if (attn::launch_kv_append_bf16(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

int attn_add_rmsnorm(const void* x, const void* residual, const void* weight, void* out,
                     void* residual_out, int rows, int hidden, float eps, attn_dtype dtype,
                     void* stream) {
  if (x == nullptr || residual == nullptr || weight == nullptr || out == nullptr ||
      residual_out == nullptr)
    return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (rows < 1 || hidden < 8 || hidden % 8 != 0) return ATTN_ERR_SHAPE;
  if (hidden > attn::kNormMaxHidden) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || eps < 0.f) return ATTN_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(weight, 16) || !aligned(out, 16) ||
      !aligned(residual_out, 16))
    return ATTN_ERR_ALIGN;
  const int64_t bytes = (int64_t)rows * hidden * 2;
  const int64_t wbytes = (int64_t)hidden * 2;
  // residual_out may be residual itself (in-place update), nothing else may overlap
  if (overlap(out, bytes, x, bytes) || overlap(out, bytes, residual, bytes) ||
      overlap(out, bytes, weight, wbytes) || overlap(out, bytes, residual_out, bytes) ||
      overlap(residual_out, bytes, x, bytes) || overlap(residual_out, bytes, weight, wbytes) ||
      (residual_out != residual && overlap(residual_out, bytes, residual, bytes)))
    return ATTN_ERR_SHAPE;
  if (rows > kMaxGrid) return ATTN_ERR_SHAPE;
  attn::NormArgs a;
  a.x = x; a.residual = residual; a.weight = weight; a.out = out; a.residual_out = residual_out;
  a.rows = rows; a.hidden = hidden; a.eps = eps;
  if (attn::launch_add_rmsnorm_bf16(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

}  // extern "C"
