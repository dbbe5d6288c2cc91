// Single-token decode against a paged KV cache, bf16 in / fp32 accumulate.
//
// The cache stores keys and values in fixed 16-token blocks and a block table
// maps each sequence's logical positions to physical blocks; the kernel
// translates every position through that table ("Fast attention kernels and
// operator fusion", the-ai.news, section "FlashAttention-style attention and
// paged attention", second and third paragraphs: fixed-size blocks, the
// block table, block_size = 16). Decode reads every cached K/V element once
// for few flops, so it is bound by HBM bandwidth (the decode argument of
// "torch.compile and CUDA graphs", llmdeepdive.com, section "Concept").
//
// Work decomposition (split-KV). One wave = one workgroup = one work item
// (partition p of P tokens, KV head g, sequence n); all G = Hq/Hkv query
// heads of the group share each K/V block read. The grid is sized for the
// host's bound max_parts per sequence, but workgroups are mapped onto the
// batch's real partitions only (a prefix sum over the per-sequence counts,
// read on the device), so the real work is dispatched first and the spare
// workgroups at the end of the grid exit at once.
//
// Memory path. The bound is HBM latency x bytes in flight, so the wave keeps
// several blocks in flight without spending registers on them: each 16-token
// block (K 16 x d, V 16 x d) is copied straight from HBM into an LDS ring
// slot with global_load_lds_dwordx4 (lane L of a copy instruction writes the
// 16 bytes at M0 + 16 L; every instruction moves one contiguous KiB, fully
// coalesced). The ring holds kRing slots, kRing-1 blocks ahead of the one
// being consumed. The copies are issued from inline assembly and waited for
// with explicit vmcnt counts (the compiler would otherwise assume any
// outstanding LDS copy may alias every LDS read and wait for all of them).
// The K tile is stored with its 16-byte chunks XOR-swizzled by row, so the
// MFMA operand reads (16 rows, same chunk) hit distinct LDS banks.
//
// Per block, MFMA for both products (the contraction is tiny but MFMA keeps
// the VALU free for the softmax):
//   S = K Q^T   v_mfma_f32_16x16x32_bf16: A = K block (token = l%16, 8
//               consecutive d), B = Q^T (head = l%16), C = S[token][head]
//               with lane l holding tokens 4*(l/16)+r, head l%16.
//   O += P V    v_mfma_f32_16x16x16bf16_1k: A = P[head][token], which is the
//               S accumulator of the lane as is; B = V[token][d] for tokens
//               4*(l/16)+e: lane l reads rows 4*(l/16)..+3 at d-chunk
//               DPL*(l%16)..+DPL-1 and MFMA number m takes element m of each
//               row, so its output column j is d = DPL*j + m.
// Positions >= L are never read from HBM (rows past the end of the last
// block re-read the last valid row) and their scores are selected to -inf.
//
// A sequence with a single partition writes its output directly. Otherwise
// the wave writes its normalised fp32 partial o_p and log2-sum-exp, and a
// second kernel, one workgroup per (sequence, KV head), merges them:
//   lse = log2 sum_p 2^(lse_p),  o = sum_p 2^(lse_p - lse) o_p.
// The merge identity is exact; only rounding differs from the unsplit sum.
// (Merging in the last finishing workgroup would need device-scope fences,
// which write back and invalidate a whole L2 per workgroup; the kernel
// boundary orders the partials for free.)

#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegInf = -__builtin_inff();
// LDS slots per wave (kRing-1 blocks in flight ahead). Three slots (24 KiB
// per wave at d = 128) let six single-wave workgroups reside on a CU at once;
// four slots (32 KiB) fit fewer than five in practice, and a batch's work
// items then no longer start together.
constexpr int kRing = 3;

template <int D>
struct Tile {
  static constexpr int ROW = D * 2;            // bytes per token row
  static constexpr int NCH = D / 8;            // 16-byte chunks per row
  static constexpr int KV = 16 * ROW;          // bytes of the K (or V) part of a block
  static constexpr int SLOT = 2 * KV;          // K then V
  static constexpr int COPIES = KV / 1024;     // 1 KiB copy instructions per part
  static constexpr int DPL = D / 16;           // V elements per lane per row
};

// One 16-byte-per-lane HBM -> LDS copy: lane L's bytes at `src` go to LDS
// address lds + 16 L.
// M0 holds the LDS address and is set inside the same asm statement; it is
// declared clobbered, and the compiler keeps no value of its own in M0 across
// these statements (on gfx950 LDS instructions do not read M0), so its
// warning that a reserved register is clobbered is expected here.
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(src) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Issue the copies of one block into ring slot `slot` (LDS address). Rows at
// or past `valid` re-read row valid-1, so nothing past the sequence is read.
template <int D>
__device__ __forceinline__ void issue_block(const uint16_t* kblk, const uint16_t* vblk,
                                           int valid, uint32_t slot, int lane) {
  using C = Tile<D>;
  const char* kb = (const char*)kblk;
  const char* vb = (const char*)vblk;
#pragma unroll
  for (int s = 0; s < C::COPIES; ++s) {
    const int off = s * 1024 + 16 * lane;    // LDS byte offset written by this lane
    const int t = off / C::ROW;              // token row
    const int pc = (off % C::ROW) / 16;      // chunk position in the LDS row
    const int ts = min(t, valid - 1);
    const int kc = pc ^ (t % C::NCH);        // K: logical chunk stored at pc
    copy_to_lds(kb + ts * C::ROW + kc * 16, slot + s * 1024);
    copy_to_lds(vb + ts * C::ROW + pc * 16, slot + C::KV + s * 1024);
  }
}

__device__ __forceinline__ uint32_t elem16(const u32x4& x, int m) {
  const uint32_t w = x[m >> 1];
  return (m & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}


// Partitions of sequence n handled by the decode path: ceil(L/P) for a
// single-query sequence (one for L <= 0, which writes o = 0), none for a
// sequence with another query count (handled by the prefill path).
__device__ __forceinline__ int decode_parts(const PagedArgs& a, int n) {
  if (a.qsl != nullptr && a.qsl[n + 1] - a.qsl[n] != 1) return 0;
  const int L = a.seq_lens[n];
  return L <= 0 ? 1 : (L + a.partition_size - 1) / a.partition_size;
}

constexpr int kScanChunks = 16;  // batches of up to 1024 sequences use the packed item list

// Work item k (per KV head) -> (sequence n, partition p), where the items of
// the whole batch are listed sequence by sequence, every partition once. All
// 64 lanes compute the same answer with a wave-wide prefix sum over the
// per-sequence partition counts (loaded up front, one round trip). Returns
// false for k past the last item.
__device__ __forceinline__ bool packed_item(const PagedArgs& a, int k, int lane, int& n_out,
                                            int& p_out) {
  int cnt[kScanChunks];
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c) {
    const int n = 64 * c + lane;
    cnt[c] = n < a.num_seqs ? decode_parts(a, n) : 0;
  }
  int base = 0;
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c) {
    if (64 * c >= a.num_seqs) break;
    int incl = cnt[c];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d);
      incl += lane >= d ? up : 0;
    }
    const int excl = incl - cnt[c];
    const bool hit = cnt[c] > 0 && base + excl <= k && k < base + incl;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
    if (m) {
      const int hl = __builtin_ctzll(m);
      n_out = 64 * c + hl;
      p_out = k - base - __shfl(excl, hl);
      return true;
    }
    base += __shfl(incl, 63);
  }
  return false;
}

template <int D>
__global__ __launch_bounds__(64) void decode_kernel(PagedArgs a, float c) {
  using C = Tile<D>;
  constexpr int DPL = C::DPL;
  constexpr int NI = 2 * C::COPIES;  // copy instructions per block
  __shared__ __attribute__((aligned(1024))) char ring[kRing * C::SLOT];

  // Item order: with up to 1024 sequences, the batch's real partitions are
  // packed sequence by sequence (no idle workgroups ahead of real ones);
  // larger batches use the partition-major order bid = (p*num_seqs + n)*Hkv + g,
  // whose workgroups past a sequence's end exit at once.
  const int bid = blockIdx.x;
  const int g = bid % a.Hkv;
  const int lane = threadIdx.x;
  int n, p;
  if (a.num_seqs <= 64 * kScanChunks) {
    if (!packed_item(a, bid / a.Hkv, lane, n, p)) return;
  } else {
    n = (bid / a.Hkv) % a.num_seqs;
    p = bid / (a.Hkv * a.num_seqs);
    if (decode_parts(a, n) <= p) return;
  }
  const int G = a.Hq / a.Hkv;
  const int t0 = a.qsl != nullptr ? a.qsl[n] : n;
  const int L = a.seq_lens[n];
  const int P = a.partition_size;
  if (L <= 0) {
    // no key at all: o = 0, lse = -inf
    for (int i = lane; i < G * D; i += 64) {
      const int hh = i / D, d = i % D;
      ((uint16_t*)a.o)[((int64_t)t0 * a.Hq + g * G + hh) * D + d] = 0;
      if (a.lse != nullptr && d == 0) a.lse[(int64_t)t0 * a.Hq + g * G + hh] = kNegInf;
    }
    return;
  }
  const int np = (L + P - 1) / P;
  const int start = p * P;
  const int end = min(L, start + P);
  const int nb = (end - start + 15) >> 4;  // blocks of this partition (<= 256)
  const int first = start >> 4;
  const int head = lane & 15;  // query head (column) owned in S
  const int grp = lane >> 4;

  // Q^T fragments (B operand of S = K Q^T); lanes past G read head G-1
  // (their columns are ignored)
  bf16x8 qf[D / 32];
  {
    const uint16_t* qrow =
        (const uint16_t*)a.q + ((int64_t)t0 * a.Hq + g * G + min(head, G - 1)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + (D / 4) * grp + 8 * s));
  }
  // physical blocks of the partition: lane i holds blocks i, i+64, ...
  const int32_t* table = a.block_table + (int64_t)n * a.max_blocks_per_seq + first;
  int tbl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tbl[j] = (64 * j + lane < nb) ? table[64 * j + lane] : 0;
  // Q and the table entries have landed before any copy is issued: from here
  // on, the only outstanding loads are the ring copies, counted exactly.
  __builtin_amdgcn_s_waitcnt(0);

  const uint32_t ring0 = (uint32_t)(uintptr_t)ring;

  // element offset of block b's (block, head g) rows in the caches
  auto offset_of = [&](int b) -> int64_t {
    const int j = b >> 6;
    const int v = j == 0 ? tbl[0] : j == 1 ? tbl[1] : j == 2 ? tbl[2] : tbl[3];
    return paged_kv_offset(__builtin_amdgcn_readlane(v, b & 63), g, a.Hkv, D);
  };
  auto issue = [&](int b) {
    const int64_t off = offset_of(b);
    issue_block<D>((const uint16_t*)a.k_cache + off, (const uint16_t*)a.v_cache + off,
                   min(16, end - (start + 16 * b)), ring0 + (b % kRing) * C::SLOT, lane);
  };

  f32x4 acc[DPL];
#pragma unroll
  for (int m = 0; m < DPL; ++m) acc[m] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;

#pragma unroll
  for (int u = 0; u < kRing - 1; ++u)
    if (u < nb) issue(u);
  // fold the softmax scale in log2 units (c = scale * log2 e) into q while
  // the first blocks are in flight: the score MFMA then yields c * s (each
  // q * c rounded to bf16, as in prefill)
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)((float)qf[s][e] * c);

  for (int b = 0; b < nb; ++b) {
    if (b + kRing - 1 < nb) issue(b + kRing - 1);
    // wait until this block's copies have landed: the copies of the blocks
    // issued after it may stay in flight
    const int ahead = min(kRing - 1, nb - 1 - b);
    static_assert(kRing <= 4, "wait ladder covers up to 3 blocks ahead");
    if (ahead >= 3) wait_copies<3 * NI>();
    else if (ahead == 2) wait_copies<2 * NI>();
    else if (ahead == 1) wait_copies<NI>();
    else wait_copies<0>();

    const char* sk = ring + (b % kRing) * C::SLOT;
    const char* sv = sk + C::KV;
    const int valid = min(16, end - (start + 16 * b));
    // S = K Q^T; K operand: token head-lane, chunk (D/32)*grp + st, swizzled
    f32x4 s = f32x4{};
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const int ch = (D / 32) * grp + st;
      const bf16x8 ka =
          *(const bf16x8*)(sk + head * C::ROW + ((ch ^ (head % C::NCH)) * 16));
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[st], s, 0, 0, 0);
    }
    if (valid < 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = (4 * grp + r < valid) ? s[r] : kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx;
    const bool need = mt > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(need)) {
      // per-head decision: heads that do not need it keep m and scale by 1
      const float m_new = need ? fmaxf(m_run, mt) : m_run;
      const float alpha =
          (!need || m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      // accumulator rows are heads 4*grp + r; their alpha lives in lane 4*grp + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
        for (int m = 0; m < DPL; ++m) acc[m][r] *= ar;
      }
    }
    const float mu = (m_run == kNegInf) ? 0.f : m_run;
    bf16x4 pa;
    float ps[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ps[r] = __builtin_amdgcn_exp2f(s[r] - mu);
      pa[r] = (__bf16)ps[r];
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // V operand rows 4*grp + i, elements DPL*head .. +DPL-1
    u32x4 vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* vp = sv + (4 * grp + i) * C::ROW + head * DPL * 2;
      if constexpr (DPL == 8) {
        vr[i] = *(const u32x4*)vp;
      } else {
        const u32x2 y = *(const u32x2*)vp;
        vr[i] = u32x4{y[0], y[1], 0, 0};
      }
    }
    // O += P V
#pragma unroll
    for (int m = 0; m < DPL; ++m) {
      const uint32_t lo = elem16(vr[0], m) | (elem16(vr[1], m) << 16);
      const uint32_t hi = elem16(vr[2], m) | (elem16(vr[3], m) << 16);
      const bf16x4 vb = __builtin_bit_cast(bf16x4, u32x2{lo, hi});
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[m], 0, 0, 0);
    }
  }

  // row sums of the four lane groups (same head, different tokens)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // this lane's accumulator rows are heads 4*grp + r
  const int64_t orow0 = (int64_t)t0 * a.Hq + g * G;
  const int64_t prow0 = ((int64_t)n * a.Hq + g * G) * a.max_parts + p;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hh = 4 * grp + r;
    const float lr = __shfl(l_run, hh);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (hh < G) {
      if (np == 1) {
        uint32_t w[DPL / 2];
#pragma unroll
        for (int m = 0; m < DPL; m += 2)
          w[m / 2] = (uint32_t)to_bf16_bits(acc[m][r] * inv) |
                     ((uint32_t)to_bf16_bits(acc[m + 1][r] * inv) << 16);
        uint16_t* dst = (uint16_t*)a.o + (orow0 + hh) * D + DPL * head;
        if constexpr (DPL == 8) *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
        else *(u32x2*)dst = u32x2{w[0], w[1]};
      } else {
        float* dst = a.ws_o + (prow0 + (int64_t)hh * a.max_parts) * D + DPL * head;
#pragma unroll
        for (int m = 0; m < DPL; m += 4)
          *(f32x4*)(dst + m) =
              f32x4{acc[m][r] * inv, acc[m + 1][r] * inv, acc[m + 2][r] * inv, acc[m + 3][r] * inv};
      }
    }
  }
  if (lane < G) {
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : kNegInf;
    if (np == 1) {
      if (a.lse != nullptr) a.lse[orow0 + lane] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
    } else {
      a.ws_lse[prow0 + (int64_t)lane * a.max_parts] = lse2;
    }
  }
}

// Merge of the split-KV partials of one (sequence, KV head, query head, d).
// Sequences with one partition were finished by the split kernel. The loads
// of the metadata, of every partial's lse and of every partial output
// element are issued together (slots past the sequence's last partition are
// read but not used), so the merge costs one memory round trip.
constexpr int kMergeMaxParts = 16;

// Grid: (sequence, KV head, chunk of 256 (head, d) items); one item per thread.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(PagedArgs a, int chunks) {
  const int G = a.Hq / a.Hkv;
  const int chunk = blockIdx.x % chunks;
  const int g = (blockIdx.x / chunks) % a.Hkv;
  const int n = blockIdx.x / chunks / a.Hkv;
  const int i = chunk * 256 + threadIdx.x;
  if (i >= G * D) return;
  const int hh = i / D, d = i % D;
  const int MP = a.max_parts;  // <= kMergeMaxParts on this path
  const int64_t r0 = ((int64_t)n * a.Hq + g * G + hh) * MP;
  float lse[kMergeMaxParts], ov[kMergeMaxParts];
#pragma unroll
  for (int q = 0; q < kMergeMaxParts; ++q) {
    if (q < MP) {
      lse[q] = a.ws_lse[r0 + q];
      ov[q] = a.ws_o[(r0 + q) * D + d];
    }
  }
  const bool single = a.qsl == nullptr || a.qsl[n + 1] - a.qsl[n] == 1;
  const int L = a.seq_lens[n];
  const int t0 = a.qsl != nullptr ? a.qsl[n] : n;
  if (!single || L <= 0) return;
  const int np = (L + a.partition_size - 1) / a.partition_size;
  if (np <= 1) return;
  float M = kNegInf;
#pragma unroll
  for (int q = 0; q < kMergeMaxParts; ++q)
    if (q < np) M = fmaxf(M, lse[q]);
  float wsum = 0.f, osum = 0.f;
#pragma unroll
  for (int q = 0; q < kMergeMaxParts; ++q) {
    if (q < np) {
      const float w = (lse[q] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(lse[q] - M);
      wsum += w;
      osum += w * ov[q];
    }
  }
  const float out = wsum > 0.f ? osum / wsum : 0.f;
  ((uint16_t*)a.o)[((int64_t)t0 * a.Hq + g * G + hh) * D + d] = to_bf16_bits(out);
  if (a.lse != nullptr && d == 0)
    a.lse[(int64_t)t0 * a.Hq + g * G + hh] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : kNegInf;
}

// The same merge for any number of partitions: loops over the partials.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_loop_kernel(PagedArgs a) {
  const int g = blockIdx.x % a.Hkv, n = blockIdx.x / a.Hkv;
  const int tid = threadIdx.x;
  if (a.qsl != nullptr && a.qsl[n + 1] - a.qsl[n] != 1) return;
  const int L = a.seq_lens[n];
  if (L <= 0) return;
  const int np = (L + a.partition_size - 1) / a.partition_size;
  if (np <= 1) return;
  const int t0 = a.qsl != nullptr ? a.qsl[n] : n;
  const int G = a.Hq / a.Hkv;
  const int64_t row0 = ((int64_t)n * a.Hq + g * G) * a.max_parts;
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D, d = i % D;
    const int64_t r0 = row0 + (int64_t)hh * a.max_parts;
    float M = kNegInf;
    for (int q = 0; q < np; ++q) M = fmaxf(M, a.ws_lse[r0 + q]);
    float wsum = 0.f, osum = 0.f;
    for (int q = 0; q < np; ++q) {
      const float lq = a.ws_lse[r0 + q];
      const float w = (lq == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(lq - M);
      wsum += w;
      osum += w * a.ws_o[(r0 + q) * D + d];
    }
    const float out = wsum > 0.f ? osum / wsum : 0.f;
    ((uint16_t*)a.o)[((int64_t)t0 * a.Hq + g * G + hh) * D + d] = to_bf16_bits(out);
    if (a.lse != nullptr && d == 0)
      a.lse[(int64_t)t0 * a.Hq + g * G + hh] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_paged_decode_bf16(const PagedArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const dim3 grid((unsigned)((int64_t)a.max_parts * a.Hkv * a.num_seqs));
  if (a.d == 128)
    hipLaunchKernelGGL((decode_kernel<128>), grid, dim3(64), 0, s, a, c);
  else
    hipLaunchKernelGGL((decode_kernel<64>), grid, dim3(64), 0, s, a, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;  // one partition: nothing to merge
  if (a.max_parts <= kMergeMaxParts) {
    const int chunks = ((a.Hq / a.Hkv) * a.d + 255) / 256;
    const dim3 mgrid((unsigned)((int64_t)chunks * a.Hkv * a.num_seqs));
    if (a.d == 128)
      hipLaunchKernelGGL((decode_merge_kernel<128>), mgrid, dim3(256), 0, s, a, chunks);
    else
      hipLaunchKernelGGL((decode_merge_kernel<64>), mgrid, dim3(256), 0, s, a, chunks);
  } else {
    const dim3 mgrid((unsigned)((int64_t)a.Hkv * a.num_seqs));
    if (a.d == 128)
      hipLaunchKernelGGL((decode_merge_loop_kernel<128>), mgrid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_merge_loop_kernel<64>), mgrid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace attn
