// Tiled causal attention prefill, bf16 in / fp32 accumulate, for gfx950.
//
// What is computed ("Fast attention kernels and operator fusion",
// the-ai.news, section "FlashAttention-style attention and paged
// attention", first paragraph): queries, keys and values are processed in
// blocks; for each key block the kernel forms part of the scores, updates the
// running softmax statistics and accumulates the output on chip, so the
// T x T score matrix never exists in HBM. The result equals the naive
// sequence Q K^T -> scale -> causal mask -> softmax -> @V ("Hugging Face
// attention profiling guide", aiexpert.news, second paragraph) up to
// rounding order.
//
// Work decomposition
//   workgroup  = NW waves = (batch b | sequence n, query head h, tile of
//                BM = 32*NW query rows); K/V head = h / (Hq/Hkv).
//   key tile   = BN = 64 keys, staged in LDS (double buffered: the next
//                tile's global loads are in flight while the current tile is
//                computed).
//   wave       = 32 query rows. The wave computes the TRANSPOSED scores
//                S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that each lane
//                owns one query column: the row max and row sum of the
//                softmax are then in-lane reductions plus one exchange with
//                the lane 32 apart. O^T = V^T P^T is the second MFMA chain;
//                P^T is fed straight from the S^T accumulators (rounded to
//                bf16), with no LDS round trip.
//
// MFMA 32x32x16 bf16 operand layout (checked on gfx950): lane l holds
//   A[i = l%32][k = 8*(l/32) + e], B[k = 8*(l/32) + e][j = l%32], e = 0..7,
//   C[i = 8*(r/4) + 4*(l/32) + r%4][j = l%32], r = 0..15.
// The A rows of S^T are loaded in the order sigma(i) (bits 2 and 3 of i
// swapped); then accumulator register r of key block kb in lane l holds key
//   32*kb + 16*(r/8) + 8*(l/32) + r%8,
// so registers 8h..8h+7 are exactly the B operand (keys 16h + 8*(l/32) + e)
// of the P^T V^T product, and V^T is read from LDS as one 16-byte row piece.
//
// Online softmax (the pages say "updates the softmax statistics"; the
// recurrence here is the standard running max / running sum): scores are
// taken in log2 units t = s * scale * log2(e). A row keeps a reference max m;
// the weights are p = 2^(t - m), the running sum l and the accumulator O are
// rescaled by 2^(m_old - m_new) only when the tile's max exceeds m by more
// than 8 (then p <= 2^8 at most, harmless in fp32 and bf16). The final
// o = O / l is exact whatever reference m was used.
//
// Causal tile skipping: a workgroup visits only the key tiles up to its last
// query; a wave skips the compute of tiles entirely after its own 32 rows.
// Masking (select to -inf) is applied only on tiles that straddle the
// diagonal or the end of the keys.

#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native vector types rather than HIP's struct-based vectors: they stay in
// registers through inlining, where the struct types can end up in scratch.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BN = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kNegInf = -__builtin_inff();

template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;           // threads
  static constexpr int BM = NW * 32;           // query rows per workgroup
  static constexpr int KP = D * 2 + 16;        // LDS pitch of a K row (bytes), padded
  static constexpr int VP = BN * 2 + 16;       // LDS pitch of a V^T row (bytes), padded
  static constexpr int K_BYTES = BN * KP;
  static constexpr int V_BYTES = D * VP;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int NDC = D / 8;            // 16-byte chunks per row
  static constexpr int K_ROWS = NT / NDC;      // K rows per load pass
  static constexpr int K_PASSES = BN / K_ROWS;
  static constexpr int NKG = NT / NDC;         // V key groups
  static constexpr int KPG = BN / NKG;         // keys per V key group
  static_assert(K_PASSES >= 1 && BN % K_ROWS == 0, "K tile mapping");
  static_assert(KPG == 2 || KPG == 4, "V tile mapping");
};

// Where a workgroup's K/V rows live.
template <bool PAGED>
struct KvSrc;

template <>
struct KvSrc<false> {
  const uint16_t* k;  // K[b][g] base, rows of D elements
  const uint16_t* v;
  template <int D>
  __device__ __forceinline__ int64_t row_off(int key) const { return (int64_t)key * D; }
};

template <>
struct KvSrc<true> {
  const uint16_t* k;  // cache base [num_blocks][Hkv][16][D], already offset by head g
  const uint16_t* v;
  const int32_t* table;  // this sequence's block table row
  int64_t block_stride;  // Hkv * 16 * D elements
  template <int D>
  __device__ __forceinline__ int64_t row_off(int key) const {
    const int64_t phys = table[key >> 4];
    return phys * block_stride + (int64_t)(key & 15) * D;
  }
};

struct Prefetch {
  u32x4 k[4];
  u32x4 v[4];
};

__device__ __forceinline__ int sigma32(int i) {
  // swap bits 2 and 3
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Global -> registers for the key tile starting at n0. Rows past the last
// key re-read the last key's row (kv_len >= 1 whenever a tile exists): the
// loads stay unconditional and in bounds, never touch storage past the
// sequence, and the copies are harmless because those keys' scores are
// masked to -inf, so their weights are exactly 0 and their (finite) values
// contribute exactly 0.
template <int D, int NW, bool PAGED>
__device__ __forceinline__ void load_tile(Prefetch& pf, const KvSrc<PAGED>& src, int n0,
                                          int kv_len, int tid) {
  using C = Cfg<D, NW>;
  const int chunk = tid % C::NDC;
#pragma unroll
  for (int i = 0; i < C::K_PASSES; ++i) {
    const int row = tid / C::NDC + i * C::K_ROWS;
    const int key = min(n0 + row, kv_len - 1);
    pf.k[i] = *(const u32x4*)(src.k + src.template row_off<D>(key) + chunk * 8);
  }
  const int dc = tid / C::NKG;
  const int kg = tid % C::NKG;
#pragma unroll
  for (int i = 0; i < C::KPG; ++i) {
    const int key = min(n0 + kg * C::KPG + i, kv_len - 1);
    pf.v[i] = *(const u32x4*)(src.v + src.template row_off<D>(key) + dc * 8);
  }
}

// Registers -> LDS: K row-major (padded), V transposed to V^T[d][key] (padded).
template <int D, int NW>
__device__ __forceinline__ void store_tile(const Prefetch& pf, char* stage, int tid) {
  using C = Cfg<D, NW>;
  char* sk = stage;
  char* sv = stage + C::K_BYTES;
  const int chunk = tid % C::NDC;
#pragma unroll
  for (int i = 0; i < C::K_PASSES; ++i) {
    const int row = tid / C::NDC + i * C::K_ROWS;
    *(u32x4*)(sk + row * C::KP + chunk * 16) = pf.k[i];
  }
  const int dc = tid / C::NKG;
  const int kg = tid % C::NKG;
  uint32_t w[4][4] = {};
#pragma unroll
  for (int i = 0; i < C::KPG; ++i) {
    w[i][0] = pf.v[i][0];
    w[i][1] = pf.v[i][1];
    w[i][2] = pf.v[i][2];
    w[i][3] = pf.v[i][3];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // element j of each of the KPG rows, packed in key order
    char* dst = sv + (dc * 8 + j) * C::VP + kg * C::KPG * 2;
    if constexpr (C::KPG == 4) {
      uint32_t e0, e1, e2, e3;
      if (j & 1) {
        e0 = w[0][j >> 1] >> 16; e1 = w[1][j >> 1] >> 16;
        e2 = w[2][j >> 1] >> 16; e3 = w[3][j >> 1] >> 16;
      } else {
        e0 = w[0][j >> 1] & 0xffffu; e1 = w[1][j >> 1] & 0xffffu;
        e2 = w[2][j >> 1] & 0xffffu; e3 = w[3][j >> 1] & 0xffffu;
      }
      *(u32x2*)dst = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    } else {
      uint32_t e0, e1;
      if (j & 1) {
        e0 = w[0][j >> 1] >> 16; e1 = w[1][j >> 1] >> 16;
      } else {
        e0 = w[0][j >> 1] & 0xffffu; e1 = w[1][j >> 1] & 0xffffu;
      }
      *(uint32_t*)dst = e0 | (e1 << 16);
    }
  }
}

// One workgroup's problem, resolved from the grid position.
struct Problem {
  const uint16_t* q;  // first row of this (b|n, h)
  uint16_t* o;
  float* lse;         // first row or nullptr
  int lse_stride;     // floats between consecutive rows' lse
  int row_stride;     // elements between consecutive query rows
  int q_len;          // query rows of this (b|n, h)
  int kv_len;         // keys available
  int ctx;            // absolute position of query row 0 (query i sees keys <= ctx + i)
  int m0;             // first query row of this workgroup
};

template <int D, int NW, bool PAGED, bool CAUSAL>
__device__ __forceinline__ void run_tile(const Problem& pb, const KvSrc<PAGED>& src, float c,
                                         char* lds) {
  using C = Cfg<D, NW>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;  // query column owned by this lane
  const int hf = lane >> 5;  // which half of the key rows

  // key range of the workgroup and of this wave
  const int wg_last_q = min(pb.m0 + C::BM, pb.q_len);  // exclusive
  const int wg_keys = CAUSAL ? min(pb.kv_len, pb.ctx + wg_last_q) : pb.kv_len;
  const int n_tiles = (wg_keys + BN - 1) / BN;
  const int wq0 = pb.m0 + wave * 32;
  const int w_last_q = min(wq0 + 32, pb.q_len);
  const int w_keys = wq0 >= pb.q_len ? 0 : (CAUSAL ? min(pb.kv_len, pb.ctx + w_last_q) : pb.kv_len);
  const int w_tiles = (w_keys + BN - 1) / BN;

  // Q^T fragments: B operand, lane holds Q[wq0 + lq][16*s + 8*hf + e]
  bf16x8 qf[D / 16];
  {
    const int qrow = wq0 + lq;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 val = u32x4{0, 0, 0, 0};
      if (qrow < pb.q_len)
        val = *(const u32x4*)(pb.q + (int64_t)qrow * pb.row_stride + 16 * s + 8 * hf);
      qf[s] = __builtin_bit_cast(bf16x8, val);
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;  // reference max, log2 units
  float l_run = 0.f;      // partial row sum over this lane's keys
  const int qpos = pb.ctx + wq0 + lq;  // absolute position of this lane's query

  Prefetch pf;
  if (n_tiles > 0) {
    load_tile<D, NW, PAGED>(pf, src, 0, pb.kv_len, tid);
    store_tile<D, NW>(pf, lds, tid);
  }
  // Every load of the prologue (Q fragments, first tile) has landed: with no
  // load outstanding at the loop entry, the waits inside the loop only cover
  // the prefetch of the next tile, which then overlaps the current tile's
  // compute.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int n0 = j * BN;
    if (j + 1 < n_tiles) load_tile<D, NW, PAGED>(pf, src, n0 + BN, pb.kv_len, tid);

    if (j < w_tiles) {
      const char* sk = lds + (j & 1) * C::STAGE;
      const char* sv = sk + C::K_BYTES;
      // S^T = K Q^T for 2 blocks of 32 keys
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const char* kp = sk + (32 * kb + sigma32(lq)) * C::KP + hf * 16;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          const bf16x8 a = *(const bf16x8*)(kp + st * 32);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
        }
      }
      // mask keys after the query (causal) and keys past the end
      const bool diag = CAUSAL ? (n0 + BN - 1 > pb.ctx + wq0) : false;
      if (diag || n0 + BN > pb.kv_len) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = n0 + 32 * kb + 16 * (r >> 3) + 8 * hf + (r & 7);
            const bool dead = (CAUSAL && key > qpos) || key >= pb.kv_len;
            s[kb][r] = dead ? kNegInf : s[kb][r];
          }
      }
      // tile row max (raw scores), shared by the two lane halves
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * c;
      const bool need = mt > m_run + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(need)) {
        // lanes that do not need it keep m and scale by 1, so a row's result
        // never depends on the other rows of the wave
        const float m_new = need ? fmaxf(m_run, mt) : m_run;
        const float alpha =
            (!need || m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      }
      const float mu = (m_run == kNegInf) ? 0.f : m_run;
      // weights p = 2^(s*c - m), row sum, and bf16 P^T fragments
      bf16x8 pk[4];
      float part[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * h + e], c, -mu));
            pk[2 * kb + h][e] = (__bf16)pv[e];
          }
          // pairwise partial sums: short dependency chains
          part[2 * kb + h] = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        }
      l_run += (part[0] + part[1]) + (part[2] + part[3]);
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* vp = sv + (32 * db + lq) * C::VP + hf * 16;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = *(const bf16x8*)(vp + kk * 32);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kk], acc[db], 0, 0, 0);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile<D, NW>(pf, lds + ((j + 1) & 1) * C::STAGE, tid);
    __syncthreads();
  }

  // epilogue: o = O / l, lse = m*ln2 + ln(l)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int qrow = wq0 + lq;
  if (qrow < pb.q_len) {
    uint16_t* orow = pb.o + (int64_t)qrow * pb.row_stride;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hf;
        __bf16 b0 = (__bf16)(acc[db][4 * g4 + 0] * inv);
        __bf16 b1 = (__bf16)(acc[db][4 * g4 + 1] * inv);
        __bf16 b2 = (__bf16)(acc[db][4 * g4 + 2] * inv);
        __bf16 b3 = (__bf16)(acc[db][4 * g4 + 3] * inv);
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *(u32x2*)(orow + d0) = u32x2{lo, hi};
      }
    if (pb.lse != nullptr && hf == 0)
      pb.lse[(int64_t)qrow * pb.lse_stride] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : kNegInf;
  }
}

// Workgroup id -> logical work index. Consecutive workgroup ids are spread
// round-robin over the 8 XCDs; this makes each XCD own a contiguous range of
// logical work, so that query heads sharing K/V (and tiles of the same head)
// run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical(int bid, int nwg) {
  const int x = bid & 7, slot = bid >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  return x * per + min(x, rem) + slot;
}

// Logical index -> (unit, query tile), longest tiles first. Units are
// (batch, head) pairs in head order, so GQA siblings are adjacent.
__device__ __forceinline__ void logical_to_work(int logical, int units, int n_qt, int& unit,
                                                int& qt) {
  if ((units & 7) == 0) {
    const int ux = units >> 3;            // units per XCD
    const int per = ux * n_qt;            // work per XCD
    const int x = logical / per, s = logical % per;
    qt = n_qt - 1 - s / ux;
    unit = x * ux + s % ux;
  } else {
    qt = n_qt - 1 - logical / units;
    unit = logical % units;
  }
}

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void prefill_bf16_kernel(PrefillArgs a, float c, int n_qt) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg<D, NW>::LDS];
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  int unit, qt;
  logical_to_work(logical, a.B * a.Hq, n_qt, unit, qt);
  const int b = unit / a.Hq, h = unit % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  Problem pb;
  const int64_t qoff = ((int64_t)b * a.Hq + h) * a.T * D;
  const int64_t kvoff = ((int64_t)b * a.Hkv + g) * a.T * D;
  pb.q = (const uint16_t*)a.q + qoff;
  pb.o = (uint16_t*)a.o + qoff;
  pb.lse = a.lse ? a.lse + ((int64_t)b * a.Hq + h) * a.T : nullptr;
  pb.lse_stride = 1;
  pb.row_stride = D;
  pb.q_len = a.T;
  pb.kv_len = a.T;
  pb.ctx = 0;
  pb.m0 = qt * Cfg<D, NW>::BM;
  KvSrc<false> src;
  src.k = (const uint16_t*)a.k + kvoff;
  src.v = (const uint16_t*)a.v + kvoff;
  run_tile<D, NW, false, CAUSAL>(pb, src, c, lds);
}

// Paged prefill: sequences with q_len >= 2 of a paged batch (chunked prefill).
// Their K/V tiles are gathered through the block table; q/o are token-major.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void paged_prefill_bf16_kernel(PagedArgs a, float c,
                                                                          int n_qt) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg<D, NW>::LDS];
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  int unit, qt;
  logical_to_work(logical, a.num_seqs * a.Hq, n_qt, unit, qt);
  const int n = unit / a.Hq, h = unit % a.Hq;
  const int t0 = a.qsl[n];
  const int q_len = a.qsl[n + 1] - t0;
  if (q_len < 2 || qt * Cfg<D, NW>::BM >= q_len) return;  // uniform over the workgroup
  const int L = a.seq_lens[n];
  const int g = h / (a.Hq / a.Hkv);
  Problem pb;
  pb.q = (const uint16_t*)a.q + ((int64_t)t0 * a.Hq + h) * D;
  pb.o = (uint16_t*)a.o + ((int64_t)t0 * a.Hq + h) * D;
  pb.lse = a.lse ? a.lse + (int64_t)t0 * a.Hq + h : nullptr;
  pb.lse_stride = a.Hq;
  pb.row_stride = a.Hq * D;
  pb.q_len = q_len;
  pb.kv_len = L;
  pb.ctx = L - q_len;
  pb.m0 = qt * Cfg<D, NW>::BM;
  KvSrc<true> src;
  src.k = (const uint16_t*)a.k_cache + (int64_t)g * kBlockSize * D;
  src.v = (const uint16_t*)a.v_cache + (int64_t)g * kBlockSize * D;
  src.table = a.block_table + (int64_t)n * a.max_blocks_per_seq;
  src.block_stride = (int64_t)a.Hkv * kBlockSize * D;
  run_tile<D, NW, true, true>(pb, src, c, lds);
}

constexpr int kNW = 4;

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  constexpr int BM = Cfg<128, kNW>::BM;
  const int n_qt = (a.T + BM - 1) / BM;
  const dim3 grid((unsigned)(n_qt * a.B * a.Hq));
  const dim3 block(kNW * 64);
  if (a.d == 128) {
    if (a.causal)
      hipLaunchKernelGGL((prefill_bf16_kernel<128, kNW, true>), grid, block, 0, s, a, c, n_qt);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<128, kNW, false>), grid, block, 0, s, a, c, n_qt);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((prefill_bf16_kernel<64, kNW, true>), grid, block, 0, s, a, c, n_qt);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<64, kNW, false>), grid, block, 0, s, a, c, n_qt);
  }
  return hipGetLastError();
}

hipError_t launch_paged_prefill_bf16(const PagedArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  constexpr int BM = Cfg<128, kNW>::BM;
  const int n_qt = (a.max_query_len + BM - 1) / BM;
  const dim3 grid((unsigned)(n_qt * a.num_seqs * a.Hq));
  const dim3 block(kNW * 64);
  if (a.d == 128)
    hipLaunchKernelGGL((paged_prefill_bf16_kernel<128, kNW>), grid, block, 0, s, a, c, n_qt);
  else
    hipLaunchKernelGGL((paged_prefill_bf16_kernel<64, kNW>), grid, block, 0, s, a, c, n_qt);
  return hipGetLastError();
}

}  // namespace attn
