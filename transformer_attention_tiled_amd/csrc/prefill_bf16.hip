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
// Work decomposition (details with the two-group schedule below)
//   workgroup  = 8 waves = (batch b | sequence n, query head h, tile of 256
//                query rows); K/V head = h / (Hq/Hkv).
//   key tile   = BN = 64 keys. K and V tiles are copied from HBM straight
//                into LDS (global_load_lds_dwordx4: each instruction moves
//                one contiguous KiB, lane L's 16 bytes to M0 + 16 L), into
//                four buffers each, three tiles ahead. Each lane's source
//                offsets are fixed for the whole loop and the tile base is a
//                scalar (for a paged cache: the block's table entry, read
//                ahead with a scalar load), so the copies cost no vector ALU
//                work; only the ragged last tile clamps its rows to the last
//                key.
//   wave       = 32 query rows. The wave computes the TRANSPOSED scores
//                S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that each lane
//                owns one query column: the row max and row sum of the
//                softmax are in-lane reductions plus one exchange with the
//                lane 32 apart. O^T = V^T P^T is the second MFMA chain; P^T
//                is fed straight from the S^T accumulators (rounded to bf16).
//                The V^T operand comes from the LDS transpose read
//                ds_read_b64_tr_b16. Row sums add the unrounded fp32 weights.
//
// MFMA 32x32x16 bf16 operand layout (checked on gfx950): lane l holds
//   A[i = l%32][k = 8*(l/32) + e], B[k = 8*(l/32) + e][j = l%32], e = 0..7,
//   C[i = 8*(r/4) + 4*(l/32) + r%4][j = l%32], r = 0..15.
// The A rows of S^T are read in the order sigma(i) (bits 2 and 3 of i
// swapped); then accumulator register r of key block kb in lane l holds key
//   32*kb + 16*(r/8) + 8*(l/32) + r%8,
// so registers 8h..8h+7 are exactly the B operand (keys 16h + 8*(l/32) + e)
// of the P^T V^T product.
//
// ds_read_b64_tr_b16 (checked on gfx950): in each group of 16 lanes, lane
// j = 4a + b receives element b of the 8-byte chunks addressed by lanes
// 4r + a, r = 0..3. With lane i of a group addressing row K0 + i/4 at column
// d0 + 4*(i%4), lane j receives V[K0..K0+3][d0 + j]: four consecutive keys
// of one d column. Two such reads give the 8 keys of one V^T operand.
//
// LDS layout: K and V tiles row-major (one key per row). K tiles have their
// 16-byte chunks XOR-swizzled per row with f(r) = 4*(r%4) + (r/4)%4, which
// spreads the K operand reads (16 rows, same chunk) over the banks; V tiles
// have their own swizzle for the transpose reads (below).
//
// Online softmax (the pages say "updates the softmax statistics"; the
// recurrence here is the standard running max / running sum): scores are
// taken in log2 units t = s * scale * log2(e). A row keeps a reference max m;
// the weights are p = 2^(t - m), the running sum l and the accumulator O are
// rescaled by 2^(m_old - m_new) only when the tile's max exceeds m by more
// than 8 (then p <= 2^8 at most, harmless in fp32 and bf16). The final
// o = O / l is exact whatever reference m was used.
// The softmax phase's vector work competes with the other wave's MFMAs, so
// it is kept to exp2, bf16 rounding and sums: Q is multiplied by
// c = scale * log2(e) once (rounded to bf16) and the score MFMA starts from
// -m instead of 0, so it yields t - m itself; the tile max is computed only
// when some lane's weights sum past 2^8 (a weight past 2^8 implies it).
//
// Causal tile skipping: a workgroup visits only the key tiles up to its last
// query; a wave skips the compute of tiles entirely after its own 32 rows.
// Masking (select to -inf) is applied only on tiles that straddle the
// diagonal or the end of the keys.

#include <hip/hip_runtime.h>

#include <algorithm>

#include <type_traits>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int BN = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int swz(int r, int nch) { return (4 * (r & 3) + ((r >> 2) & 3)) & (nch - 1); }

__device__ __forceinline__ int sigma32(int i) {
  // swap bits 2 and 3
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// HBM -> LDS copy, 16 bytes per lane to LDS address lds + 16 L.
// Scalar 64-bit base + per-lane 32-bit byte offset.
// M0 holds the LDS address and is set inside the same asm statement; it is
// declared clobbered, and the compiler keeps no value of its own in M0 across
// these statements (on gfx950 LDS instructions do not read M0), so its
// warning that a reserved register is clobbered is expected here.
__device__ __forceinline__ void copy_saddr(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}
// Per-lane 64-bit address.
__device__ __forceinline__ void copy_vaddr(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds), "v"(src) : "memory", "m0");
}

// Where a workgroup's K/V rows live.
template <bool PAGED>
struct KvSrc;

template <>
struct KvSrc<false> {
  const char* k;  // K[b][g] row 0
  const char* v;
};

template <>
struct KvSrc<true> {
  const char* k;         // cache base [num_blocks][Hkv][16][D], offset by head g
  const char* v;
  const int32_t* table;  // this sequence's block table row
  int64_t block_bytes;   // Hkv * 16 * D * 2
};

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
  // Key range: tiles tile0 .. tile1 - 1 of the workgroup's keys (the whole
  // range: 0 .. INT_MAX). With part_o set, the workgroup writes, per query
  // row, its normalised fp32 partial output and log2-sum-exp over that range
  // (to be merged with the other ranges' partials) instead of o and lse.
  int tile0 = 0;
  int tile1 = 0x7fffffff;
  float* part_o = nullptr;      // row 0's partial output [D] fp32
  float* part_lse = nullptr;    // row 0's partial log2-sum-exp
  int64_t part_stride = 0;      // floats between consecutive rows' partial outputs
  int64_t part_lse_stride = 0;  // floats between consecutive rows' partial lse
};

// ---------------------------------------------------------------------------
// Two-group schedule. On gfx950 the vector ALU work of one wave runs alongside
// the MFMA work of another wave on the same SIMD, but hardly alongside the
// MFMA work of its own instruction stream. So the workgroup has 8 waves in
// two groups of 4 (waves w and w+4 share a SIMD) that run half a tile apart,
// separated by workgroup barriers: while one group does the products of a
// tile (M phase: O += P V for the previous tile, then S^T = K Q^T for this
// one), the other does the softmax of its tile (S phase), then they swap.
//
//   phase t:     0      1      2      3      4     ...
//   group 0:    M(0)   S(0)   M(1)   S(1)   M(2)
//   group 1:     -     M(0)   S(0)   M(1)   S(1)
//
// K and V tiles live in four LDS buffers each. At the start of its S(j)
// each wave issues its share of the copies of K tile j+3 and V tile j+2,
// so the M phase holds nothing but LDS reads and MFMAs; at the end of M(j)
// it waits for its own copies of K tile j+1 and V tile j (issued in
// S(j-2)). The barrier that follows the later group's M(j) therefore
// publishes both tiles to every wave before either group starts M(j+1). The
// buffer a copy overwrites was last read in M(j-1) of both groups, which
// ended before an earlier barrier.
//
// A workgroup covers 256 query rows; the two waves on SIMD s own rows
// 64s .. 64s+31 (group 0) and 64s+32 .. 64s+63 (group 1), so both stop at the
// same key tile.

constexpr int kPPW = 8;       // waves per workgroup
constexpr int kPPBM = 256;    // query rows per workgroup
constexpr int kBufs = 4;      // LDS buffers for K tiles (and as many for V)

template <int D>
struct PP {
  static constexpr int ROW = D * 2;
  static constexpr int NCH = D / 8;
  static constexpr int TILE = BN * ROW;          // bytes of one K or V tile
  static constexpr int LDS = 2 * kBufs * TILE;   // 128 KiB at D = 128
  static constexpr int CP = TILE / 1024 / kPPW;  // KiB copies per wave per tile
  static constexpr int RPC = 1024 / ROW;         // rows per KiB copy
  static_assert(CP >= 1 && TILE % (1024 * kPPW) == 0, "tile copy split");
};

// V tiles use their own swizzle: chunk c of row r sits at chunk c ^ vswz(r),
// which moves each of 4 consecutive rows (D = 128; 2 pairs of rows at D = 64)
// into its own quarter of the 64 banks. A transpose read touches 4 rows x
// 64 bytes per 32 lanes, so it is conflict free, and its address is one
// per-lane base per 32-column block plus immediates for the row offsets.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS accesses and keeps the compiler from
// moving any instruction across it (the two groups' phases must not blur).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// This wave's share of the copies of one K or V tile (rows n0 .. n0+63) into
// the LDS buffer at `buf`. Rows past the last key re-read the last key's row.
template <int D, bool PAGED>
__device__ __forceinline__ void pp_copy(const char* base, const KvSrc<PAGED>& src, int n0,
                                        int kv_len, uint32_t buf, int wave, int lane,
                                        const uint32_t* off) {
  using C = PP<D>;
  const bool full = n0 + BN <= kv_len;
#pragma unroll
  for (int s = 0; s < C::CP; ++s) {
    const uint32_t l = buf + (wave * C::CP + s) * 1024;
    const int t = (wave * C::CP + s) * C::RPC + lane / (C::ROW / 16);  // tile row
    if constexpr (!PAGED) {
      if (full) {
        copy_saddr(base + (int64_t)n0 * C::ROW, off[s], l);
      } else {
        const int tc = min(t, kv_len - 1 - n0);
        copy_saddr(base + (int64_t)n0 * C::ROW, off[s] + (uint32_t)((tc - t) * C::ROW), l);
      }
    } else {
      const int key = min(n0 + t, kv_len - 1);
      const int64_t row = paged_block_index(src.table[key >> 4]) * src.block_bytes + (key & 15) * C::ROW;
      copy_vaddr(base + row + (off[s] - (uint32_t)(t * C::ROW)), l);
    }
  }
}

// Steady-state copy of a full tile: `tile` is the tile's first row in HBM,
// `dst` this wave's first KiB in the LDS buffer.
template <int D>
__device__ __forceinline__ void pp_copy_full(const char* tile, uint32_t dst, const uint32_t* off) {
  using C = PP<D>;
#pragma unroll
  for (int s = 0; s < C::CP; ++s) copy_saddr(tile, off[s], dst + s * 1024);
}

// Steady-state copy of a full tile through the block table. The RPC rows of
// one KiB copy instruction are consecutive keys inside one 16-key block, so
// the instruction needs one table entry, the same for the whole wave:
// `blk[s]`, read ahead of time with a scalar load. `dst` is this wave's first
// KiB in the LDS buffer.
template <int D>
__device__ __forceinline__ void pp_copy_paged(const char* base, int64_t block_bytes,
                                              const int* blk, int n0, uint32_t dst, int wave,
                                              const uint32_t* off) {
  using C = PP<D>;
  static_assert(kBlockSize % C::RPC == 0, "a copy instruction stays inside one block");
#pragma unroll
  for (int s = 0; s < C::CP; ++s) {
    const int tb = (wave * C::CP + s) * C::RPC;  // first tile row of copy s
    const char* row = base + paged_block_index(blk[s]) * block_bytes + ((n0 + tb) & 15) * C::ROW;
    copy_saddr(row, off[s] - (uint32_t)(tb * C::ROW), dst + s * 1024);
  }
}

// M phase: O^T += V^T P^T over the previous tile (16 MFMAs at D = 128), then
// S^T = K Q^T for this tile (16 MFMAs). The instruction order is pinned so
// that the LDS operand reads run LOOKAHEAD MFMAs ahead of their MFMA: the
// other wave on the SIMD is in its softmax phase meanwhile, so any MFMA that
// waits for LDS leaves the matrix core idle.
// kabs / vabs: per-lane LDS addresses within K buffer 0 / V buffer 0; KOFF
// and VOFF select the buffers and become instruction offsets, so the phase
// needs no vector ALU work for addressing.
template <int D, bool DO_PV, bool DO_S, int KOFF, int VOFF>
__device__ __forceinline__ void m_phase(f32x16* acc, f32x16* sc, const bf16x8* pk,
                                        const bf16x8* qf, const uint32_t* vabs,
                                        const uint32_t* kabs, const f32x16& cinit) {
  using C = PP<D>;
  constexpr int LOOKAHEAD = 8;
  constexpr int NPV = DO_PV ? 4 * (D / 32) : 0;  // MFMAs, 2 transpose reads each
  constexpr int NS = DO_S ? 2 * (D / 16) : 0;    // MFMAs, 1 b128 read each
  if constexpr (DO_PV) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        u32x2 half[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const lds_char* p =
              (const lds_char*)(uintptr_t)vabs[db] + (VOFF + (16 * kk + 4 * hh) * C::ROW);
          half[hh] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                         (s16x4 __attribute__((address_space(3)))*)p));
        }
        const u32x4 both = {half[0][0], half[0][1], half[1][0], half[1][1]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both),
                                                          pk[kk], acc[db], 0, 0, 0);
      }
    }
  }
  if constexpr (DO_S) {
    sc[0] = cinit;
    sc[1] = cinit;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8 __attribute__((address_space(3)))*)(
            (const lds_char*)(uintptr_t)kabs[s] + (KOFF + 32 * kb * C::ROW));
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc[kb], 0, 0, 0);
      }
    }
  }
  // pinned order: reads of the first LOOKAHEAD MFMAs, then MFMA k followed by
  // the reads of MFMA k + LOOKAHEAD
  constexpr int N = NPV + NS;
  constexpr int first = (LOOKAHEAD < NPV ? 2 * LOOKAHEAD : 2 * NPV) +
                        (LOOKAHEAD > NPV ? (LOOKAHEAD - NPV < NS ? LOOKAHEAD - NPV : NS) : 0);
  __builtin_amdgcn_sched_group_barrier(0x100, first, 0);
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    const int nx = k + LOOKAHEAD;
    if (nx < NPV)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    else if (nx < N)
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <int D, bool PAGED, bool CAUSAL>
__device__ __forceinline__ void run_pp(const Problem& pb, const KvSrc<PAGED>& src, float c,
                                       char* lds) {
  using C = PP<D>;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31;  // query column owned by this lane
  const int hf = lane >> 5;  // which half of the key rows
  const int grp = wave >> 2;
  const int wq0 = pb.m0 + 64 * (wave & 3) + 32 * grp;

  const int wg_last_q = min(pb.m0 + kPPBM, pb.q_len);
  const int wg_keys = CAUSAL ? min(pb.kv_len, pb.ctx + wg_last_q) : pb.kv_len;
  const int n_all = (wg_keys + BN - 1) / BN;
  const int w_last_q = min(wq0 + 32, pb.q_len);
  const int w_keys =
      wq0 >= pb.q_len ? 0 : (CAUSAL ? min(pb.kv_len, pb.ctx + w_last_q) : pb.kv_len);
  // this workgroup's key tiles: t0 .. t0 + n - 1 (a piece of the range, or
  // all of it); the loop counts j = 0 .. n, tile t0 + j
  const int t0 = min(pb.tile0, n_all);
  const int n = min(pb.tile1, n_all) - t0;
  // tiles this wave computes, counted from t0 (<= n)
  const int wt = max(0, min((w_keys + BN - 1) / BN, t0 + n) - t0);

  // per-lane source offsets of the copies (tile-relative): K and V tiles
  // are swizzled differently
  uint32_t koff[C::CP], voff[C::CP];
#pragma unroll
  for (int s = 0; s < C::CP; ++s) {
    const int lds_off = (wave * C::CP + s) * 1024 + 16 * lane;
    const int t = lds_off / C::ROW;
    const int pc = (lds_off % C::ROW) / 16;
    koff[s] = (uint32_t)(t * C::ROW + ((pc ^ swz(t, C::NCH)) * 16));
    voff[s] = (uint32_t)(t * C::ROW + ((pc ^ vswz<D>(t)) * 16));
  }
  // LDS read offsets (buffer-relative). K operand of key block kb and
  // k-step s: row 32 kb + sigma(lq), chunk (2 s + hf) ^ swz(row); the kb
  // part is an immediate. V^T operand of column block db: rows
  // 16 kk + 8 (g16 / 2) + 4 hh + i16 / 4 (kk, hh immediates).
  const int krow0 = sigma32(lq);
  const int g16 = lane >> 4, i16 = lane & 15;
  uint32_t kaddr[D / 16], vaddr[D / 32];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    kaddr[s] = (uint32_t)(krow0 * C::ROW + (((2 * s + hf) ^ swz(krow0, C::NCH)) * 16));
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int row = 8 * (g16 >> 1) + (i16 >> 2);
    const int chunk = 4 * db + 2 * (g16 & 1) + ((i16 >> 1) & 1);
    vaddr[db] = (uint32_t)(row * C::ROW + 16 * (chunk ^ vswz<D>(row)) + 8 * (i16 & 1));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto kbuf = [&](int j) { return lds0 + (uint32_t)((j % kBufs) * C::TILE); };
  auto vbuf = [&](int j) { return lds0 + (uint32_t)((kBufs + j % kBufs) * C::TILE); };
  // (the empty asm keeps the addresses in registers: recomputing them from
  // the lane id in every tile would cost vector ALU time in the M phase)
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kaddr[s] += lds0;
    asm volatile("" : "+v"(kaddr[s]));
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    vaddr[db] += lds0 + kBufs * C::TILE;
    asm volatile("" : "+v"(vaddr[db]));
  }

  // K tile 0 and the Q^T fragments (B operand, lane holds
  // Q[wq0 + lq][16*s + 8*hf + e]); both are waited for before the first
  // phase, then K tiles 1, 2 and V tiles 0, 1 are put in flight (in the
  // order the waits in the loop assume: K1, V0, then K2, V1).
  pp_copy<D, PAGED>(src.k, src, t0 * BN, pb.kv_len, kbuf(0), wave, lane, koff);
  bf16x8 qf[D / 16];
  {
    const int qrow = min(wq0 + lq, pb.q_len - 1);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = __builtin_bit_cast(
          bf16x8, *(const u32x4*)(pb.q + (int64_t)qrow * pb.row_stride + 16 * s + 8 * hf));
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (1 < n) pp_copy<D, PAGED>(src.k, src, (t0 + 1) * BN, pb.kv_len, kbuf(1), wave, lane, koff);
  pp_copy<D, PAGED>(src.v, src, t0 * BN, pb.kv_len, vbuf(0), wave, lane, voff);
  if (2 < n) pp_copy<D, PAGED>(src.k, src, (t0 + 2) * BN, pb.kv_len, kbuf(2), wave, lane, koff);
  if (1 < n) pp_copy<D, PAGED>(src.v, src, (t0 + 1) * BN, pb.kv_len, vbuf(1), wave, lane, voff);
  // fold the softmax scale in log2 units (c = scale * log2 e) into Q, once:
  // the score MFMA then yields c * s directly (each q * c rounded to bf16)
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)((float)qf[s][e] * c);
  {
    // M(0) multiplies P = 0 with the V buffer of "tile -1": make it zeros
    // (V tile 3, the first copy into that buffer, is issued in S(1), after
    // two more barriers)
    constexpr int PER = C::TILE / (kPPW * 64);  // bytes per thread
    lds_char* z = (lds_char*)(uintptr_t)(vbuf(kBufs - 1) + tid * PER);
#pragma unroll
    for (int i = 0; i < PER / 16; ++i)
      *(u32x4 __attribute__((address_space(3)))*)(z + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  }
  phase_barrier();

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  f32x16 sc[2] = {f32x16{}, f32x16{}};
  bf16x8 pk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = bf16x8{};
  float m_run = kNegInf;  // reference max, log2 units
  float nmu = 0.f;        // -m_run, or 0 while there is no reference
  // the score MFMA starts from nmu instead of 0, so it yields c * s - m_run:
  // the exponent of the weight, with no further vector work
  f32x16 negm = f32x16{};
  // wave-uniform: every lane has a reference (m_run moves only in the
  // rescale path below, so this is updated there)
  bool all_ref = false;
  float l_run = 0.f;      // partial row sum over this lane's keys
  const int qpos = pb.ctx + wq0 + lq;
  // Paged: the table entries of this wave's copy rows, read with scalar loads
  // one step before use (the copies of K tile t in S(t-3) and of V tile t in
  // S(t-2) need the same entries): ev for the V copy of this step, ek for the
  // K copy. Reads past the sequence are clamped to its last key.
  int ek[C::CP], ev[C::CP];
  auto table_row = [&](int tile, int s) -> int {
    if constexpr (PAGED) {
      const __attribute__((address_space(4))) int32_t* t4 =
          (const __attribute__((address_space(4))) int32_t*)src.table;
      const int key = min(tile * BN + (wave * C::CP + s) * C::RPC, pb.kv_len - 1);
      return t4[key >> 4];
    } else {
      return 0;
    }
  };
  if constexpr (PAGED) {
#pragma unroll
    for (int s = 0; s < C::CP; ++s) {
      ev[s] = table_row(t0 + 2, s);
      ek[s] = table_row(t0 + 3, s);
    }
  }

  // Both groups run the same sequence M(j), barrier, S(j), barrier; group 1
  // starts one barrier later (and group 0 ends with one), which puts the two
  // groups half a tile apart.
  const int n_full = pb.kv_len / BN;                          // tiles without a ragged end
  const uint32_t wdst = (uint32_t)(wave * C::CP * 1024);       // this wave's part of a tile
  if (grp == 1) phase_barrier();
  // one step per key tile; the buffer index B = j % 4 is a template constant
  // in each of the four unrolled copies, so LDS offsets are immediates
  auto step = [&](const int j, auto bconst) {
    constexpr int B = decltype(bconst)::value;
    // ---- M(j): O^T += V^T P^T (tile j-1), then S^T = K Q^T (tile j).
    // Both products, so the phase is one block: before the first tile P is
    // 0 and the V buffer read is zero-filled; at the wave's last tile wt the
    // scores are computed and ignored. A wave past its last tile (j > wt:
    // P of tile j-1 is 0 and the scores unused) skips the phase and only
    // keeps to the barriers.
    if (j <= wt)
      m_phase<D, true, true, B * C::TILE, ((B + kBufs - 1) % kBufs) * C::TILE>(acc, sc, pk, qf,
                                                                               vaddr, kaddr, negm);
    // this wave's copies of K tile j+1 and V tile j (issued at the start of
    // S(j-2)) have landed; the barrier after the later group's M(j) makes
    // every wave's copies visible before either group's M(j+1). Only the
    // copies issued in S(j-1) may still be in flight.
    if (j + 2 < n)
      wait_copies<2 * C::CP>();
    else if (j + 1 < n)
      wait_copies<C::CP>();
    else
      wait_copies<0>();
    phase_barrier();

    // ---- S(j): copies of K tile j+3 and V tile j+2 first (their buffers
    // held K tile j-1 and V tile j-2, last read in M(j-1) of both groups,
    // before the previous barrier), then mask, running max, weights, sums.
    if (j + 3 < n) {
      const uint32_t buf = lds0 + (uint32_t)(((B + 3) % kBufs) * C::TILE);
      if (t0 + j + 3 < n_full) {
        if constexpr (PAGED)
          pp_copy_paged<D>(src.k, src.block_bytes, ek, (t0 + j + 3) * BN, buf + wdst, wave, koff);
        else
          pp_copy_full<D>(src.k + (int64_t)(t0 + j + 3) * C::TILE, buf + wdst, koff);
      } else {
        pp_copy<D, PAGED>(src.k, src, (t0 + j + 3) * BN, pb.kv_len, buf, wave, lane, koff);
      }
    }
    if (j + 2 < n) {
      const uint32_t buf = lds0 + (uint32_t)((kBufs + (B + 2) % kBufs) * C::TILE);
      if (t0 + j + 2 < n_full) {
        if constexpr (PAGED)
          pp_copy_paged<D>(src.v, src.block_bytes, ev, (t0 + j + 2) * BN, buf + wdst, wave, voff);
        else
          pp_copy_full<D>(src.v + (int64_t)(t0 + j + 2) * C::TILE, buf + wdst, voff);
      } else {
        pp_copy<D, PAGED>(src.v, src, (t0 + j + 2) * BN, pb.kv_len, buf, wave, lane, voff);
      }
    }
    if constexpr (PAGED) {
#pragma unroll
      for (int s = 0; s < C::CP; ++s) {
        ev[s] = ek[s];
        ek[s] = table_row(t0 + j + 4, s);
      }
    }
    if (j < wt) {
      const int n0 = (t0 + j) * BN;
      const bool diag = CAUSAL ? (n0 + BN - 1 > pb.ctx + wq0) : false;
      if (diag || n0 + BN > pb.kv_len) {
        // register (kb, r) holds key n0 + 8 hf + o, o = 32 kb + 16 (r >> 3) +
        // (r & 7) a constant; the key is dead when past this lane's query
        // (o > qpos - n0 - 8 hf) or past the keys (o >= kv_len - n0 - 8 hf):
        // one bound per lane, one compare per register
        const int tk = pb.kv_len - n0 - 8 * hf;
        const int t = CAUSAL ? min(qpos - n0 - 8 * hf + 1, tk) : tk;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = 32 * kb + 16 * (r >> 3) + (r & 7);
            sc[kb][r] = o >= t ? kNegInf : sc[kb][r];
          }
      }
      // weights p = 2^(s*c - m) against the current reference max m: rounded
      // to bf16 for the product with V, summed in fp32 (v_dot2 on the packed
      // weights would be fewer instructions, but it cannot issue while the
      // other wave's MFMAs occupy the matrix core; plain adds can)
      auto weights = [&]() -> float {
        float part[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pv = __builtin_amdgcn_exp2f(sc[kb][8 * h + e]);
              pk[2 * kb + h][e] = (__bf16)pv;
              // each partial sum starts with its first weight (weights are
              // never -0, so this is the sum from 0)
              if (kb == 0 && h == 0 && e < 4)
                part[e & 3] = pv;
              else
                part[e & 3] += pv;
            }
        return (part[0] + part[1]) + (part[2] + part[3]);
      };
      float ts = weights();
      // The reference max must move when the tile's max exceeds it by more
      // than 8 (log2 units), i.e. when some weight exceeds 2^8; then this
      // lane's sum exceeds 2^8 too. Only then (or while a lane has no
      // reference yet) is the tile max computed, the same decision taken
      // as when it is computed up front, and the weights recomputed, so the
      // result is the same; most tiles skip the max entirely.
      if (__builtin_amdgcn_ballot_w64(ts > 256.f) || !all_ref) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        const float tmax = mx - nmu;  // this lane's max of c * s
        if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleThreshold)) {
          const float mt = fmaxf(tmax, __shfl_xor(tmax, 32));
          const bool need = mt > m_run + kRescaleThreshold;
          const float m_new = need ? mt : m_run;
          const float alpha =
              (!need || m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          const float nmu_new = (m_run == kNegInf) ? 0.f : -m_run;
          const float dm = nmu_new - nmu;
          nmu = nmu_new;
#pragma unroll
          for (int r = 0; r < 16; ++r) negm[r] = nmu;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
          // this tile's scores against the new reference
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[kb][r] += dm;
          ts = weights();
          all_ref = __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0;
        }
      }
      l_run += ts;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = bf16x8{};
    }
    if constexpr (PAGED) {
      // the table entries read at the start of this phase are taken into
      // registers here: a scalar load still in flight in the next M phase
      // would make each of its LDS operand reads wait for all outstanding
      // reads (scalar loads complete out of order), serialising the phase
#pragma unroll
      for (int s = 0; s < C::CP; ++s) asm volatile("" ::"s"(ek[s]));
    }
    phase_barrier();
  };
  static_assert(kBufs == 4, "the loop below is unrolled by kBufs");
  for (int j = 0; j <= n; j += kBufs) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 > n) break;
    step(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 > n) break;
    step(j + 2, std::integral_constant<int, 2>{});
    if (j + 3 > n) break;
    step(j + 3, std::integral_constant<int, 3>{});
  }
  if (grp == 0) phase_barrier();

  // epilogue: o = O / l, lse = m*ln2 + ln(l).
  // The accumulators give each lane 4 consecutive d of one query row, so a
  // direct store instruction would write 16-byte pieces of 32 rows. Instead
  // the wave stages its 32 x D tile in LDS (free now: the last barrier came
  // after every wave's last LDS read and copy) and writes whole rows, 64 x 16
  // bytes per instruction, with a streaming (non-temporal) hint: the output
  // then does not sit dirty in the last-level cache, to be written back while
  // the next kernel on the stream reads HBM.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (pb.part_o != nullptr) {
    // a piece of the key range: the normalised fp32 partial of each row
    // (lane: 4 consecutive d per register group, d = 32 db + 8 g4 + 4 hf)
    // and its log2-sum-exp, merged later with the other pieces'
    const int qrow = wq0 + lq;
    if (qrow < pb.q_len) {
      float* dst = pb.part_o + (int64_t)qrow * pb.part_stride + 4 * hf;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *(f32x4*)(dst + 32 * db + 8 * g4) =
              f32x4{acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv, acc[db][4 * g4 + 2] * inv,
                    acc[db][4 * g4 + 3] * inv};
      if (hf == 0)
        pb.part_lse[(int64_t)qrow * pb.part_lse_stride] =
            l_tot > 0.f ? m_run + __log2f(l_tot) : kNegInf;
    }
    return;
  }
  {
    // row-major tile, 16-byte chunks XOR-swizzled by row so that the 32 rows
    // of one staging write spread over the banks
    lds_char* wtile = (lds_char*)(uintptr_t)(lds0 + (uint32_t)(wave * 32 * C::ROW));
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint32_t b0 = __builtin_bit_cast(uint16_t, (__bf16)(acc[db][4 * g4 + 0] * inv));
        const uint32_t b1 = __builtin_bit_cast(uint16_t, (__bf16)(acc[db][4 * g4 + 1] * inv));
        const uint32_t b2 = __builtin_bit_cast(uint16_t, (__bf16)(acc[db][4 * g4 + 2] * inv));
        const uint32_t b3 = __builtin_bit_cast(uint16_t, (__bf16)(acc[db][4 * g4 + 3] * inv));
        const int ch = 4 * db + g4;  // d = 8 ch + 4 hf .. +3
        lds_char* p = wtile + lq * C::ROW + ((ch ^ (lq & (C::NCH - 1))) * 16) + 8 * hf;
        *(u32x2 __attribute__((address_space(3)))*)p = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < 32 * C::NCH / 64; ++s) {
      const int idx = 64 * s + lane;
      const int r = idx / C::NCH, ch = idx % C::NCH;
      const u32x4 val = *(const u32x4 __attribute__((address_space(3)))*)(
          wtile + r * C::ROW + ((ch ^ (r & (C::NCH - 1))) * 16));
      if (wq0 + r < pb.q_len)
        __builtin_nontemporal_store(val, (u32x4*)(pb.o + (int64_t)(wq0 + r) * pb.row_stride + 8 * ch));
    }
  }
  const int qrow = wq0 + lq;
  if (qrow < pb.q_len && pb.lse != nullptr && hf == 0)
    pb.lse[(int64_t)qrow * pb.lse_stride] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : kNegInf;
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPPW * 64, 1) void prefill_pp_kernel(PrefillArgs a, float c, int n_qt) {
  __shared__ __attribute__((aligned(1024))) char lds[PP<D>::LDS];
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
  pb.m0 = qt * kPPBM;
  KvSrc<false> src;
  src.k = (const char*)((const uint16_t*)a.k + kvoff);
  src.v = (const char*)((const uint16_t*)a.v + kvoff);
  run_pp<D, false, CAUSAL>(pb, src, c, lds);
}

// Chunked prefill of a paged batch: the sequences with q_len >= 2 (their
// K/V tiles gathered through the block table), with the two-group kernel.
// Work units are (sequence, 256-row query tile, query head), or a piece of
// one's key range when long rows are split along the keys.
//
// Planned (batches of up to kPagedMaxSeqs sequences): one workgroup plans the
// call first. It lists the chunk sequences, orders them by the size of their
// largest unit (up to kSortMax of them; more keep batch order), picks the
// piece length (chunk_piece_target) and writes the list of head groups: a
// head group is (sequence, key piece, query tile, KV head), the G = Hq / Hkv
// units whose query heads read the same keys. Per sequence they are listed
// piece by piece, within a piece the last query tile (the most keys) first,
// within a tile KV head by KV head. Then one workgroup per unit, none looping
// over units: head group j runs on XCD j mod 8 (workgroups are dealt out to
// the XCDs round-robin) in slot j div 8, so each XCD takes every eighth head
// group, largest first, and its L2 serves the G query heads of each one (and
// with Hkv = 8, every query tile of a KV head). Workgroups past the list's end
// exit at once; the host sizes the grid by a bound on its length.
// Otherwise (more sequences) one workgroup per (query tile, sequence, head)
// of the host's bound, no split; workgroups of sequences with fewer rows exit
// at once.
constexpr int kSortMax = 128;      // chunk sequences ordered by unit size, at most
constexpr int kPlanThreads = 1024;

// Key tiles of query tile qt of a chunk sequence (L keys, q_len queries
// at the end, the query at position t seeing keys 0..t), as run_pp counts
// them.
__device__ __forceinline__ int chunk_item_tiles(int L, int q_len, int qt) {
  const int last_q = min((qt + 1) * kPPBM, q_len);
  return (min(L, L - q_len + last_q) + BN - 1) / BN;
}

// Key tiles per piece the call aims at: the chunk items' key tiles (over
// every query head) shared out over kPlanWGs compute units, never below
// kChunkPieceTiles. Only an item longer than that share is split, into the
// fewest pieces no longer than it: a unit that outlasts a compute unit's fair
// share sets the kernel's span, while splitting shorter ones only adds
// partial results and their merge. Computed by one wave (lanes stride the
// sequences).
__device__ int chunk_piece_target(const PagedArgs& a) {
  const int lane = threadIdx.x & 63;
  long long tot = 0;
  for (int n = lane; n < a.num_seqs; n += 64) {
    const int q_len = a.qsl[n + 1] - a.qsl[n];
    if (q_len < 2) continue;
    const int L = a.seq_lens[n];
    const int cnt = (q_len + kPPBM - 1) / kPPBM;
    for (int qt = 0; qt < cnt; ++qt) tot += chunk_item_tiles(L, q_len, qt);
  }
#pragma unroll
  for (int dd = 32; dd >= 1; dd >>= 1) tot += __shfl_xor(tot, dd);
  return (int)max((long long)kChunkPieceTiles, (tot * a.Hq + kPlanWGs - 1) / kPlanWGs);
}

// Pieces an item of `tiles` key tiles splits into at that target (1 when the
// call does not split chunk items, a.chunk_pieces == 1). The target is at
// least kChunkPieceTiles, so this stays within the chunk_pieces slots the
// workspace holds; the min only keeps it there should seq_lens exceed the
// max_seq_len the workspace was sized for. Piece k holds tiles
// k * tiles / np .. (k + 1) * tiles / np - 1.
__device__ __forceinline__ int chunk_item_pieces(const PagedArgs& a, int tiles, int target) {
  if (a.chunk_pieces <= 1) return 1;
  return min(a.chunk_pieces, max(1, (tiles - 1) / target + 1));
}

// One chunk item, or one piece of its key range. Returns false (uniformly,
// having done nothing) if the item has no such piece.
template <int D>
__device__ __forceinline__ bool run_paged_item(const PagedArgs& a, float c, char* lds, int n,
                                               int qt, int h, int t0, int q_len, int L,
                                               int piece, int target) {
  const int tiles = chunk_item_tiles(L, q_len, qt);
  const int np = chunk_item_pieces(a, tiles, target);
  if (piece >= np) return false;
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
  pb.m0 = qt * kPPBM;
  if (np > 1) {
    const int64_t slot = ((int64_t)t0 * a.Hq + h) * a.chunk_pieces + piece;
    pb.tile0 = piece * tiles / np;
    pb.tile1 = (piece + 1) * tiles / np;
    pb.part_o = a.chunk_o + slot * D;
    pb.part_lse = a.chunk_lse + slot;
    pb.part_stride = (int64_t)a.Hq * a.chunk_pieces * D;
    pb.part_lse_stride = (int64_t)a.Hq * a.chunk_pieces;
  }
  KvSrc<true> src;
  src.k = (const char*)((const uint16_t*)a.k_cache + (int64_t)g * kBlockSize * D);
  src.v = (const char*)((const uint16_t*)a.v_cache + (int64_t)g * kBlockSize * D);
  src.table = a.block_table + (int64_t)n * a.max_blocks_per_seq;
  src.block_bytes = (int64_t)a.Hkv * kBlockSize * D * 2;
  run_pp<D, true, true>(pb, src, c, lds);
  return true;
}

template <int D>
__global__ __launch_bounds__(kPPW * 64, 1) void prefill_pp_paged_kernel(PagedArgs a, float c,
                                                                         int n_qt) {
  __shared__ __attribute__((aligned(1024))) char lds[PP<D>::LDS];
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  int unit, qt;
  logical_to_work(logical, a.num_seqs * a.Hq, n_qt, unit, qt);
  const int n = unit / a.Hq, h = unit % a.Hq;
  const int t0 = a.qsl[n];
  const int q_len = a.qsl[n + 1] - t0;
  if (q_len < 2 || qt * kPPBM >= q_len) return;  // uniform over the workgroup
  run_paged_item<D>(a, c, lds, n, qt, h, t0, q_len, a.seq_lens[n], 0, 0x7fffffff);
}

// The plan: a.chunk_plan[0] = head groups listed, [1] = piece target, then
// from int 4 on one int4 {sequence, piece, query tile, KV head} per head group
// (at most a.plan_cap of them).
__global__ __launch_bounds__(kPlanThreads) void chunk_plan_kernel(PagedArgs a) {
  __shared__ int ids[kPagedMaxSeqs];       // chunk sequences, batch order
  __shared__ int key[kPagedMaxSeqs];       // their sort keys
  __shared__ int seq_of[kPagedMaxSeqs];    // r-th chunk sequence of the plan
  __shared__ int first_of[kPagedMaxSeqs];  // its first head group
  __shared__ int s_m, s_target, s_total;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // wave 0: the piece target, and the sequences with q_len >= 2 compacted
    // in batch order
    const int target = a.chunk_pieces > 1 ? chunk_piece_target(a) : 0x7fffffff;
    const int lane = tid;
    int m = 0;
    for (int n0 = 0; n0 < a.num_seqs; n0 += 64) {
      const int n = n0 + lane;
      const bool chunk = n < a.num_seqs && a.qsl[n + 1] - a.qsl[n] >= 2;
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(chunk);
      if (chunk) ids[m + (int)__builtin_popcountll(bal & ((1ull << lane) - 1))] = n;
      m += (int)__builtin_popcountll(bal);
    }
    if (lane == 0) {
      s_m = m;
      s_target = target;
    }
  }
  __syncthreads();
  const int m = s_m, target = s_target;
  // sort key: the key tiles of the sequence's largest unit (a piece of its
  // last query tile)
  for (int i = tid; i < m; i += kPlanThreads) {
    const int n = ids[i];
    const int q_len = a.qsl[n + 1] - a.qsl[n];
    const int tl = chunk_item_tiles(a.seq_lens[n], q_len, (q_len + kPPBM - 1) / kPPBM - 1);
    const int np = chunk_item_pieces(a, tl, target);
    key[i] = (tl + np - 1) / np;
  }
  __syncthreads();
  for (int i = tid; i < m; i += kPlanThreads) {
    if (m <= kSortMax) {
      // rank by counting, largest first; ties keep batch order
      const int ki = key[i];
      int rank = 0;
      for (int j = 0; j < m; ++j) {
        const int kj = key[j];
        rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
      }
      seq_of[rank] = ids[i];
    } else {
      seq_of[i] = ids[i];
    }
  }
  __syncthreads();
  if (tid < 64) {
    // wave 0: first head group of each sequence, by a running sum over
    // Hkv * (pieces summed over its query tiles)
    const int lane = tid;
    int base = 0;
    for (int r0 = 0; r0 < m; r0 += 64) {
      const int r = r0 + lane;
      int cnt = 0;
      if (r < m) {
        const int n = seq_of[r];
        const int q_len = a.qsl[n + 1] - a.qsl[n];
        const int L = a.seq_lens[n];
        const int tiles = (q_len + kPPBM - 1) / kPPBM;
        for (int qt = 0; qt < tiles; ++qt)
          cnt += a.Hkv * chunk_item_pieces(a, chunk_item_tiles(L, q_len, qt), target);
      }
      int incl = cnt;
#pragma unroll
      for (int dd = 1; dd < 64; dd <<= 1) {
        const int up = __shfl_up(incl, dd);
        incl += lane >= dd ? up : 0;
      }
      if (r < m) first_of[r] = base + incl - cnt;
      base += __shfl(incl, 63);
    }
    // the host's bound holds the list of any batch within the documented
    // preconditions; the min only keeps a batch outside them (query_start_loc
    // past num_tokens, q_len past max_query_len) inside the workspace
    if (lane == 0) s_total = min(base, a.plan_cap);
  }
  __syncthreads();
  const int total = s_total;
  int4* list = reinterpret_cast<int4*>(a.chunk_plan + 4);
  for (int j = tid; j < total; j += kPlanThreads) {
    // the sequence holding head group j: the largest r with first_of[r] <= j
    int lo = 0, hi = m - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first_of[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int n = seq_of[lo];
    int local = j - first_of[lo];
    const int q_len = a.qsl[n + 1] - a.qsl[n];
    const int L = a.seq_lens[n];
    const int cnt = (q_len + kPPBM - 1) / kPPBM;
    // its piece: a later query tile has at least as many keys, hence pieces,
    // so the tiles that have piece p are the last cnt - t_lo of them
    int p = 0, t_lo = 0;
    for (;; ++p) {
      while (t_lo < cnt && chunk_item_pieces(a, chunk_item_tiles(L, q_len, t_lo), target) <= p)
        ++t_lo;
      const int here = a.Hkv * (cnt - t_lo);
      if (local < here) break;
      local -= here;
    }
    list[j] = int4{n, p, cnt - 1 - local / a.Hkv, local % a.Hkv};
  }
  if (tid == 0) {
    a.chunk_plan[0] = total;
    a.chunk_plan[1] = target;
  }
}

// One unit of the plan per workgroup: head group j = 8 (s div G) + x, query
// head g * G + s mod G of it, for workgroup 8 s + x (on XCD x).
template <int D>
__global__ __launch_bounds__(kPPW * 64, 1) void prefill_pp_planned_kernel(PagedArgs a, float c) {
  __shared__ __attribute__((aligned(1024))) char lds[PP<D>::LDS];
  const int G = a.Hq / a.Hkv;
  const int x = blockIdx.x & 7, s = blockIdx.x >> 3;
  const int j = (s / G) * 8 + x;
  if (j >= __builtin_amdgcn_readfirstlane(a.chunk_plan[0])) return;
  const int4 e = reinterpret_cast<const int4*>(a.chunk_plan + 4)[j];
  const int n = __builtin_amdgcn_readfirstlane(e.x);
  const int piece = __builtin_amdgcn_readfirstlane(e.y);
  const int qt = __builtin_amdgcn_readfirstlane(e.z);
  const int h = __builtin_amdgcn_readfirstlane(e.w) * G + s % G;
  const int target = __builtin_amdgcn_readfirstlane(a.chunk_plan[1]);
  const int t0 = __builtin_amdgcn_readfirstlane(a.qsl[n]);
  const int q_len = __builtin_amdgcn_readfirstlane(a.qsl[n + 1]) - t0;
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[n]);
  run_paged_item<D>(a, c, lds, n, qt, h, t0, q_len, L, piece, target);
}

// Merge of the key-range pieces of the split chunk rows: per row and query
// head, o = sum_k 2^(lse_k - M) o_k / sum_k 2^(lse_k - M), M = max_k lse_k,
// lse = M + log2 of that sum (in natural-log units on output). One workgroup
// per query head of each head group of piece 0 in the plan (so per (sequence,
// query tile, query head)), one thread per 4 consecutive d of a row;
// workgroups of other pieces, past the list or of unsplit tiles exit at once.
constexpr int kMergeThreads = 1024;
constexpr int kMergeBatch = 8;  // pieces whose loads are in flight together

template <int D>
__global__ __launch_bounds__(kMergeThreads) void chunk_merge_kernel(PagedArgs a) {
  const int G = a.Hq / a.Hkv;
  const int j = blockIdx.x / G;
  if (j >= a.chunk_plan[0]) return;
  const int4 e = reinterpret_cast<const int4*>(a.chunk_plan + 4)[j];
  if (e.y != 0) return;
  const int n = e.x, qt = e.z, h = e.w * G + blockIdx.x % G;
  const int t0 = a.qsl[n];
  const int q_len = a.qsl[n + 1] - t0;
  const int L = a.seq_lens[n];
  const int np = chunk_item_pieces(a, chunk_item_tiles(L, q_len, qt), a.chunk_plan[1]);
  if (np <= 1) return;
  constexpr int Q4 = D / 4;
  const int P = a.chunk_pieces;
  const int rows = min(kPPBM, q_len - qt * kPPBM);
  for (int e = threadIdx.x; e < rows * Q4; e += kMergeThreads) {
    const int t = t0 + qt * kPPBM + e / Q4, d0 = 4 * (e % Q4);
    const int64_t slot = ((int64_t)t * a.Hq + h) * P;
    // every piece's lse and partial output, kMergeBatch pieces in flight at
    // once; the running max rescales the sums when it grows
    float M = kNegInf, W = 0.f;
    f32x4 acc = f32x4{};
    for (int k0 = 0; k0 < np; k0 += kMergeBatch) {
      float lk[kMergeBatch];
      f32x4 ok[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        lk[i] = k0 + i < np ? a.chunk_lse[slot + k0 + i] : kNegInf;
        ok[i] = k0 + i < np ? *(const f32x4*)(a.chunk_o + (slot + k0 + i) * D + d0) : f32x4{};
      }
      float Mb = M;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) Mb = fmaxf(Mb, lk[i]);
      if (Mb != kNegInf) {
        const float r = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
        W *= r;
        acc *= r;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
          const float w = lk[i] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(lk[i] - Mb);
          W += w;
          acc += w * ok[i];
        }
        M = Mb;
      }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    uint16_t* dst = (uint16_t*)a.o + ((int64_t)t * a.Hq + h) * D + d0;
    *(u32x2*)dst = u32x2{(uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[0] * inv)) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[1] * inv)) << 16),
                         (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[2] * inv)) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(acc[3] * inv)) << 16)};
    if (a.lse != nullptr && d0 == 0)
      a.lse[(int64_t)t * a.Hq + h] = W > 0.f ? (M + __log2f(W)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const int n_qt = (a.T + kPPBM - 1) / kPPBM;
  const dim3 grid((unsigned)(n_qt * a.B * a.Hq));
  const dim3 block(kPPW * 64);
  if (a.d == 128) {
    if (a.causal)
      hipLaunchKernelGGL((prefill_pp_kernel<128, true>), grid, block, 0, s, a, c, n_qt);
    else
      hipLaunchKernelGGL((prefill_pp_kernel<128, false>), grid, block, 0, s, a, c, n_qt);
  } else {
    if (a.causal)
      hipLaunchKernelGGL((prefill_pp_kernel<64, true>), grid, block, 0, s, a, c, n_qt);
    else
      hipLaunchKernelGGL((prefill_pp_kernel<64, false>), grid, block, 0, s, a, c, n_qt);
  }
  return hipGetLastError();
}

hipError_t launch_paged_prefill_bf16(const PagedArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const dim3 block(kPPW * 64);
  if (a.chunk_plan != nullptr) {
    hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // head groups j < plan_cap, each G workgroups, dealt 8 at a time
    const int G = a.Hq / a.Hkv;
    const dim3 grid((unsigned)(((int64_t)a.plan_cap + 7) / 8 * 8 * G));
    if (a.d == 128)
      hipLaunchKernelGGL((prefill_pp_planned_kernel<128>), grid, block, 0, s, a, c);
    else
      hipLaunchKernelGGL((prefill_pp_planned_kernel<64>), grid, block, 0, s, a, c);
    if (a.chunk_pieces > 1) {
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      const dim3 mgrid((unsigned)((int64_t)a.plan_cap * G));
      if (a.d == 128)
        hipLaunchKernelGGL((chunk_merge_kernel<128>), mgrid, dim3(kMergeThreads), 0, s, a);
      else
        hipLaunchKernelGGL((chunk_merge_kernel<64>), mgrid, dim3(kMergeThreads), 0, s, a);
    }
  } else {
    const int n_qt = (a.max_query_len + kPPBM - 1) / kPPBM;
    const dim3 grid((unsigned)((int64_t)n_qt * a.num_seqs * a.Hq));
    if (a.d == 128)
      hipLaunchKernelGGL((prefill_pp_paged_kernel<128>), grid, block, 0, s, a, c, n_qt);
    else
      hipLaunchKernelGGL((prefill_pp_paged_kernel<64>), grid, block, 0, s, a, c, n_qt);
  }
  return hipGetLastError();
}

}  // namespace attn
