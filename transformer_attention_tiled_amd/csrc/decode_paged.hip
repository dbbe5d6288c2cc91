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
// Split-KV: one workgroup per (KV partition p, KV head g, sequence n); all
// G = Hq/Hkv query heads of the group share each K/V block read. The four
// waves of the workgroup take every fourth 16-token block of the partition,
// each keeping its own running max / sum / accumulator; they are combined in
// LDS and the workgroup writes one normalised fp32 partial o_p and its
// log2-sum-exp. A second kernel merges the partials of each (sequence, head):
//   lse = log2 sum_p 2^(lse_p),  o = sum_p 2^(lse_p - lse) o_p.
// This merge identity is exact; only rounding differs from the unsplit sum.
//
// Per 16-token block a wave uses MFMA for both products (the contraction is
// tiny but MFMA keeps the VALU free for the softmax):
//   S = K Q^T      v_mfma_f32_16x16x32_bf16: A = K block (token = l%16,
//                  8 consecutive d), B = Q^T (head = l%16), C = S[token][head]
//                  with lane l holding tokens 4*(l/16)+r, head l%16.
//   O += P V       v_mfma_f32_16x16x16bf16_1k: A = P[head][token], which is the
//                  S accumulator of the lane as is; B = V[token][d] for the
//                  tokens 4*(l/16)+e: lane l loads rows 4*(l/16)..+3 at the
//                  d-chunk DPL*(l%16)..+DPL-1 and MFMA number m takes element m
//                  of each row, so its output column j is d = DPL*j + m.
// Positions >= L are never loaded (their storage may hold anything) and
// their scores are selected to -inf.

#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct BlockRegs {
  uint4 k[D / 32];  // K[token l%16][d = (D/4)*(l/16) + 8*s .. +7]
  uint4 v[4];       // V[token 4*(l/16)+i][d = (D/16)*(l%16) ..], D/16 elements used
};

template <int D>
__device__ __forceinline__ void load_block(BlockRegs<D>& br, const uint16_t* kblk,
                                           const uint16_t* vblk, int valid, int lane) {
  constexpr int DL = D / 4;   // d-range per lane group for K
  constexpr int DPL = D / 16; // d-range per lane for V
  const int tk = lane & 15;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (tk < valid) x = *(const uint4*)(kblk + tk * D + DL * (lane >> 4) + 8 * s);
    br.k[s] = x;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tv = 4 * (lane >> 4) + i;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (tv < valid) {
      if constexpr (DPL == 8) {
        x = *(const uint4*)(vblk + tv * D + DPL * (lane & 15));
      } else {
        const uint2 y = *(const uint2*)(vblk + tv * D + DPL * (lane & 15));
        x = make_uint4(y.x, y.y, 0, 0);
      }
    }
    br.v[i] = x;
  }
}

__device__ __forceinline__ uint32_t elem16(const uint4& x, int m) {
  const uint32_t w = (m >> 1) == 0 ? x.x : (m >> 1) == 1 ? x.y : (m >> 1) == 2 ? x.z : x.w;
  return (m & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(PagedArgs a, float c) {
  constexpr int DPL = D / 16;
  __shared__ float sm_o[kWaves][16][D];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];

  const int p = blockIdx.x % a.max_parts;
  const int g = (blockIdx.x / a.max_parts) % a.Hkv;
  const int n = blockIdx.x / a.max_parts / a.Hkv;
  int t0 = n;
  if (a.qsl != nullptr) {
    t0 = a.qsl[n];
    if (a.qsl[n + 1] - t0 != 1) return;
  }
  const int L = a.seq_lens[n];
  const int P = a.partition_size;
  const int start = p * P;
  if (start >= L) return;
  const int end = min(L, start + P);
  const int nblk = (end - start + 15) >> 4;
  const int first = start >> 4;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.Hq / a.Hkv;
  const int head = lane & 15;  // query head (column) owned in S
  const int grp = lane >> 4;

  // Q^T fragments (B operand of S = K Q^T)
  bf16x8 qf[D / 32];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)t0 * a.Hq + g * G + head) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (head < G) x = *(const uint4*)(qrow + (D / 4) * grp + 8 * s);
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x4 acc[DPL];
#pragma unroll
  for (int m = 0; m < DPL; ++m) acc[m] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;

  const int32_t* table = a.block_table + (int64_t)n * a.max_blocks_per_seq;
  const int64_t bstride = (int64_t)a.Hkv * kBlockSize * D;
  const uint16_t* kbase = (const uint16_t*)a.k_cache + (int64_t)g * kBlockSize * D;
  const uint16_t* vbase = (const uint16_t*)a.v_cache + (int64_t)g * kBlockSize * D;

  BlockRegs<D> cur, nxt;
  int b = wave;
  if (b < nblk) {
    const int64_t phys = table[first + b];
    load_block<D>(cur, kbase + phys * bstride, vbase + phys * bstride,
                  end - (start + 16 * b), lane);
  }
  for (; b < nblk; b += kWaves) {
    const int bn = b + kWaves;
    if (bn < nblk) {
      const int64_t phys = table[first + bn];
      load_block<D>(nxt, kbase + phys * bstride, vbase + phys * bstride,
                    end - (start + 16 * bn), lane);
    }
    // S = K Q^T
    f32x4 s = f32x4{};
#pragma unroll
    for (int st = 0; st < D / 32; ++st)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[st]), qf[st], s,
                                                  0, 0, 0);
    const int valid = end - (start + 16 * b);
    if (valid < 16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = (4 * grp + r < valid) ? s[r] : kNegInf;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * c;
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
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mu));
      l_run += pr;
      pa[r] = (__bf16)pr;
    }
    // O += P V
#pragma unroll
    for (int m = 0; m < DPL; ++m) {
      const uint32_t lo = elem16(cur.v[0], m) | (elem16(cur.v[1], m) << 16);
      const uint32_t hi = elem16(cur.v[2], m) | (elem16(cur.v[3], m) << 16);
      const bf16x4 vb = __builtin_bit_cast(bf16x4, make_uint2(lo, hi));
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[m], 0, 0, 0);
    }
    cur = nxt;
  }

  // combine the four lane groups' row sums (same head, different tokens)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lane < 16) {
    sm_m[wave][lane] = m_run;
    sm_l[wave][lane] = l_run;
  }
#pragma unroll
  for (int m = 0; m < DPL; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wave][4 * grp + r][DPL * head + m] = acc[m][r];
  __syncthreads();

  // combine the waves and write the partition's partial
  for (int i = tid; i < G * D; i += kWaves * 64) {
    const int hh = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][hh]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (sm_m[w][hh] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(sm_m[w][hh] - M);
      lsum += f * sm_l[w][hh];
      osum += f * sm_o[w][hh][d];
    }
    const int64_t row = ((int64_t)n * a.Hq + g * G + hh) * a.max_parts + p;
    a.ws_o[row * D + d] = lsum > 0.f ? osum / lsum : 0.f;
    if (d == 0) a.ws_lse[row] = lsum > 0.f ? M + __log2f(lsum) : kNegInf;
  }
}

// Merge of the split-KV partials of one (sequence, query head).
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(PagedArgs a) {
  const int h = blockIdx.x % a.Hq, n = blockIdx.x / a.Hq, d = threadIdx.x;
  int t0 = n;
  if (a.qsl != nullptr) {
    t0 = a.qsl[n];
    if (a.qsl[n + 1] - t0 != 1) return;
  }
  const int L = a.seq_lens[n];
  const int np = (L + a.partition_size - 1) / a.partition_size;
  const int64_t row0 = ((int64_t)n * a.Hq + h) * a.max_parts;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, a.ws_lse[row0 + p]);
  float wsum = 0.f, osum = 0.f;
  for (int p = 0; p < np; ++p) {
    const float lp = a.ws_lse[row0 + p];
    const float w = (lp == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(lp - M);
    wsum += w;
    osum += w * a.ws_o[(row0 + p) * D + d];
  }
  const float out = wsum > 0.f ? osum / wsum : 0.f;
  uint16_t* o = (uint16_t*)a.o + ((int64_t)t0 * a.Hq + h) * D;
  o[d] = __builtin_bit_cast(uint16_t, (__bf16)out);
  if (a.lse != nullptr && d == 0)
    a.lse[(int64_t)t0 * a.Hq + h] = wsum > 0.f ? (M + __log2f(wsum)) * kLn2 : kNegInf;
}

}  // namespace

int decode_partition_size(int num_seqs, int Hkv, int max_seq_len) {
  if (num_seqs < 1 || Hkv < 1 || max_seq_len < 1) return 0;
  // Aim for about 8192 work items over the whole batch, never partitions
  // shorter than 256 tokens; round the length up to whole 16-token blocks.
  const int64_t units = (int64_t)num_seqs * Hkv;
  const int64_t max_parts_cap = (max_seq_len + 255) / 256;
  int64_t parts = (8192 + units - 1) / units;
  if (parts > max_parts_cap) parts = max_parts_cap;
  if (parts < 1) parts = 1;
  int64_t P = (max_seq_len + parts - 1) / parts;
  P = (P + 15) / 16 * 16;
  return (int)P;
}

hipError_t launch_paged_decode_bf16(const PagedArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const dim3 grid((unsigned)((int64_t)a.max_parts * a.Hkv * a.num_seqs));
  if (a.d == 128) {
    hipLaunchKernelGGL((decode_split_kernel<128>), grid, dim3(kWaves * 64), 0, s, a, c);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<64>), grid, dim3(kWaves * 64), 0, s, a, c);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)((int64_t)a.Hq * a.num_seqs));
  if (a.d == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), mgrid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<64>), mgrid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
