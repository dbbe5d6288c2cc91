// Tiled causal attention prefill in fp32 (fp32 in, fp32 arithmetic, fp32 out).
//
// Same method as the bf16 kernel ("Fast attention kernels and operator
// fusion", the-ai.news, section "FlashAttention-style attention and paged
// attention", first paragraph): key/value blocks are staged on chip, the
// scores of a block are formed, the running softmax statistics updated and
// the output accumulated in registers; the T x T score matrix is never
// stored. This path serves fp32 inputs, where the pages' advice is to check
// results with a tolerance fitted to the type ("Fast attention kernels and
// operator fusion", section "Fusion and CUDA Graphs with torch.compile").
//
// Layout: a workgroup of 256 threads owns 64 query rows of one (b, h); four
// consecutive lanes share a query row, each holding a quarter of the head
// dimension of q and of the output accumulator. Scores are quarter dot
// products reduced across the four lanes. Key/value tiles of 32 rows sit in
// LDS in fp32; every lane of a wave reads the same LDS words (broadcast).
// The softmax recurrence is the exact running max / running sum (rescale at
// every tile), in log2 units with exp2.

#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKeys = 32;   // keys per tile
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillArgs a, float c) {
  constexpr int DQ = D / 4;  // dims per lane
  __shared__ float4 sk[kKeys * D / 4];
  __shared__ float4 sv[kKeys * D / 4];

  const int tid = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.Hq / a.Hkv);
  const int T = a.T;
  const int row = qt * kRows + tid / 4;  // this lane's query
  const int part = tid & 3;
  const float* q = (const float*)a.q + ((int64_t)b * a.Hq + h) * T * D;
  const float* k = (const float*)a.k + ((int64_t)b * a.Hkv + g) * T * D;
  const float* v = (const float*)a.v + ((int64_t)b * a.Hkv + g) * T * D;
  float* o = (float*)a.o + ((int64_t)b * a.Hq + h) * T * D;

  float qr[DQ], acc[DQ];
#pragma unroll
  for (int i = 0; i < DQ; i += 4) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < T) x = *(const float4*)(q + (int64_t)row * D + part * DQ + i);
    qr[i] = x.x; qr[i + 1] = x.y; qr[i + 2] = x.z; qr[i + 3] = x.w;
    acc[i] = acc[i + 1] = acc[i + 2] = acc[i + 3] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f;

  const int last_q = min(T, (qt + 1) * kRows);  // exclusive
  const int n_keys = CAUSAL ? last_q : T;
  for (int n0 = 0; n0 < n_keys; n0 += kKeys) {
    __syncthreads();
    for (int i = tid; i < kKeys * D / 4; i += kThreads) {
      const int r = i / (D / 4), cc = i % (D / 4);
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (n0 + r < T) {
        kx = *(const float4*)(k + (int64_t)(n0 + r) * D + cc * 4);
        vx = *(const float4*)(v + (int64_t)(n0 + r) * D + cc * 4);
      }
      sk[i] = kx;
      sv[i] = vx;
    }
    __syncthreads();

    float s[kKeys];
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float part_dot = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const float4 kx = sk[j * (D / 4) + (part * DQ + i) / 4];
        part_dot = __builtin_fmaf(qr[i], kx.x, part_dot);
        part_dot = __builtin_fmaf(qr[i + 1], kx.y, part_dot);
        part_dot = __builtin_fmaf(qr[i + 2], kx.z, part_dot);
        part_dot = __builtin_fmaf(qr[i + 3], kx.w, part_dot);
      }
      part_dot += __shfl_xor(part_dot, 1);
      part_dot += __shfl_xor(part_dot, 2);
      const int key = n0 + j;
      const bool dead = (CAUSAL && key > row) || key >= T;
      s[j] = dead ? kNegInf : part_dot * c;
    }
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) mt = fmaxf(mt, s[j]);
    const float m_new = fmaxf(m_run, mt);
    const float mu = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - mu);  // m_run = -inf -> 0
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < DQ; ++i) acc[i] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = exp2f(s[j] - mu);
      l_run += p;
#pragma unroll
      for (int i = 0; i < DQ; i += 4) {
        const float4 vx = sv[j * (D / 4) + (part * DQ + i) / 4];
        acc[i] = __builtin_fmaf(p, vx.x, acc[i]);
        acc[i + 1] = __builtin_fmaf(p, vx.y, acc[i + 1]);
        acc[i + 2] = __builtin_fmaf(p, vx.z, acc[i + 2]);
        acc[i + 3] = __builtin_fmaf(p, vx.w, acc[i + 3]);
      }
    }
  }

  if (row < T) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int i = 0; i < DQ; i += 4)
      *(float4*)(o + (int64_t)row * D + part * DQ + i) =
          make_float4(acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv);
    if (a.lse != nullptr && part == 0)
      a.lse[((int64_t)b * a.Hq + h) * T + row] = l_run > 0.f ? m_run * kLn2 + logf(l_run) : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2e;
  const dim3 grid((unsigned)((a.T + kRows - 1) / kRows), (unsigned)a.Hq, (unsigned)a.B);
  const dim3 block(kThreads);
  if (a.d == 128) {
    if (a.causal) hipLaunchKernelGGL((prefill_f32_kernel<128, true>), grid, block, 0, s, a, c);
    else hipLaunchKernelGGL((prefill_f32_kernel<128, false>), grid, block, 0, s, a, c);
  } else {
    if (a.causal) hipLaunchKernelGGL((prefill_f32_kernel<64, true>), grid, block, 0, s, a, c);
    else hipLaunchKernelGGL((prefill_f32_kernel<64, false>), grid, block, 0, s, a, c);
  }
  return hipGetLastError();
}

}  // namespace attn
