// Measurement probe for the benchmark (libattn_probe.so, loaded by bench.py
// only; not part of the attention library): the shader clock the chip holds
// under dense bf16 MFMA load, and the MFMA rate a pure MFMA loop reaches at
// that clock. Every SIMD of every CU runs one wave that issues `iters`
// rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains, reading
// s_memtime (shader clock) and s_memrealtime (constant-rate clock) around
// the loop.

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_clock_kernel(unsigned long long* out, int iters,
                                                        float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (lane + e));
    b[e] = (__bf16)(seed * (lane - e));
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float keep = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) keep += acc[i][lane & 15];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (lane == 0) {
    out[3 * wave + 0] = t1 - t0;
    out[3 * wave + 1] = r1 - r0;
    out[3 * wave + 2] = keep == 12345.f ? 1 : 0;  // keeps the chains alive
  }
}

}  // namespace

// out: device memory for 3 * waves unsigned 64-bit values, waves = blocks * 4
// (one wave per SIMD: 256 threads per block, one block per CU).
extern "C" int attn_probe_mfma_clock(unsigned long long* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_clock_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters, 0.001f);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
