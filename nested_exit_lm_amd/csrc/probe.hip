// A register-only loop of bf16 MFMAs on caller-supplied operand data: a
// measurement aid, not a step of the method.  Every wavefront loads kSets
// operand pairs into registers once, then cycles through them (consecutive
// MFMAs see different data, as in a GEMM) into four independent accumulator
// chains, with no memory traffic.
//
// Its rate is no ceiling for the head GEMM: launched from this library it
// reads about 1290 TF/s on random operands, while the same instruction loop
// built as a standalone program sustains 1800-1960 TF/s on the same machine
// and data; the cause of the difference was not found.
#include "common.h"
#include "internal.h"

namespace nel {

namespace {

constexpr int kSets = 8;

__global__ __launch_bounds__(256) void mfma_rate_kernel(const u32x4* __restrict__ ops, int iters,
                                                        float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
    const u32x4 ra = ops[(2 * s) * 64 + lane];
    const u32x4 rb = ops[(2 * s + 1) * 64 + lane];
    a[s] = __builtin_bit_cast(bf16x8, ra);
    b[s] = __builtin_bit_cast(bf16x8, rb);
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
      acc[s & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc[s & 3], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[k][r];
  t = wave_sum(t);
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = t;
}

}  // namespace

hipError_t launch_mfma_rate(const void* operands, int iters, int blocks, float* sink,
                            hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const u32x4*>(operands), iters, sink);
  return hipGetLastError();
}

}  // namespace nel
