// Internal helpers shared by the gfx950 kernels: element types, 16-byte
// vectors, bf16 <-> fp32, base-2 exp/log, wavefront (64-lane) reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nel {

constexpr float kLog2e = 1.4426950408889634f;   // log2(e)
constexpr float kLn2 = 0.6931471805599453f;     // ln(2)
constexpr int kWave = 64;

typedef uint16_t bf16_t;   // bfloat16 storage
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 r = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, r);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// e^x and ln(x) through the base-2 hardware transcendentals.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float flog(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Element-type traits: 16-byte chunks hold kChunk elements.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kChunk = 8;
  __device__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static constexpr int kChunk = 4;
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};

// Online (max, sum of exp) merge: (m, s) <- (m, s) (+) (m2, s2).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * fexp(m - m2) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s += s2 * fexp(m2 - m);
  }
}

}  // namespace nel
