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
// Two at once: one v_cvt_pk_bf16_f32, the same rounding as f32_to_bf16.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// fp16 <-> fp32 (round to nearest even).  The loss path keeps its 16-bit
// scratch (tile-shifted logits l - m <= 0, teacher weights in [0, 1]) in fp16:
// relative rounding 2^-11, three bits more than bf16, and the range of
// l - m (down to -65504) is far beyond where exp(l - m) vanishes.
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const half2_t h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

// e^x and ln(x) through the base-2 hardware transcendentals.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float flog(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// Makes this wavefront's LDS stores visible to its own later LDS loads of
// other lanes' slots.  The wave barrier alone is treated by the compiler as
// touching no memory, so it could forward a lane's own stored value to a load
// of another lane's slot; wavefront-scope release/acquire fences around it
// forbid that reordering.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reductions over the lane pairs l, l ^ 16 and l, l ^ 32 on the gfx950 lane
// swaps (no LDS round trip): a swap of a value with itself hands each lane of
// one half its partner's value in one output and leaves the other output as
// it was, so combining the two outputs covers both orders of the swap.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Codec of the loss path's per-entry scratch for element type T: fp16 bits
// for bf16 inputs (see above), the fp32 value itself for fp32 inputs.  A
// 16-byte chunk holds Elem<T>::kChunk entries either way.
template <typename T> struct Scratch;
template <> struct Scratch<bf16_t> {
  __device__ static float get(const u32x4& r, int i) {
    const uint32_t w = r[i >> 1];   // (a vector element through a scalar first)
    return f16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
  }
  __device__ static float load(const bf16_t* p) { return f16_bits_to_f32(*p); }
  __device__ static bf16_t encode(float v) { return f32_to_f16_bits(v); }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
};
template <> struct Scratch<float> {
  __device__ static float get(const u32x4& r, int i) { return __uint_as_float(r[i]); }
  __device__ static float load(const float* p) { return *p; }
  __device__ static float encode(float v) { return v; }
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
