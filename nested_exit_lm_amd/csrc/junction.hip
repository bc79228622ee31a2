// Junction between block m and block m+1 (one wavefront, or a lane group of
// one, per token).
//
// The paper's Eq. 1 as the pages state it in prose ("Matryoshka Language
// Model Suites", junction paragraph; key-visual explainer, bottom panel):
// block m's output for a token is rescaled to the L2 norm of the fresh
// residual embedding e_{m+1}[x_t] and concatenated with it along channels.
// Block 1 reads e_1[x_t] alone (copyedit of Sec. 2, D_0 = 0).
//
// Modes (the 200M ablations of the same passages): kJunctionNoRescale passes
// h through unscaled; kJunctionZeroFill writes zeros in place of the
// embedding while the rescale target stays ||e_{m+1}[x_t]||.
//
// HBM-bound: each token reads d_in + (d_out - d_in) elements and writes d_out.
// Every lane moves 16-byte chunks; the token's chunks stay in registers
// between the norm pass and the write pass, so h and the embedding row are
// read from memory once.
#include "common.h"
#include "internal.h"

namespace nel {

namespace {

constexpr int kTokPerBlock = 4;     // 4 wavefronts per 256-thread block
constexpr int kMaxChunks = 10;      // register cache per lane: up to 640 chunks per row

template <typename T>
__device__ __forceinline__ float chunk_sumsq(const u32x4& c) {
  float s = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lo = __uint_as_float(c[j] << 16), hi = __uint_as_float(c[j] & 0xffff0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = __uint_as_float(c[j]);
      s = fmaf(v, v, s);
    }
  }
  return s;
}

template <typename T>
__device__ __forceinline__ u32x4 chunk_scale(const u32x4& c, float k) {
  u32x4 r;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float lo = __uint_as_float(c[j] << 16), hi = __uint_as_float(c[j] & 0xffff0000u);
      r[j] = pack_bf16x2(lo * k, hi * k);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __float_as_uint(__uint_as_float(c[j]) * k);
  }
  return r;
}

__device__ __forceinline__ float norm_ratio(float sh, float se) {
  // ||e|| / ||h||, and 0 when either norm is 0 (no epsilon).
  return (sh > 0.f && se > 0.f) ? sqrtf(se) / sqrtf(sh) : 0.f;
}

// 16-byte chunk path: d_in and d_out - d_in are multiples of the chunk and
// every row fits the register cache.  G lanes serve one token (G = 64: one
// token per wavefront; narrower rows put 64 / G tokens in a wavefront), chosen
// so that each lane keeps several chunks in flight; the norms are reduced
// within the G lanes of a token.
template <typename T, int G>
__global__ __launch_bounds__(256) void junction_vec(int64_t n, int d_in, int d_out, int vocab,
                                                    const T* __restrict__ h,
                                                    const int32_t* __restrict__ ids,
                                                    const T* __restrict__ emb, T* __restrict__ out,
                                                    int32_t* __restrict__ flags, int mode) {
  constexpr int C = Elem<T>::kChunk;
  constexpr int TPW = 64 / G;   // tokens per wavefront
  const int lane = threadIdx.x & 63, sub = lane % G;
  const int64_t t = (static_cast<int64_t>(blockIdx.x) * kTokPerBlock + (threadIdx.x >> 6)) * TPW +
                    lane / G;
  if (t >= n) return;   // a token's G lanes leave together; the reductions stay inside them
  const int de = d_out - d_in;
  const int nh = d_in / C, ne = de / C;
  const int id = ids[t];
  u32x4* orow = reinterpret_cast<u32x4*>(out + t * d_out);
  if (id < 0 || id >= vocab) {
    if (sub == 0 && flags) atomicOr(flags, 1 /*NEL_FLAG_BAD_ID*/);
    const u32x4 nanv = {0x7fc00000u, 0x7fc00000u, 0x7fc00000u, 0x7fc00000u};
    const u32x4 nanb = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
    for (int c = sub; c < nh + ne; c += G) orow[c] = sizeof(T) == 2 ? nanb : nanv;
    return;
  }
  const u32x4* hrow = reinterpret_cast<const u32x4*>(h + t * d_in);
  const u32x4* erow = reinterpret_cast<const u32x4*>(emb + static_cast<int64_t>(id) * de);
  u32x4 hc[kMaxChunks], ec[kMaxChunks];
  float sh = 0.f, se = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = sub + G * j;
    if (c < nh) hc[j] = __builtin_nontemporal_load(hrow + c);
    if (c < ne) ec[j] = erow[c];
  }
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = sub + G * j;
    if (c < nh) sh += chunk_sumsq<T>(hc[j]);
    if (c < ne) se += chunk_sumsq<T>(ec[j]);
  }
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) {
    sh += __shfl_xor(sh, o, kWave);
    se += __shfl_xor(se, o, kWave);
  }
  const float k = mode == kJunctionNoRescale ? 1.f : norm_ratio(sh, se);
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = sub + G * j;
    if (c < nh) __builtin_nontemporal_store(chunk_scale<T>(hc[j], k), orow + c);
    if (c < ne) __builtin_nontemporal_store(mode == kJunctionZeroFill ? zero : ec[j], orow + nh + c);
  }
}

// Element path for any widths (rows not a multiple of 16 bytes, or rows
// longer than the register cache): two passes over the row.
template <typename T>
__global__ __launch_bounds__(256) void junction_elem(int64_t n, int d_in, int d_out, int vocab,
                                                     const T* __restrict__ h,
                                                     const int32_t* __restrict__ ids,
                                                     const T* __restrict__ emb, T* __restrict__ out,
                                                     int32_t* __restrict__ flags, int mode) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= n) return;
  const int de = d_out - d_in;
  const int id = ids[t];
  T* orow = out + t * d_out;
  if (id < 0 || id >= vocab) {
    if (lane == 0 && flags) atomicOr(flags, 1 /*NEL_FLAG_BAD_ID*/);
    for (int c = lane; c < d_out; c += 64) orow[c] = Elem<T>::from_f32(__builtin_nanf(""));
    return;
  }
  const T* hrow = h + t * d_in;
  const T* erow = emb + static_cast<int64_t>(id) * de;
  float sh = 0.f, se = 0.f;
  for (int c = lane; c < d_in; c += 64) {
    const float v = Elem<T>::to_f32(hrow[c]);
    sh = fmaf(v, v, sh);
  }
  for (int c = lane; c < de; c += 64) {
    const float v = Elem<T>::to_f32(erow[c]);
    se = fmaf(v, v, se);
  }
  sh = wave_sum(sh);
  se = wave_sum(se);
  const float k = mode == kJunctionNoRescale ? 1.f : norm_ratio(sh, se);
  for (int c = lane; c < d_in; c += 64) orow[c] = Elem<T>::from_f32(Elem<T>::to_f32(hrow[c]) * k);
  for (int c = lane; c < de; c += 64)
    orow[d_in + c] = mode == kJunctionZeroFill ? Elem<T>::from_f32(0.f) : erow[c];
}

}  // namespace

template <typename T>
hipError_t launch_junction(int64_t n, int d_in, int d_out, int vocab, const void* h,
                           const int32_t* ids, const void* emb, void* out, int32_t* flags,
                           int mode, hipStream_t s) {
  if (n == 0) return hipSuccess;
  constexpr int C = Elem<T>::kChunk;
  const int de = d_out - d_in;
  const bool vec = (d_in % C == 0) && (de % C == 0) && (d_in / C <= 64 * kMaxChunks) &&
                   (de / C <= 64 * kMaxChunks);
  const T* hp = static_cast<const T*>(h);
  const T* ep = static_cast<const T*>(emb);
  T* op = static_cast<T*>(out);
  if (!vec) {
    const dim3 grid(static_cast<unsigned>((n + kTokPerBlock - 1) / kTokPerBlock));
    hipLaunchKernelGGL(junction_elem<T>, grid, dim3(256), 0, s, n, d_in, d_out, vocab, hp, ids,
                       ep, op, flags, mode);
    return hipGetLastError();
  }
  // lanes per token: about four chunks per lane, between 8 and 64 lanes, and
  // never more chunks per lane than the register cache holds
  const int chunks = d_in / C + de / C;
  int G = 64;
  while (G > 8 && chunks < 4 * G) G /= 2;
  while (G < 64 && (d_in / C > G * kMaxChunks || de / C > G * kMaxChunks)) G *= 2;
  const int64_t per_block = static_cast<int64_t>(kTokPerBlock) * (64 / G);
  const dim3 grid(static_cast<unsigned>((n + per_block - 1) / per_block));
  switch (G) {
    case 8:
      hipLaunchKernelGGL((junction_vec<T, 8>), grid, dim3(256), 0, s, n, d_in, d_out, vocab, hp,
                         ids, ep, op, flags, mode);
      break;
    case 16:
      hipLaunchKernelGGL((junction_vec<T, 16>), grid, dim3(256), 0, s, n, d_in, d_out, vocab, hp,
                         ids, ep, op, flags, mode);
      break;
    case 32:
      hipLaunchKernelGGL((junction_vec<T, 32>), grid, dim3(256), 0, s, n, d_in, d_out, vocab, hp,
                         ids, ep, op, flags, mode);
      break;
    default:
      hipLaunchKernelGGL((junction_vec<T, 64>), grid, dim3(256), 0, s, n, d_in, d_out, vocab, hp,
                         ids, ep, op, flags, mode);
      break;
  }
  return hipGetLastError();
}

template hipError_t launch_junction<bf16_t>(int64_t, int, int, int, const void*, const int32_t*,
                                            const void*, void*, int32_t*, int, hipStream_t);
template hipError_t launch_junction<float>(int64_t, int, int, int, const void*, const int32_t*,
                                           const void*, void*, int32_t*, int, hipStream_t);

}  // namespace nel
