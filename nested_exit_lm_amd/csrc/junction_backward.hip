// Backward of the junction between block m and block m+1.
//
// Forward ("Matryoshka Language Model Suites", junction paragraph; key-visual
// explainer, bottom panel), per token t with g = e[x_t], a = ||h_t||,
// b = ||g||:  out_t = [h_t b / a, g]  (the rescaled half is 0 if a or b is 0).
// Given delta = dL/dout_t = [delta_h, delta_g], the chain rule gives
//     dL/dh_t   = (b / a) (delta_h - h_t (h_t . delta_h) / a^2)
//     dL/de[v]  = sum_{t: x_t = v} delta_g[t]  +  (sum_{t: x_t = v} c_t) g_v / ||g_v||,
//     c_t       = (h_t . delta_h) / a
// (the second term is d||g|| / dg = g / ||g|| carried by the rescaled half).
// Both are 0 where the forward's rescaled half is identically 0.  With the
// stop-gradient option ("Is nesting the cheapest way to build a model
// suite?", follow-up 2, arm (B): each block learns only from its own exit)
// dL/dh_t = 0 while the embedding still receives both terms.
//
// Three kernels: clear the row-used marks; one wavefront per token (dL/dh,
// c_t, mark x_t used); one workgroup per embedding row (rows nobody used are
// written as 0 at once; used rows scan the ids in token order and sum, so the
// result does not depend on scheduling; no atomics on floats).
#include "common.h"
#include "internal.h"

namespace nel {

namespace {

constexpr int kTokPerBlock = 4;   // one wavefront per token, 4 per 256-thread block

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return Elem<T>::to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(256) void junction_bwd_token(
    int64_t n, int d_in, int d_out, int vocab, const T* __restrict__ h,
    const int32_t* __restrict__ ids, const T* __restrict__ emb, const T* __restrict__ dout,
    int stop_grad, T* __restrict__ dh, float* __restrict__ ct, int32_t* __restrict__ used,
    int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= n) return;
  const int de = d_out - d_in;
  const int id = ids[t];
  if (id < 0 || id >= vocab) {
    if (lane == 0) {
      if (flags) atomicOr(flags, 1 /*NEL_FLAG_BAD_ID*/);
      ct[t] = 0.f;
    }
    if (dh)
      for (int c = lane; c < d_in; c += 64) dh[t * d_in + c] = Elem<T>::from_f32(__builtin_nanf(""));
    return;
  }
  if (lane == 0) used[id] = 1;   // every writer stores the same value
  const T* hrow = h + t * d_in;
  const T* drow = dout + t * d_out;   // delta_h = drow[0, d_in)
  const T* erow = emb + static_cast<int64_t>(id) * de;
  float sh = 0.f, se = 0.f, hd = 0.f;
  for (int c = lane; c < d_in; c += 64) {
    const float hv = ld(hrow, c), dv = ld(drow, c);
    sh = fmaf(hv, hv, sh);
    hd = fmaf(hv, dv, hd);
  }
  for (int c = lane; c < de; c += 64) {
    const float ev = ld(erow, c);
    se = fmaf(ev, ev, se);
  }
  sh = wave_sum(sh);
  se = wave_sum(se);
  hd = wave_sum(hd);
  const bool live = sh > 0.f && se > 0.f;   // the rescaled half is not identically 0
  const float a = sqrtf(sh);
  if (lane == 0) ct[t] = live ? hd / a : 0.f;
  if (!dh) return;
  const float k = (live && !stop_grad) ? sqrtf(se) / a : 0.f;
  const float proj = live ? hd / sh : 0.f;
  for (int c = lane; c < d_in; c += 64)
    dh[t * d_in + c] = Elem<T>::from_f32(k * (ld(drow, c) - ld(hrow, c) * proj));
}

// One 256-thread workgroup per embedding row v.  Each scan step reads 1024
// ids (4 per thread), lists the matching tokens in token order in LDS, and
// adds their delta_g rows into per-thread fp32 column accumulators; columns
// go in slabs of 256 x kCols.  VEC (rows in whole 16-byte chunks): thread t
// owns columns kCols t .. kCols t + 7 of the slab and reads them as 16-byte
// chunks; otherwise it owns columns t + 256 j with element reads.  Eight
// tokens' rows are requested before any is added, in token order.
constexpr int kCols = 8;

template <typename T>
__device__ __forceinline__ void load_cols(const T* p, float (&x)[kCols]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(r[j] << 16);
      x[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
  } else {
    const u32x4 r0 = *reinterpret_cast<const u32x4*>(p);
    const u32x4 r1 = *reinterpret_cast<const u32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = __uint_as_float(r0[j]);
      x[4 + j] = __uint_as_float(r1[j]);
    }
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void junction_bwd_emb(
    int64_t n, int d_in, int d_out, int vocab, const int32_t* __restrict__ ids,
    const T* __restrict__ emb, const T* __restrict__ dout, const float* __restrict__ ct,
    const int32_t* __restrict__ used, float* __restrict__ demb) {
  __shared__ int32_t list[1024];
  __shared__ int32_t wcount[4];
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v = blockIdx.x;
  const int de = d_out - d_in;
  float* orow = demb + static_cast<int64_t>(v) * de;
  if (!used[v]) {   // no token has this id: its gradient is 0
    for (int c = tid; c < de; c += 256) orow[c] = 0.f;
    return;
  }
  const T* erow = emb + static_cast<int64_t>(v) * de;
  // ||e[v]||, in a fixed reduction order
  float se = 0.f;
  for (int c = tid; c < de; c += 256) {
    const float ev = ld(erow, c);
    se = fmaf(ev, ev, se);
  }
  se = wave_sum(se);
  if (lane == 0) red[wave] = se;
  __syncthreads();
  se = (red[0] + red[1]) + (red[2] + red[3]);
  const float ginv = se > 0.f ? 1.f / sqrtf(se) : 0.f;

  for (int c0 = 0; c0 < de; c0 += 256 * kCols) {
    float acc[kCols];
#pragma unroll
    for (int j = 0; j < kCols; ++j) acc[j] = 0.f;
    float csum = 0.f;
    for (int64_t base = 0; base < n; base += 1024) {
      // this thread's 4 ids: tokens base + 4 tid + i
      int cnt = 0;
      bool m[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = base + 4 * tid + i;
        m[i] = t < n && ids[t] == v;
        cnt += m[i];
      }
      // exclusive prefix of the counts over the workgroup, in thread order
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      __syncthreads();   // the previous step's list is consumed
      if (lane == 63) wcount[wave] = incl;
      __syncthreads();
      int before = incl - cnt;
      for (int w = 0; w < wave; ++w) before += wcount[w];
      const int total = (wcount[0] + wcount[1]) + (wcount[2] + wcount[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m[i]) list[before++] = static_cast<int32_t>(base + 4 * tid + i - base);
      __syncthreads();
      // 8 tokens' rows are requested together (beyond the list: the last
      // listed token, not added), then added in token order
      for (int k0 = 0; k0 < total; k0 += 8) {
        float x[8][kCols], cx[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t t = base + list[min(k0 + u, total - 1)];
          const T* drow = dout + t * d_out + d_in;   // delta_g
          if constexpr (VEC) {
            const int cb = c0 + tid * kCols;
            if (cb < de) load_cols(drow + cb, x[u]);
          } else {
#pragma unroll
            for (int j = 0; j < kCols; ++j) {
              const int c = c0 + tid + 256 * j;
              x[u][j] = c < de ? ld(drow, c) : 0.f;
            }
          }
          cx[u] = ct[t];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k0 + u >= total) break;
#pragma unroll
          for (int j = 0; j < kCols; ++j) acc[j] += x[u][j];
          csum += cx[u];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      const int c = VEC ? c0 + tid * kCols + j : c0 + tid + 256 * j;
      if (c < de) orow[c] = acc[j] + csum * ld(erow, c) * ginv;
    }
  }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int64_t count) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0;
}

}  // namespace

JunctionBwdWs junction_bwd_ws_layout(int64_t n, int vocab) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  JunctionBwdWs L;
  L.ct = 0;
  L.used = up(sizeof(float) * static_cast<size_t>(n));
  L.total = L.used + up(sizeof(int32_t) * static_cast<size_t>(vocab));
  return L;
}

template <typename T>
hipError_t launch_junction_backward(int64_t n, int d_in, int d_out, int vocab, const void* h,
                                    const int32_t* ids, const void* emb, const void* dout,
                                    int stop_grad, void* dh, float* demb, float* ct,
                                    int32_t* used, int32_t* flags, hipStream_t s) {
  const int64_t vb = (vocab + 255) / 256;
  hipLaunchKernelGGL(zero_i32_kernel, dim3(static_cast<unsigned>(vb < 4096 ? vb : 4096)),
                     dim3(256), 0, s, used, static_cast<int64_t>(vocab));
  if (n > 0) {
    hipLaunchKernelGGL((junction_bwd_token<T>),
                       dim3(static_cast<unsigned>((n + kTokPerBlock - 1) / kTokPerBlock)),
                       dim3(256), 0, s, n, d_in, d_out, vocab, static_cast<const T*>(h), ids,
                       static_cast<const T*>(emb), static_cast<const T*>(dout), stop_grad,
                       static_cast<T*>(dh), ct, used, flags);
  }
  if (demb) {
    // 16-byte chunks of delta_g: the buffer, every row start (t d_out + d_in) and the width aligned
    constexpr int C = Elem<T>::kChunk;
    const int de = d_out - d_in;
    if (d_out % C == 0 && d_in % C == 0 && de % kCols == 0 &&
        reinterpret_cast<uintptr_t>(dout) % 16 == 0)
      hipLaunchKernelGGL((junction_bwd_emb<T, true>), dim3(static_cast<unsigned>(vocab)), dim3(256),
                         0, s, n, d_in, d_out, vocab, ids, static_cast<const T*>(emb),
                         static_cast<const T*>(dout), ct, used, demb);
    else
      hipLaunchKernelGGL((junction_bwd_emb<T, false>), dim3(static_cast<unsigned>(vocab)),
                         dim3(256), 0, s, n, d_in, d_out, vocab, ids, static_cast<const T*>(emb),
                         static_cast<const T*>(dout), ct, used, demb);
  }
  return hipGetLastError();
}

template hipError_t launch_junction_backward<bf16_t>(int64_t, int, int, int, const void*,
                                                     const int32_t*, const void*, const void*, int,
                                                     void*, float*, float*, int32_t*, int32_t*,
                                                     hipStream_t);
template hipError_t launch_junction_backward<float>(int64_t, int, int, int, const void*,
                                                    const int32_t*, const void*, const void*, int,
                                                    void*, float*, float*, int32_t*, int32_t*,
                                                    hipStream_t);

}  // namespace nel
