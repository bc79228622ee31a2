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
// dL/dh_t = 0 while the embedding still receives both terms.  The ablation
// modes drop terms: no rescale has dL/dh = delta_h, c_t = 0; zero fill has no
// delta_g term.
//
// dL/dh and c_t: one wavefront per token (16-byte chunks where rows allow).  dL/de is a sum over the tokens of
// each id, and ids follow a Zipf law (one id can hold 15 % of the tokens), so
// the tokens are first put in a stable order by id (a counting sort), and each
// id's list is cut into segments of kSeg tokens, one workgroup per segment:
//   rank     per block of 256 tokens: each token's rank among the earlier
//            tokens of its block with the same id, and the block's count per id
//   colscan  per id: counts of earlier blocks (exclusive) and the total count
//   rowscan  per id: start of its list, of its segments and of its
//            partial-sum slots; the segment -> id table
//   scatter  token t to list[start(id) + earlier blocks + rank]
//   segsum   per segment: the sum of its tokens' delta_g rows in list order.
//            An id with one segment writes its row; otherwise each segment
//            writes a partial
//   combine  per id with several segments: its partials added in segment order
//   zerorows rows of ids no token has are 0.
// Every sum runs in an order fixed by the token order alone (no atomics on
// floats), so reruns are bit-identical.
#include "common.h"
#include "internal.h"

namespace nel {

namespace {

constexpr int kTokPerBlock = 4;   // token kernel: one wavefront per token
constexpr int kRankBlock = 256;   // tokens per rank block (one per thread)
#ifndef NEL_JBWD_SEG
#define NEL_JBWD_SEG 64
#endif
constexpr int kSeg = NEL_JBWD_SEG;  // tokens per segment of an id's list
constexpr int kCols = 8;          // columns per thread per slab of 2048
constexpr int64_t kMaxGrid = 4096;  // workgroups of the grid-stride segment kernels

__host__ __device__ __forceinline__ int seg_count(int c) { return (c + kSeg - 1) / kSeg; }
__host__ __device__ __forceinline__ int part_count(int c) {
  const int s = seg_count(c);
  return s > 1 ? s : 0;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) {
  return Elem<T>::to_f32(p[i]);
}

template <typename T>
__global__ __launch_bounds__(256) void junction_bwd_token(
    int64_t n, int d_in, int d_out, int vocab, const T* __restrict__ h,
    const int32_t* __restrict__ ids, const T* __restrict__ emb, const T* __restrict__ dout,
    int stop_grad, T* __restrict__ dh, float* __restrict__ ct, int32_t* __restrict__ flags, int mode) {
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
  const bool norm = mode != kJunctionNoRescale;
  const bool live = norm && sh > 0.f && se > 0.f;   // the rescaled half depends on a and b
  const float a = sqrtf(sh);
  if (lane == 0) ct[t] = live ? hd / a : 0.f;
  if (!dh) return;
  const float k = stop_grad ? 0.f : norm ? (live ? sqrtf(se) / a : 0.f) : 1.f;
  const float proj = live ? hd / sh : 0.f;
  for (int c = lane; c < d_in; c += 64)
    dh[t * d_in + c] = Elem<T>::from_f32(k * (ld(drow, c) - ld(hrow, c) * proj));
}

// 16-byte chunks: C elements of T as fp32 and back (RNE to bf16).
template <typename T> struct Chunk;
template <> struct Chunk<bf16_t> {
  static constexpr int C = 8;
  __device__ static void get(const u32x4& r, float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(r[j] << 16);
      x[2 * j + 1] = __uint_as_float(r[j] & 0xffff0000u);
    }
  }
  __device__ static u32x4 put(const float (&x)[8]) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
    return r;
  }
};
template <> struct Chunk<float> {
  static constexpr int C = 4;
  __device__ static void get(const u32x4& r, float (&x)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(r[j]);
  }
  __device__ static u32x4 put(const float (&x)[4]) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __float_as_uint(x[j]);
    return r;
  }
};

// The token kernel on 16-byte chunks (every row start and width a whole
// number of chunks): lane l holds chunks l + 64 i (i < NCH) of h_t and
// delta_h in registers between the sums and the dL/dh store.
constexpr int kTokNch = 8;

template <typename T>
__global__ __launch_bounds__(256) void junction_bwd_token_vec(
    int64_t n, int d_in, int d_out, int vocab, const T* __restrict__ h,
    const int32_t* __restrict__ ids, const T* __restrict__ emb, const T* __restrict__ dout,
    int stop_grad, T* __restrict__ dh, float* __restrict__ ct, int32_t* __restrict__ flags, int mode) {
  constexpr int C = Chunk<T>::C;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + (threadIdx.x >> 6);
  if (t >= n) return;
  const int de = d_out - d_in;
  const int nin = d_in / C, nde = de / C;
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
  const u32x4* hrow = reinterpret_cast<const u32x4*>(h + t * d_in);
  const u32x4* drow = reinterpret_cast<const u32x4*>(dout + t * d_out);   // delta_h first
  const u32x4* erow = reinterpret_cast<const u32x4*>(emb + static_cast<int64_t>(id) * de);
  u32x4 hv[kTokNch], dv[kTokNch];
#pragma unroll
  for (int i = 0; i < kTokNch; ++i) {
    const int ci = lane + 64 * i;
    if (ci < nin) {
      hv[i] = hrow[ci];
      dv[i] = drow[ci];
    }
  }
  float sh = 0.f, se = 0.f, hd = 0.f;
  for (int ci = lane; ci < nde; ci += 64) {
    float e[C];
    Chunk<T>::get(erow[ci], e);
#pragma unroll
    for (int j = 0; j < C; ++j) se = fmaf(e[j], e[j], se);
  }
#pragma unroll
  for (int i = 0; i < kTokNch; ++i) {
    if (lane + 64 * i < nin) {
      float x[C], d[C];
      Chunk<T>::get(hv[i], x);
      Chunk<T>::get(dv[i], d);
#pragma unroll
      for (int j = 0; j < C; ++j) {
        sh = fmaf(x[j], x[j], sh);
        hd = fmaf(x[j], d[j], hd);
      }
    }
  }
  sh = wave_sum(sh);
  se = wave_sum(se);
  hd = wave_sum(hd);
  const bool norm = mode != kJunctionNoRescale;
  const bool live = norm && sh > 0.f && se > 0.f;
  const float a = sqrtf(sh);
  if (lane == 0) ct[t] = live ? hd / a : 0.f;
  if (!dh) return;
  const float k = stop_grad ? 0.f : norm ? (live ? sqrtf(se) / a : 0.f) : 1.f;
  const float proj = live ? hd / sh : 0.f;
  u32x4* orow = reinterpret_cast<u32x4*>(dh + t * d_in);
#pragma unroll
  for (int i = 0; i < kTokNch; ++i) {
    const int ci = lane + 64 * i;
    if (ci < nin) {
      float x[C], d[C], o[C];
      Chunk<T>::get(hv[i], x);
      Chunk<T>::get(dv[i], d);
#pragma unroll
      for (int j = 0; j < C; ++j) o[j] = k * (d[j] - x[j] * proj);
      orow[ci] = Chunk<T>::put(o);
    }
  }
}

// Block b holds tokens [256 b, 256 b + 256), one per thread.  rank[t] =
// number of tokens of the block before t with t's id; the last token of each
// id in the block stores the block's count in hist[b][id] (hist is zero
// beforehand).  Tokens past n or with a bad id take no part.
__global__ __launch_bounds__(256) void rank_kernel(int64_t n, int vocab,
                                                   const int32_t* __restrict__ ids,
                                                   int32_t* __restrict__ rank,
                                                   int32_t* __restrict__ hist) {
  __shared__ __align__(16) int32_t sid[kRankBlock];
  const int tid = threadIdx.x;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRankBlock + tid;
  int id = t < n ? ids[t] : -1;
  if (id < 0 || id >= vocab) id = -1;
  sid[tid] = id;
  __syncthreads();
  int before = 0, same = 0;
  for (int j = 0; j < kRankBlock; j += 4) {
    const int4 x = *reinterpret_cast<const int4*>(&sid[j]);   // same address in every lane
    const int xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool eq = xs[q] == id;
      before += eq && j + q < tid;
      same += eq;
    }
  }
  if (t >= n) return;
  rank[t] = id >= 0 ? before : -1;
  if (id >= 0 && before + 1 == same)   // the block's last token with this id
    hist[static_cast<int64_t>(blockIdx.x) * vocab + id] = same;
}

// Exclusive scan of three per-thread counts over a 256-thread workgroup, in
// thread order; also returns the workgroup totals.
__device__ __forceinline__ void block_scan3(int (&x)[3], int (&total)[3], int* red /*[4][3]*/) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl[3] = {x[0], x[1], x[2]};
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int y = __shfl_up(incl[k], o, 64);
      if (lane >= o) incl[k] += y;
    }
  }
  __syncthreads();   // red is free
  if (lane == 63)
    for (int k = 0; k < 3; ++k) red[wave * 3 + k] = incl[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    int before = incl[k] - x[k];
    for (int w = 0; w < wave; ++w) before += red[w * 3 + k];
    total[k] = (red[k] + red[3 + k]) + (red[6 + k] + red[9 + k]);
    x[k] = before;
  }
}

// Per id v (one per thread): hist[b][v] <- tokens with id v in blocks before
// b; cnt[v] <- its total.  Each workgroup stores the totals of its 256 ids'
// tokens, segments and partial slots in wgtot[blockIdx.x].
__global__ __launch_bounds__(256) void colscan_kernel(int nblk, int vocab,
                                                      int32_t* __restrict__ hist,
                                                      int32_t* __restrict__ cnt,
                                                      int32_t* __restrict__ wgtot) {
  __shared__ int red[12];
  const int v = blockIdx.x * 256 + threadIdx.x;
  int run = 0;
  if (v < vocab) {
    constexpr int U = 8;   // blocks read together
    int b = 0;
    for (; b + U <= nblk; b += U) {
      int c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = hist[static_cast<int64_t>(b + u) * vocab + v];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        hist[static_cast<int64_t>(b + u) * vocab + v] = run;
        run += c[u];
      }
    }
    for (; b < nblk; ++b) {
      int32_t* p = hist + static_cast<int64_t>(b) * vocab + v;
      const int c = *p;
      *p = run;
      run += c;
    }
    cnt[v] = run;
  }
  int x[3] = {run, seg_count(run), part_count(run)}, tot[3];
  block_scan3(x, tot, red);
  if (threadIdx.x < 3) wgtot[blockIdx.x * 3 + threadIdx.x] = tot[threadIdx.x];
}

// Per id, in id order: rowoff = start of its token list, poff = its first
// partial slot; for each of its segments the record {id, list begin, list
// end, partial slot or -1}; the partial slot -> id table; the totals of
// segments and of partial slots in counts[0..1].  Workgroup w adds the totals
// of workgroups < w.
__global__ __launch_bounds__(256) void rowscan_kernel(int vocab, const int32_t* __restrict__ cnt,
                                                      const int32_t* __restrict__ wgtot,
                                                      int32_t* __restrict__ rowoff,
                                                      int32_t* __restrict__ poff,
                                                      int4* __restrict__ seginfo,
                                                      int32_t* __restrict__ prow_id,
                                                      int32_t* __restrict__ counts) {
  __shared__ int red[12];
  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  // carry: the totals of workgroups before w, summed in a fixed order
  int carry[3] = {0, 0, 0};
  for (int k = tid; k < w; k += 256) {
    carry[0] += wgtot[3 * k];
    carry[1] += wgtot[3 * k + 1];
    carry[2] += wgtot[3 * k + 2];
  }
  int tot[3];
  block_scan3(carry, tot, red);   // tot = the sum over all threads
  const int v = w * 256 + tid;
  const int c = v < vocab ? cnt[v] : 0;
  int x[3] = {c, seg_count(c), part_count(c)}, wt[3];
  block_scan3(x, wt, red);
  if (v < vocab) {
    const int r0 = tot[0] + x[0], s0 = tot[1] + x[1], p0 = tot[2] + x[2];
    rowoff[v] = r0;
    poff[v] = p0;
    const int ns = seg_count(c);
    for (int j = 0; j < ns; ++j)
      seginfo[s0 + j] = make_int4(v, r0 + j * kSeg, r0 + min(c, (j + 1) * kSeg), ns > 1 ? p0 + j : -1);
    for (int j = 0; j < part_count(c); ++j) prow_id[p0 + j] = v;
  }
  if (w == static_cast<int>(gridDim.x) - 1 && tid == 0) {
    counts[0] = tot[1] + wt[1];
    counts[1] = tot[2] + wt[2];
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(int64_t n, int vocab,
                                                      const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ hist,
                                                      const int32_t* __restrict__ rowoff,
                                                      int32_t* __restrict__ list) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n) return;
  const int id = ids[t];
  if (id < 0 || id >= vocab) return;
  const int64_t b = t / kRankBlock;
  list[rowoff[id] + hist[b * vocab + id] + rank[t]] = static_cast<int32_t>(t);
}

// Thread columns of a slab of 256 x kCols: VEC (rows in whole 16-byte chunks)
// owns kCols consecutive columns read as 16-byte chunks, else columns
// tid + 256 j read one by one.
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

template <bool VEC>
__device__ __forceinline__ int col_of(int c0, int j) {
  return VEC ? c0 + static_cast<int>(threadIdx.x) * kCols + j : c0 + static_cast<int>(threadIdx.x) + 256 * j;
}

// 1 / ||e[v]||, summed in a fixed order (0 for a zero row).
template <typename T>
__device__ float inv_norm(const T* erow, int de, float* red) {
  const int tid = threadIdx.x;
  float se = 0.f;
  for (int c = tid; c < de; c += 256) {
    const float ev = ld(erow, c);
    se = fmaf(ev, ev, se);
  }
  se = wave_sum(se);
  __syncthreads();   // red is free
  if ((tid & 63) == 0) red[tid >> 6] = se;
  __syncthreads();
  se = (red[0] + red[1]) + (red[2] + red[3]);
  return se > 0.f ? 1.f / sqrtf(se) : 0.f;
}

// Segments g = blockIdx.x, blockIdx.x + gridDim.x, ... < counts[0].  An id
// with one segment gets its row; otherwise the segment's column sums go to
// its partial slot (and its sum of c_t to pcs) for combine_kernel.  ONE
// (16-byte chunks, a single slab): the thread's kCols columns of e[v] are
// read with the tokens' rows and serve both ||e[v]|| and the output.
template <typename T, bool VEC, bool ONE>
__global__ __launch_bounds__(256) void segsum_kernel(
    int d_in, int d_out, const T* __restrict__ emb, const T* __restrict__ dout,
    const float* __restrict__ ct, const int32_t* __restrict__ list,
    const int4* __restrict__ seginfo, const int32_t* __restrict__ counts,
    float* __restrict__ partial, float* __restrict__ pcs, float* __restrict__ demb, int use_dg) {
  static_assert(!ONE || VEC, "one-slab path reads 16-byte chunks");
  __shared__ float red[4];
  const int de = d_out - d_in;
  const int nseg = counts[0];
  for (int g = blockIdx.x; g < nseg; g += gridDim.x) {
    const int4 si = seginfo[g];
    const int v = si.x, k0 = si.y, k1 = si.z, slot = si.w;
    const T* erow = emb + static_cast<int64_t>(v) * de;
    float* orow = demb + static_cast<int64_t>(v) * de;
    float* prow = slot >= 0 ? partial + static_cast<int64_t>(slot) * de : nullptr;
    float ev[kCols];
    float ginv = 0.f;
    if constexpr (ONE) {
      const int cb = col_of<true>(0, 0);
      if (slot < 0 && cb < de) load_cols(erow + cb, ev);
    } else {
      if (slot < 0) ginv = inv_norm(erow, de, red);
    }
    float csum = 0.f;
    for (int c0 = 0; c0 < de; c0 += 256 * kCols) {
      float acc[kCols];
#pragma unroll
      for (int q = 0; q < kCols; ++q) acc[q] = 0.f;
      csum = 0.f;
      // 8 tokens' rows are requested together (past k1: the last token, not
      // added), then added in list order
      for (int k = k0; k < k1; k += 8) {
        float x[8][kCols], cx[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t t = list[min(k + u, k1 - 1)];
          const T* drow = dout + t * d_out + d_in;   // delta_g
          if (!use_dg) {
#pragma unroll
            for (int q = 0; q < kCols; ++q) x[u][q] = 0.f;
          } else if constexpr (VEC) {
            const int cb = col_of<true>(c0, 0);
            if (cb < de) load_cols(drow + cb, x[u]);
          } else {
#pragma unroll
            for (int q = 0; q < kCols; ++q) {
              const int cc = col_of<false>(c0, q);
              x[u][q] = cc < de ? ld(drow, cc) : 0.f;
            }
          }
          cx[u] = ct[t];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k + u >= k1) break;
#pragma unroll
          for (int q = 0; q < kCols; ++q) acc[q] += x[u][q];
          csum += cx[u];
        }
      }
      if constexpr (ONE) {
        if (slot < 0) {
          const bool mine = col_of<true>(0, 0) < de;
          float se = 0.f;
          if (mine) {
#pragma unroll
            for (int q = 0; q < kCols; ++q) se = fmaf(ev[q], ev[q], se);
          }
          se = wave_sum(se);
          __syncthreads();   // red is free
          if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = se;
          __syncthreads();
          se = (red[0] + red[1]) + (red[2] + red[3]);
          ginv = se > 0.f ? 1.f / sqrtf(se) : 0.f;
          if (mine) {
#pragma unroll
            for (int q = 0; q < kCols; ++q)
              orow[col_of<true>(0, q)] = acc[q] + csum * ev[q] * ginv;
          }
          continue;
        }
      }
#pragma unroll
      for (int q = 0; q < kCols; ++q) {
        const int cc = col_of<VEC>(c0, q);
        if (cc >= de) continue;
        if (slot < 0)
          orow[cc] = acc[q] + csum * ld(erow, cc) * ginv;
        else
          prow[cc] = acc[q];
      }
    }
    if (slot >= 0 && threadIdx.x == 0) pcs[slot] = csum;
  }
}

// Partial slots p = blockIdx.x, ... < counts[1]; the workgroup at an id's
// first slot adds the id's partials in segment order and writes its row.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(
    int d_in, int d_out, const T* __restrict__ emb, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ poff, const int32_t* __restrict__ prow_id,
    const int32_t* __restrict__ counts, const float* __restrict__ partial,
    const float* __restrict__ pcs, float* __restrict__ demb) {
  __shared__ float red[4];
  const int de = d_out - d_in;
  const int npart = counts[1];
  for (int p = blockIdx.x; p < npart; p += gridDim.x) {
    const int v = prow_id[p];
    if (poff[v] != p) continue;
    const int ns = seg_count(cnt[v]);
    const T* erow = emb + static_cast<int64_t>(v) * de;
    float* orow = demb + static_cast<int64_t>(v) * de;
    const float* pbase = partial + static_cast<int64_t>(p) * de;
    float ctot = 0.f;
    for (int q = 0; q < ns; ++q) ctot += pcs[p + q];
    const float gi = inv_norm(erow, de, red);
    for (int c0 = 0; c0 < de; c0 += 256 * kCols) {
      float sum[kCols];
#pragma unroll
      for (int q = 0; q < kCols; ++q) sum[q] = 0.f;
      // 8 partials requested together (past ns: the last, not added), added in order
      for (int s0 = 0; s0 < ns; s0 += 8) {
        float y[8][kCols];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float* pr = pbase + static_cast<int64_t>(min(s0 + u, ns - 1)) * de;
          if constexpr (VEC) {
            const int cb = col_of<true>(c0, 0);
            if (cb < de) {
              const float4 a = *reinterpret_cast<const float4*>(pr + cb);
              const float4 b = *reinterpret_cast<const float4*>(pr + cb + 4);
              y[u][0] = a.x; y[u][1] = a.y; y[u][2] = a.z; y[u][3] = a.w;
              y[u][4] = b.x; y[u][5] = b.y; y[u][6] = b.z; y[u][7] = b.w;
            }
          } else {
#pragma unroll
            for (int q = 0; q < kCols; ++q) {
              const int cc = col_of<false>(c0, q);
              y[u][q] = cc < de ? pr[cc] : 0.f;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (s0 + u >= ns) break;
#pragma unroll
          for (int q = 0; q < kCols; ++q) sum[q] += y[u][q];
        }
      }
#pragma unroll
      for (int q = 0; q < kCols; ++q) {
        const int cc = col_of<VEC>(c0, q);
        if (cc < de) orow[cc] = sum[q] + ctot * ld(erow, cc) * gi;
      }
    }
  }
}

// Rows of ids that no token has: 0.
__global__ __launch_bounds__(256) void zerorows_kernel(int de, const int32_t* __restrict__ cnt,
                                                       float* __restrict__ demb) {
  const int v = blockIdx.x;
  if (cnt[v] != 0) return;
  float* orow = demb + static_cast<int64_t>(v) * de;
  if (de % 4 == 0) {
    float4* o4 = reinterpret_cast<float4*>(orow);
    for (int c = threadIdx.x; c < de / 4; c += 256) o4[c] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int c = threadIdx.x; c < de; c += 256) orow[c] = 0.f;
  }
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int64_t count) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0;
}

int64_t max_segments(int64_t n, int vocab) {
  return (n + kSeg - 1) / kSeg + (n < vocab ? n : vocab);
}
// An id with more than one segment has c > kSeg tokens and ceil(c / kSeg) < 2 c / kSeg
// segments, so the partial slots number fewer than 2 n / kSeg.
int64_t max_partials(int64_t n) { return 2 * (n / kSeg) + 1; }

}  // namespace

JunctionBwdWs junction_bwd_ws_layout(int64_t n, int d_in, int d_out, int vocab) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t nb = static_cast<size_t>(n), V = static_cast<size_t>(vocab);
  const size_t nblk = (nb + kRankBlock - 1) / kRankBlock;
  const size_t de = static_cast<size_t>(d_out - d_in);
  JunctionBwdWs L;
  size_t o = 0;
  L.ct = o;      o += up(4 * nb);
  L.rank = o;    o += up(4 * nb);
  L.list = o;    o += up(4 * nb);
  L.hist = o;    o += up(4 * nblk * V);
  L.cnt = o;     o += up(4 * V);
  L.rowoff = o;  o += up(4 * V);
  L.poff = o;    o += up(4 * V);
  L.counts = o;  o += up(4 * 2);
  L.wgtot = o;   o += up(4 * 3 * ((V + 255) / 256));
  L.seginfo = o; o += up(16 * static_cast<size_t>(max_segments(n, vocab)));
  L.prow = o;    o += up(4 * static_cast<size_t>(max_partials(n)));
  L.pcs = o;     o += up(4 * static_cast<size_t>(max_partials(n)));
  L.partial = o; o += up(4 * static_cast<size_t>(max_partials(n)) * de);
  L.total = o;
  return L;
}

template <typename T>
hipError_t launch_junction_backward(int64_t n, int d_in, int d_out, int vocab, const void* h,
                                    const int32_t* ids, const void* emb, const void* dout,
                                    int stop_grad, int mode, void* dh, float* demb,
                                    void* workspace, int32_t* flags, hipStream_t s) {
  const JunctionBwdWs L = junction_bwd_ws_layout(n, d_in, d_out, vocab);
  char* ws = static_cast<char*>(workspace);
  auto i32 = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  float* ct = reinterpret_cast<float*>(ws + L.ct);
  const int64_t nblk = (n + kRankBlock - 1) / kRankBlock;
  int32_t* hist = i32(L.hist);
  constexpr int C = Elem<T>::kChunk;
  auto al16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  // 16-byte chunks: every row start and width whole chunks, every buffer aligned
  const bool chunked = d_in % C == 0 && d_out % C == 0 && al16(dout) && al16(emb) &&
                       (d_in == 0 || al16(h)) && (!dh || al16(dh));
  if (n > 0) {
    const dim3 grid(static_cast<unsigned>((n + kTokPerBlock - 1) / kTokPerBlock));
    if (chunked && d_in <= 64 * kTokNch * C)
      hipLaunchKernelGGL((junction_bwd_token_vec<T>), grid, dim3(256), 0, s, n, d_in, d_out,
                         vocab, static_cast<const T*>(h), ids, static_cast<const T*>(emb),
                         static_cast<const T*>(dout), stop_grad, static_cast<T*>(dh), ct, flags,
                         mode);
    else
      hipLaunchKernelGGL((junction_bwd_token<T>), grid, dim3(256), 0, s, n, d_in, d_out, vocab,
                         static_cast<const T*>(h), ids, static_cast<const T*>(emb),
                         static_cast<const T*>(dout), stop_grad, static_cast<T*>(dh), ct, flags,
                         mode);
  }
  if (!demb) return hipGetLastError();
  const int de = d_out - d_in;
  const int64_t zc = nblk * vocab;   // 0 without tokens
  const int64_t zb = (zc + 255) / 256;
  if (zc > 0)
    hipLaunchKernelGGL(zero_i32_kernel, dim3(static_cast<unsigned>(zb < 4096 ? zb : 4096)),
                       dim3(256), 0, s, hist, zc);
  if (n > 0)
    hipLaunchKernelGGL(rank_kernel, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, n, vocab,
                       ids, i32(L.rank), hist);
  const dim3 vgrid(static_cast<unsigned>((vocab + 255) / 256));
  hipLaunchKernelGGL(colscan_kernel, vgrid, dim3(256), 0, s, static_cast<int>(nblk), vocab, hist,
                     i32(L.cnt), i32(L.wgtot));
  int4* seginfo = reinterpret_cast<int4*>(ws + L.seginfo);
  hipLaunchKernelGGL(rowscan_kernel, vgrid, dim3(256), 0, s, vocab, i32(L.cnt), i32(L.wgtot),
                     i32(L.rowoff), i32(L.poff), seginfo, i32(L.prow), i32(L.counts));
  if (n > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       s, n, vocab, ids, i32(L.rank), hist, i32(L.rowoff), i32(L.list));
    // delta_g and the partials in 16-byte chunks of kCols columns
    const bool vec = chunked && de % kCols == 0;
    auto cap = [](int64_t x) { return dim3(static_cast<unsigned>(x < kMaxGrid ? x : kMaxGrid)); };
    const dim3 sgrid = cap(max_segments(n, vocab)), cgrid = cap(max_partials(n));
    float* partial = reinterpret_cast<float*>(ws + L.partial);
    float* pcs = reinterpret_cast<float*>(ws + L.pcs);
    const T* e = static_cast<const T*>(emb);
    const T* d = static_cast<const T*>(dout);
    const int32_t* lst = i32(L.list);
    const int32_t* cn = i32(L.counts);
    const int use_dg = mode != kJunctionZeroFill;   // zero fill: the zeros do not depend on e
    if (vec && de <= 256 * kCols)
      hipLaunchKernelGGL((segsum_kernel<T, true, true>), sgrid, dim3(256), 0, s, d_in, d_out, e,
                         d, ct, lst, seginfo, cn, partial, pcs, demb, use_dg);
    else if (vec)
      hipLaunchKernelGGL((segsum_kernel<T, true, false>), sgrid, dim3(256), 0, s, d_in, d_out, e,
                         d, ct, lst, seginfo, cn, partial, pcs, demb, use_dg);
    else
      hipLaunchKernelGGL((segsum_kernel<T, false, false>), sgrid, dim3(256), 0, s, d_in, d_out, e,
                         d, ct, lst, seginfo, cn, partial, pcs, demb, use_dg);
    if (vec)
      hipLaunchKernelGGL((combine_kernel<T, true>), cgrid, dim3(256), 0, s, d_in, d_out, e,
                         i32(L.cnt), i32(L.poff), i32(L.prow), cn, partial, pcs, demb);
    else
      hipLaunchKernelGGL((combine_kernel<T, false>), cgrid, dim3(256), 0, s, d_in, d_out, e,
                         i32(L.cnt), i32(L.poff), i32(L.prow), cn, partial, pcs, demb);
  }
  hipLaunchKernelGGL(zerorows_kernel, dim3(static_cast<unsigned>(vocab)), dim3(256), 0, s, de,
                     i32(L.cnt), demb);
  return hipGetLastError();
}

template hipError_t launch_junction_backward<bf16_t>(int64_t, int, int, int, const void*,
                                                     const int32_t*, const void*, const void*, int,
                                                     int, void*, float*, void*, int32_t*,
                                                     hipStream_t);
template hipError_t launch_junction_backward<float>(int64_t, int, int, int, const void*,
                                                    const int32_t*, const void*, const void*, int,
                                                    int, void*, float*, void*, int32_t*,
                                                    hipStream_t);

}  // namespace nel
