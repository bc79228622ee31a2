// Multi-exit LM-head GEMM with fused epilogues (gfx950, bf16 MFMA 32x32x16).
//
// Each exit m's logits l_m = h_m W^m^T (copyedit of Sec. 2 "Modeling": every
// sub-model ends in its own head W^m in R^{V x D_m}) are a dense contraction
// of [tokens x D_m] by [D_m x V], run on the matrix cores with fp32
// accumulation.  The fp32 logits never leave registers.  One workgroup owns a
// 128-token x 128-vocabulary tile and runs it for every exit in turn.
//
// Loss epilogue ("Matryoshka Language Model Suites", distillation paragraph:
// the largest exit's softmax teaches the smaller exits).  The teacher exit
// (the last one) runs first; its tile is turned into w = exp(l_M - m_M) with
// m_M the tile's row maximum and kept in registers while the smaller exits run,
// so for every exit the tile emits, per token:
//     m    = max_v l          sigma = sum_v exp(l - m)
//     S    = sum_v w_v l_m,v  (smaller exits: the teacher-weighted logit sum)
//     l[y] (the label's logit, captured by the one lane that holds it)
// and, when a gradient is wanted, the tile-shifted copy l - m (rounded once to
// the caller's element type) into the caller's dlogits buffer.  A later pass
// merges the tiles (online log-sum-exp) and finalises the gradient in place.
//
// Argmax epilogue: per token the tile's (max, lowest index), optionally the
// fp32 logits.
//
// Layout.  Operands are both K-contiguous: the A operand of the MFMA is a
// 32-row block of W (vocabulary rows), the B operand 32 rows of h (tokens), so
// an accumulator lane holds one token and 16 vocabulary entries; the A rows
// are loaded in a permuted order that makes those 16 entries consecutive.
// Row reductions over the vocabulary are then in-register plus one exchange
// with the lane 32 apart.  A and B tiles are staged through LDS, double
// buffered, 128-byte rows with an XOR chunk swizzle.
#include <limits.h>

#include "common.h"
#include "internal.h"

namespace nel {

namespace {

constexpr int kThreads = 256;            // 4 wavefronts: 2 (tokens) x 2 (vocabulary)
constexpr int kRowBytes = 128;           // LDS row: 8 chunks of 16 bytes
constexpr int kStageBytes = (kVocTile + kTokTile) * kRowBytes;
constexpr int kLdsBytes = 2 * kStageBytes;

enum { kModeLoss = 0, kModeArgmax = 1 };

template <typename T> struct KStep;
template <> struct KStep<bf16_t> { static constexpr int v = 64; };   // 64 bf16 = 128 bytes
template <> struct KStep<float> { static constexpr int v = 32; };    // 32 fp32 = 128 bytes

// A-row q of a 32-row MFMA block holds vocabulary entry vperm(q), chosen so
// that accumulator register r of lane half h is vocabulary entry 16h + r.
__device__ __forceinline__ int vperm(int q) { return ((q >> 2) & 1) * 16 + (q >> 3) * 4 + (q & 3); }
// Chunk swizzles: any 8 consecutive lanes of an operand read hit 8 different
// 16-byte bank groups.
__device__ __forceinline__ int swz_a(int r) { return (r & 3) | ((r >> 2) & 4); }
__device__ __forceinline__ int swz_b(int r) { return r & 7; }

// Workgroup id -> (token tile, vocabulary tile).  Consecutive ids are spread
// over the 8 XCDs, so ids are first regrouped per XCD; each XCD then walks
// groups of 8 token tiles across the vocabulary, which keeps an 8 x 8 block
// of tiles (sharing 8 token and 8 vocabulary operand panels) resident in its L2.
__device__ __forceinline__ void tile_coords(int bid, int n_tt, int n_vt, int& tt, int& vt) {
  const int G = n_tt * n_vt;
  int L = bid;
  if ((G & 7) == 0) L = (bid & 7) * (G >> 3) + (bid >> 3);
  constexpr int kGroup = 8;
  const int per_group = kGroup * n_vt;
  const int g = L / per_group;
  const int first = g * kGroup;
  const int gs = min(n_tt - first, kGroup);
  const int r = L - g * per_group;
  tt = first + r % gs;
  vt = r / gs;
}

// One 16-byte chunk of row `row`, elements [k, k + chunk); zero outside the
// matrix.  VEC: rows are whole chunks (D a multiple of the chunk).
template <typename T, bool VEC>
__device__ __forceinline__ u32x4 load_chunk(const T* __restrict__ P, int64_t row, int64_t rows,
                                            int k, int D) {
  constexpr int C = Elem<T>::kChunk;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (row < rows && k < D) {
    const T* p = P + row * D + k;
    if constexpr (VEC) {
      r = *reinterpret_cast<const u32x4*>(p);
    } else {
      T tmp[C];
#pragma unroll
      for (int i = 0; i < C; ++i) tmp[i] = (k + i < D) ? p[i] : T(0);
      r = *reinterpret_cast<const u32x4*>(tmp);
    }
  }
  return r;
}

template <typename T, int MODE, bool VEC>
__global__ __launch_bounds__(kThreads, 2) void heads_kernel(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    const int32_t* __restrict__ labels, float* __restrict__ stats,
    float* __restrict__ lab, int n_tt, int n_vt) {
  // The exit table is the first kernel argument; indexing it through the
  // kernarg segment pointer turns a per-exit lookup into one scalar load.
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int C = Elem<T>::kChunk;
  constexpr int BK = KStep<T>::v;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ float xmax[2][2][64];     // [wt][wv][token] row maximum of a wavefront's 64 columns
  __shared__ float xsum[2][2][64][2];  // [wt][wv][token] sum exp | S   (argmax: value | index)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wt = wave >> 1, wv = wave & 1;
  const int hl = lane >> 5, q = lane & 31;
  int tt, vt;
  tile_coords(blockIdx.x, n_tt, n_vt, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kTokTile;
  const int v0 = vt * kVocTile;

  int64_t tok[2];
  int ylab[2];
  int vbase[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    tok[tb] = t0 + wt * 64 + tb * 32 + q;
    ylab[tb] = (MODE == kModeLoss && tok[tb] < n) ? labels[tok[tb]] : -1;
  }
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) vbase[vb] = v0 + wv * 64 + vb * 32 + 16 * hl;

  f32x16 acc[2][2];
  float wt_[2][2][16];   // teacher weights exp(l_M - m_M) (loss mode)

  for (int ei = 0; ei < n_exits; ++ei) {
    const int e = (MODE == kModeLoss) ? (ei == 0 ? n_exits - 1 : ei - 1) : ei;
    const bool teacher = (MODE == kModeLoss) && ei == 0;
    const int D = ex.d[e];
    const T* __restrict__ H = static_cast<const T*>(ex.h[e]);
    const T* __restrict__ W = static_cast<const T*>(ex.w[e]);

#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][vb][r] = 0.f;

    // ---------------- K loop: global -> registers -> LDS (double buffered) -> MFMA
    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qd = tid + kThreads * j;
        const int row = qd >> 3, c = qd & 7;
        ra[j] = load_chunk<T, VEC>(W, v0 + row, vocab, k0 + c * C, D);
        rb[j] = load_chunk<T, VEC>(H, t0 + row, n, k0 + c * C, D);
      }
    };
    auto sstore = [&](int buf) {
      uint8_t* A = lds + buf * kStageBytes;
      uint8_t* B = A + kVocTile * kRowBytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qd = tid + kThreads * j;
        const int row = qd >> 3, c = qd & 7;
        *reinterpret_cast<u32x4*>(A + row * kRowBytes + ((c ^ swz_a(row)) << 4)) = ra[j];
        *reinterpret_cast<u32x4*>(B + row * kRowBytes + ((c ^ swz_b(row)) << 4)) = rb[j];
      }
    };
    auto compute = [&](int buf) {
      const uint8_t* A = lds + buf * kStageBytes;
      const uint8_t* B = A + kVocTile * kRowBytes;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int c = 2 * kk + hl;
          bf16x8 a[2], b[2];
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            const int r = wv * 64 + vb * 32 + vperm(q);
            a[vb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(A + r * kRowBytes + ((c ^ swz_a(r)) << 4)));
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const int r = wt * 64 + tb * 32 + q;
            b[tb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(B + r * kRowBytes + ((c ^ swz_b(r)) << 4)));
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
              acc[tb][vb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[vb], b[tb], acc[tb][vb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < BK / 2; ++s) {
          const int kidx = 2 * s + hl;
          const int c = kidx >> 2, wi = kidx & 3;
          float a[2], b[2];
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            const int r = wv * 64 + vb * 32 + vperm(q);
            a[vb] = *reinterpret_cast<const float*>(A + r * kRowBytes + ((c ^ swz_a(r)) << 4) + wi * 4);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            const int r = wt * 64 + tb * 32 + q;
            b[tb] = *reinterpret_cast<const float*>(B + r * kRowBytes + ((c ^ swz_b(r)) << 4) + wi * 4);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int vb = 0; vb < 2; ++vb)
              acc[tb][vb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[vb], b[tb], acc[tb][vb], 0, 0, 0);
        }
      }
    };

    const int nk = (D + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk) gload((ks + 1) * BK);
      compute(ks & 1);
      if (ks + 1 < nk) sstore((ks + 1) & 1);
      __syncthreads();
    }

    // ---------------- epilogue
    if constexpr (MODE == kModeLoss) {
      // (1) row maximum over the workgroup's 128 vocabulary entries: in
      // registers, with the lane 32 apart, then with the other vocabulary
      // wavefront through LDS.  Everything below is relative to it.
      float M[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float m = -INFINITY;
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vbase[vb] + r < vocab) m = fmaxf(m, acc[tb][vb][r]);
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (hl == 0) xmax[wt][wv][tb * 32 + q] = m;
      }
      __syncthreads();
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        M[tb] = fmaxf(xmax[wt][0][tb * 32 + q], xmax[wt][1][tb * 32 + q]);

      // (2) sums, teacher weights, label logit, shifted copy.
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const float m = M[tb];
        float s = 0.f, S = 0.f;
        if (teacher) {
#pragma unroll
          for (int vb = 0; vb < 2; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float x = (vbase[vb] + r < vocab) ? fexp(acc[tb][vb][r] - m) : 0.f;
              wt_[tb][vb][r] = x;
              s += x;
            }
        } else {
#pragma unroll
          for (int vb = 0; vb < 2; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if (vbase[vb] + r < vocab) s += fexp(acc[tb][vb][r] - m);
              S = fmaf(wt_[tb][vb][r], acc[tb][vb][r], S);
            }
        }
        s += __shfl_xor(s, 32, 64);
        S += __shfl_xor(S, 32, 64);

        // the label's logit: exactly one lane in the grid holds (token, y)
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
          const int dd = ylab[tb] - vbase[vb];
          if (static_cast<unsigned>(dd) < 16u && ylab[tb] < vocab) {
            float val = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) val = (r == dd) ? acc[tb][vb][r] : val;
            lab[static_cast<int64_t>(e) * n + tok[tb]] = val;
          }
        }
        // tile-shifted logits l - M into the gradient buffer
        if (ex.out[e] != nullptr && tok[tb] < n) {
          T* orow = static_cast<T*>(ex.out[e]) + tok[tb] * vocab;
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            if (VEC && vbase[vb] + 16 <= vocab) {
              u32x4* dst = reinterpret_cast<u32x4*>(orow + vbase[vb]);
              if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                  u32x4 pk;
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    pk[j] = pack_bf16x2(acc[tb][vb][8 * h2 + 2 * j] - m,
                                        acc[tb][vb][8 * h2 + 2 * j + 1] - m);
                  __builtin_nontemporal_store(pk, dst + h2);
                }
              } else {
#pragma unroll
                for (int h4 = 0; h4 < 4; ++h4) {
                  u32x4 pk;
#pragma unroll
                  for (int j = 0; j < 4; ++j) pk[j] = __float_as_uint(acc[tb][vb][4 * h4 + j] - m);
                  __builtin_nontemporal_store(pk, dst + h4);
                }
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (vbase[vb] + r < vocab) orow[vbase[vb] + r] = Elem<T>::from_f32(acc[tb][vb][r] - m);
            }
          }
        }
        if (hl == 0) {
          xsum[wt][wv][tb * 32 + q][0] = s;
          xsum[wt][wv][tb * 32 + q][1] = S;
        }
      }
      __syncthreads();
      // (3) wave (wt, wv) adds the two vocabulary halves of token block tb = wv.
      if (hl == 0) {
        const int j = wv * 32 + q;
        const int64_t tk = t0 + wt * 64 + j;
        if (tk < n) {
          const int64_t plane = static_cast<int64_t>(n_vt) * n;
          float* st = stats + (static_cast<int64_t>(e) * 3 * n_vt + vt) * n + tk;
          st[0] = M[wv];
          st[plane] = xsum[wt][0][j][0] + xsum[wt][1][j][0];
          if (!teacher) st[2 * plane] = xsum[wt][0][j][1] + xsum[wt][1][j][1];
        }
      }
      // xmax was last read before the barrier above; xsum is next written
      // after the next exit's K-loop barriers.
    } else {
      // ---------------- argmax epilogue
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float bv = -INFINITY;
        int bi = INT_MAX;
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vbase[vb] + r < vocab && acc[tb][vb][r] > bv) {
              bv = acc[tb][vb][r];
              bi = vbase[vb] + r;
            }
        const float ov = __shfl_xor(bv, 32, 64);
        const int oi = __shfl_xor(bi, 32, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
        if (ex.out[e] != nullptr && tok[tb] < n) {
          float* orow = static_cast<float*>(ex.out[e]) + tok[tb] * vocab;
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            if (VEC && vbase[vb] + 16 <= vocab) {
              u32x4* dst = reinterpret_cast<u32x4*>(orow + vbase[vb]);
#pragma unroll
              for (int h4 = 0; h4 < 4; ++h4) {
                u32x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[j] = __float_as_uint(acc[tb][vb][4 * h4 + j]);
                dst[h4] = pk;
              }
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (vbase[vb] + r < vocab) orow[vbase[vb] + r] = acc[tb][vb][r];
            }
          }
        }
        if (hl == 0) {
          xsum[wt][wv][tb * 32 + q][0] = bv;
          xsum[wt][wv][tb * 32 + q][1] = __int_as_float(bi);
        }
      }
      __syncthreads();
      if (hl == 0) {
        const int j = wv * 32 + q;
        float bv = xsum[wt][0][j][0];
        int bi = __float_as_int(xsum[wt][0][j][1]);
        const float ov = xsum[wt][1][j][0];
        const int oi = __float_as_int(xsum[wt][1][j][1]);
        if (ov > bv) {   // the second half holds higher indices: ties keep the first
          bv = ov;
          bi = oi;
        }
        const int64_t tk = t0 + wt * 64 + j;
        if (tk < n) {
          const int64_t plane = static_cast<int64_t>(n_vt) * n;
          float* b = stats + (static_cast<int64_t>(e) * 2 * n_vt + vt) * n + tk;
          b[0] = bv;
          b[plane] = __int_as_float(bi);
        }
      }
    }
  }
}

// The chunk kernels need every width and the vocabulary to be whole 16-byte
// chunks (fp32 logits rows too: a multiple of 4 elements).
template <typename T>
bool all_chunked(int n_exits, int vocab, const ExitSet& ex) {
  constexpr int C = sizeof(T) == 2 ? 8 : 4;
  for (int e = 0; e < n_exits; ++e)
    if (ex.d[e] % C != 0) return false;
  return vocab % C == 0;
}

}  // namespace

template <typename T>
hipError_t launch_heads_loss(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                             const int32_t* labels, float* stats, float* lab, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int n_tt = static_cast<int>((n + kTokTile - 1) / kTokTile);
  const int n_vt = static_cast<int>(n_vocab_tiles(vocab));
  if (all_chunked<T>(n_exits, vocab, ex))
    hipLaunchKernelGGL((heads_kernel<T, kModeLoss, true>), dim3(n_tt * n_vt), dim3(kThreads), 0,
                       s, ex, n_exits, n, vocab, labels, stats, lab, n_tt, n_vt);
  else
    hipLaunchKernelGGL((heads_kernel<T, kModeLoss, false>), dim3(n_tt * n_vt), dim3(kThreads), 0,
                       s, ex, n_exits, n, vocab, labels, stats, lab, n_tt, n_vt);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_heads_argmax(int n_exits, int64_t n, int vocab, const ExitSet& ex, float* best,
                               hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int n_tt = static_cast<int>((n + kTokTile - 1) / kTokTile);
  const int n_vt = static_cast<int>(n_vocab_tiles(vocab));
  if (all_chunked<T>(n_exits, vocab, ex))
    hipLaunchKernelGGL((heads_kernel<T, kModeArgmax, true>), dim3(n_tt * n_vt), dim3(kThreads),
                       0, s, ex, n_exits, n, vocab, nullptr, best, nullptr, n_tt, n_vt);
  else
    hipLaunchKernelGGL((heads_kernel<T, kModeArgmax, false>), dim3(n_tt * n_vt), dim3(kThreads),
                       0, s, ex, n_exits, n, vocab, nullptr, best, nullptr, n_tt, n_vt);
  return hipGetLastError();
}

template hipError_t launch_heads_loss<bf16_t>(int, int64_t, int, const ExitSet&, const int32_t*,
                                              float*, float*, hipStream_t);
template hipError_t launch_heads_loss<float>(int, int64_t, int, const ExitSet&, const int32_t*,
                                             float*, float*, hipStream_t);
template hipError_t launch_heads_argmax<bf16_t>(int, int64_t, int, const ExitSet&, float*,
                                                hipStream_t);
template hipError_t launch_heads_argmax<float>(int, int64_t, int, const ExitSet&, float*,
                                               hipStream_t);

}  // namespace nel
