// Multi-exit LM-head GEMM with fused epilogues (gfx950, bf16 MFMA 32x32x16).
//
// Each exit m's logits l_m = h_m W^m^T (copyedit of Sec. 2 "Modeling": every
// sub-model ends in its own head W^m in R^{V x D_m}) are a dense contraction
// of [tokens x D_m] by [D_m x V], run on the matrix cores with fp32
// accumulation.  The fp32 logits never leave registers.  One workgroup owns a
// tokens x vocabulary tile and runs it for every exit in turn.
//
// Loss epilogue ("Matryoshka Language Model Suites", distillation paragraph:
// the largest exit's softmax teaches the smaller exits).  The teacher exit
// (the last one) runs first; its tile is turned into w = exp(l_M - m_M) with
// m_M the tile's row maximum and kept in registers while the smaller exits run,
// so for every exit the tile emits, per token:
//     m    = max_v l          sigma = sum_v exp(l - m)
//     S    = sum_v w_v l_m,v  (smaller exits: the teacher-weighted logit sum)
//     l[y] (the label's logit, captured by the one lane that holds it)
// and, when a gradient is wanted, the tile-shifted copy l - m (rounded once:
// fp16 for bf16 inputs, fp32 for fp32) into the caller's dlogits buffer.  A later pass
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
// with the lane 32 apart.  A wavefront owns NTB x 32 tokens and NVB x 32
// vocabulary entries; the workgroup is 2 x 2 wavefronts.  Operand tiles are
// staged through LDS in 128-byte rows (64 bf16 or 32 fp32 of K) with an XOR
// chunk swizzle chosen so that every 16-lane pass of a 16-byte LDS access
// touches all 64 banks once.
//
// Wavefront tile 64 x 64, workgroup 128 x 128, two workgroups per CU, one K
// step of register prefetch into two LDS stages, zero fill at every edge, so
// any width and vocabulary size is accepted.  (bf16 weights in the MFMA-tiled
// layout take the faster kernel in heads_packed.hip.)
#include <limits.h>

#include "common.h"
#include "internal.h"
#include "tiles.h"

namespace nel {

namespace {

constexpr int kRowBytes = 128;           // LDS row: 8 chunks of 16 bytes

template <typename T> struct KStep;
template <> struct KStep<bf16_t> { static constexpr int v = 64; };   // 64 bf16 = 128 bytes
template <> struct KStep<float> { static constexpr int v = 32; };    // 32 fp32 = 128 bytes

// wavefront 64 x 64 (2 x 2 blocks), workgroup 128 x 128
constexpr int kGenThreads = 256;
constexpr int kGenTok = 128;
constexpr int kGenVoc = 128;
constexpr int kGenStage = (kGenVoc + kGenTok) * kRowBytes;           // 32 KB
constexpr int kGroupGen = 8;

// Chunk swizzles (row r's logical chunk c sits at physical chunk c ^ swz(r)).
// The bank group of a 16-byte access is (row parity, physical chunk); the
// swizzles give distinct groups to the rows any 16 consecutive lanes read.
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) & 3) | ((r >> 2) & 4); }
__device__ __forceinline__ int swz_b(int r) { return (r >> 1) & 7; }

// Per-lane coordinates inside the accumulator tile of one wavefront.
template <int NTB, int NVB>
struct LaneMap {
  int64_t tok[NTB];   // token of column q in token block tb
  int ylab[NTB];      // its label (-1 outside the batch or in argmax mode)
  int vbase[NVB];     // first of the 16 vocabulary entries in vocabulary block vb
  int hl, q, wt, wv;
};

template <int NTB, int NVB>
__device__ __forceinline__ LaneMap<NTB, NVB> lane_map(int tid, int64_t t0, int v0, int64_t n,
                                                      const int32_t* __restrict__ labels,
                                                      bool with_labels) {
  LaneMap<NTB, NVB> L;
  const int lane = tid & 63, wave = tid >> 6;
  L.wt = wave >> 1;
  L.wv = wave & 1;
  L.hl = lane >> 5;
  L.q = lane & 31;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    L.tok[tb] = t0 + L.wt * (NTB * 32) + tb * 32 + L.q;
    L.ylab[tb] = (with_labels && L.tok[tb] < n) ? labels[L.tok[tb]] : -1;
  }
#pragma unroll
  for (int vb = 0; vb < NVB; ++vb) L.vbase[vb] = v0 + L.wv * (NVB * 32) + vb * 32 + 16 * L.hl;
  return L;
}

// LDS byte offsets of this lane's operand rows (A region first, B region at
// b_base) and the XOR key of its chunk index; the K slice's chunk pair 2kk
// is XOR-ed in when reading.
template <int NTB, int NVB>
__device__ __forceinline__ void operand_offsets(const LaneMap<NTB, NVB>& L, int b_base,
                                                int (&a_row)[NVB], int (&a_x)[NVB],
                                                int (&b_row)[NTB], int (&b_x)[NTB]) {
#pragma unroll
  for (int i = 0; i < NVB; ++i) {
    const int ra = L.wv * (NVB * 32) + i * 32 + vperm(L.q);
    a_row[i] = ra * kRowBytes;
    a_x[i] = L.hl ^ swz_a(ra);
  }
#pragma unroll
  for (int i = 0; i < NTB; ++i) {
    const int rb = L.wt * (NTB * 32) + i * 32 + L.q;
    b_row[i] = b_base + rb * kRowBytes;
    b_x[i] = L.hl ^ swz_b(rb);
  }
}

template <int NTB, int NVB>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[NTB][NVB]) {
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][vb][r] = 0.f;
}

// MFMA work of one K step (one LDS stage) for the wavefront tile.  bf16:
// four K slices of 16, the fragments of slice kk + 1 requested before slice
// kk's MFMAs issue; fp32: 16 slices of 2.
template <typename T, int BK, int NTB, int NVB>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[NTB][NVB], const uint8_t* S,
                                          const int (&a_row)[NVB], const int (&a_x)[NVB],
                                          const int (&b_row)[NTB], const int (&b_x)[NTB], int hl) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 a[2][NVB], b[2][NTB];
    auto frags = [&](int kk, bf16x8(&fa)[NVB], bf16x8(&fb)[NTB]) {
#pragma unroll
      for (int i = 0; i < NVB; ++i)
        fa[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(S + a_row[i] + (((2 * kk) ^ a_x[i]) << 4)));
#pragma unroll
      for (int i = 0; i < NTB; ++i)
        fb[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(S + b_row[i] + (((2 * kk) ^ b_x[i]) << 4)));
    };
    frags(0, a[0], b[0]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) frags(kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
          acc[tb][vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][vb], b[kk & 1][tb],
                                                                acc[tb][vb], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int s = 0; s < BK / 2; ++s) {
      // this lane's K index in the step is 2s + hl: chunk (2s + hl) >> 2, word (2s + hl) & 3
      const int kidx = 2 * s + hl;
      float a[NVB], b[NTB];
#pragma unroll
      for (int i = 0; i < NVB; ++i)
        a[i] = *reinterpret_cast<const float*>(S + a_row[i] + (((kidx >> 2) ^ (a_x[i] ^ hl)) << 4) +
                                               (kidx & 3) * 4);
#pragma unroll
      for (int i = 0; i < NTB; ++i)
        b[i] = *reinterpret_cast<const float*>(S + b_row[i] + (((kidx >> 2) ^ (b_x[i] ^ hl)) << 4) +
                                               (kidx & 3) * 4);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
          acc[tb][vb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[vb], b[tb], acc[tb][vb], 0, 0, 0);
    }
  }
}

// Vocabulary entries beyond V (only in the last vocabulary tile) get a logit
// that vanishes under exp and never wins a max.
template <int NTB, int NVB>
__device__ __forceinline__ void mask_tail(f32x16 (&acc)[NTB][NVB], const LaneMap<NTB, NVB>& L,
                                          int vocab) {
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (L.vbase[vb] + r >= vocab) acc[tb][vb][r] = kMasked;
}

// Teacher weights w = exp(l_M - m_M) in (0, 1], kept in registers between the
// teacher's epilogue and the smaller exits' ones.
template <int NTB, int NVB>
struct TeacherW32 {
  float v[NTB][NVB][16];
  __device__ __forceinline__ void set2(int tb, int vb, int r, float x0, float x1) {
    v[tb][vb][r] = x0;
    v[tb][vb][r + 1] = x1;
  }
  __device__ __forceinline__ void get2(int tb, int vb, int r, float& x0, float& x1) const {
    x0 = v[tb][vb][r];
    x1 = v[tb][vb][r + 1];
  }
};
// ---------------------------------------------------------------------------
// Loss epilogue for exit e.  Two wavefront rows (wt) of NTB x 32 tokens; the
// two vocabulary wavefronts (wv) of a row are combined through LDS.  `vt` is
// the workgroup's vocabulary tile and n_vt the number of such tiles.
template <typename T, int NTB, int NVB, bool VECSTORE, typename TW>
__device__ __forceinline__ void loss_epilogue(f32x16 (&acc)[NTB][NVB], TW& wt_,
                                              const LaneMap<NTB, NVB>& L, bool teacher, int e,
                                              int64_t n, int vocab, int64_t t0, int vt, int n_vt,
                                              void* out, float* __restrict__ stats,
                                              float* __restrict__ lab,
                                              float (&xmax)[2][2][NTB * 32],
                                              float (&xsum)[2][2][NTB * 32][2]) {
  const int hl = L.hl, q = L.q, wt = L.wt, wv = L.wv;
  // (1) row maximum over the workgroup's vocabulary tile: in registers, with
  // the lane 32 apart, then with the other vocabulary wavefront through LDS.
  // Everything below is relative to it.
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    float m0 = acc[tb][0][0], m1 = acc[tb][0][1];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int r = (vb == 0 ? 2 : 0); r < 16; r += 2) {
        m0 = fmaxf(m0, acc[tb][vb][r]);
        m1 = fmaxf(m1, acc[tb][vb][r + 1]);
      }
    float m = fmaxf(m0, m1);
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (hl == 0) xmax[wt][wv][tb * 32 + q] = m;
  }
  __syncthreads();
  float M[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) M[tb] = fmaxf(xmax[wt][0][tb * 32 + q], xmax[wt][1][tb * 32 + q]);

  // (2) sums, teacher weights, label logit, shifted copy.
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const float m = M[tb];
    const float ml = m * kLog2e;
    float s0 = 0.f, s1 = 0.f, S0 = 0.f, S1 = 0.f;
    if (teacher) {
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x0 = __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][r], kLog2e, -ml));
          const float x1 = __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][r + 1], kLog2e, -ml));
          wt_.set2(tb, vb, r, x0, x1);
          s0 += x0;
          s1 += x1;
        }
    } else {
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          s0 += __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][r], kLog2e, -ml));
          s1 += __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][r + 1], kLog2e, -ml));
          float w0, w1;
          wt_.get2(tb, vb, r, w0, w1);
          S0 = fmaf(w0, acc[tb][vb][r], S0);
          S1 = fmaf(w1, acc[tb][vb][r + 1], S1);
        }
    }
    float s = s0 + s1, S = S0 + S1;
    s += __shfl_xor(s, 32, 64);
    S += __shfl_xor(S, 32, 64);

    // the label's logit: exactly one lane in the grid holds (token, y)
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const int dd = L.ylab[tb] - L.vbase[vb];
      if (static_cast<unsigned>(dd) < 16u && L.ylab[tb] < vocab) {
        float val = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) val = (r == dd) ? acc[tb][vb][r] : val;
        lab[static_cast<int64_t>(e) * n + L.tok[tb]] = val;
      }
    }
    // tile-shifted logits l - M into the gradient buffer (codec Scratch<T>)
    if (out != nullptr && L.tok[tb] < n) {
      T* orow = static_cast<T*>(out) + L.tok[tb] * vocab;
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        if (VECSTORE && L.vbase[vb] + 16 <= vocab) {
          u32x4* dst = reinterpret_cast<u32x4*>(orow + L.vbase[vb]);
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              u32x4 pk;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                pk[j] = Scratch<T>::pack2(acc[tb][vb][8 * h2 + 2 * j] - m, acc[tb][vb][8 * h2 + 2 * j + 1] - m);
              dst[h2] = pk;
            }
          } else {
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4) {
              u32x4 pk;
#pragma unroll
              for (int j = 0; j < 4; ++j) pk[j] = __float_as_uint(acc[tb][vb][4 * h4 + j] - m);
              dst[h4] = pk;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (L.vbase[vb] + r < vocab) orow[L.vbase[vb] + r] = Scratch<T>::encode(acc[tb][vb][r] - m);
        }
      }
    }
    if (hl == 0) {
      xsum[wt][wv][tb * 32 + q][0] = s;
      xsum[wt][wv][tb * 32 + q][1] = S;
    }
  }
  __syncthreads();
  // (3) wave (wt, wv) adds the two vocabulary halves of the token blocks
  // tb with tb % 2 == wv.
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    if ((tb & 1) != wv || hl != 0) continue;
    const int j = tb * 32 + q;
    const int64_t tk = t0 + wt * (NTB * 32) + j;
    if (tk < n) {
      const int64_t plane = static_cast<int64_t>(n_vt) * n;
      float* st = stats + (static_cast<int64_t>(e) * 3 * n_vt + vt) * n + tk;
      st[0] = M[tb];
      st[plane] = xsum[wt][0][j][0] + xsum[wt][1][j][0];
      if (!teacher) st[2 * plane] = xsum[wt][0][j][1] + xsum[wt][1][j][1];
    }
  }
  // xmax was last read before the barrier above; xsum is next written after
  // at least one more barrier.
}

// Argmax epilogue for exit e: per token the tile's (max, lowest index) into
// `best`, and the fp32 logits into `out` if given.
template <int NTB, int NVB, bool VECSTORE>
__device__ __forceinline__ void argmax_epilogue(f32x16 (&acc)[NTB][NVB],
                                                const LaneMap<NTB, NVB>& L, int e, int64_t n,
                                                int vocab, int64_t t0, int vt, int n_vt, void* out,
                                                float* __restrict__ best,
                                                float (&xsum)[2][2][NTB * 32][2]) {
  const int hl = L.hl, q = L.q, wt = L.wt, wv = L.wv;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc[tb][vb][r] > bv) {   // ascending vocabulary: strict > keeps the lowest index
          bv = acc[tb][vb][r];
          bi = L.vbase[vb] + r;
        }
    const float ov = __shfl_xor(bv, 32, 64);
    const int oi = __shfl_xor(bi, 32, 64);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
    if (out != nullptr && L.tok[tb] < n) {
      float* orow = static_cast<float*>(out) + L.tok[tb] * vocab;
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        if (VECSTORE && L.vbase[vb] + 16 <= vocab && (vocab & 3) == 0) {
          u32x4* dst = reinterpret_cast<u32x4*>(orow + L.vbase[vb]);
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
            if (L.vbase[vb] + r < vocab) orow[L.vbase[vb] + r] = acc[tb][vb][r];
        }
      }
    }
    if (hl == 0) {
      xsum[wt][wv][tb * 32 + q][0] = bv;
      xsum[wt][wv][tb * 32 + q][1] = __int_as_float(bi);
    }
  }
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    if ((tb & 1) != wv || hl != 0) continue;
    const int j = tb * 32 + q;
    float bv = xsum[wt][0][j][0];
    int bi = __float_as_int(xsum[wt][0][j][1]);
    const float ov = xsum[wt][1][j][0];
    const int oi = __float_as_int(xsum[wt][1][j][1]);
    if (ov > bv) {   // the second half holds higher indices: ties keep the first
      bv = ov;
      bi = oi;
    }
    const int64_t tk = t0 + wt * (NTB * 32) + j;
    if (tk < n) {
      const int64_t plane = static_cast<int64_t>(n_vt) * n;
      float* b = best + (static_cast<int64_t>(e) * 2 * n_vt + vt) * n + tk;
      b[0] = bv;
      b[plane] = __int_as_float(bi);
    }
  }
}

// ---------------------------------------------------------------------------
// Generic kernel: any widths and vocabulary, bf16 or fp32.
template <typename T>
__device__ __forceinline__ u32x4 load_chunk_zero(const T* __restrict__ P, int64_t row, int64_t rows,
                                                 int k, int D) {
  constexpr int C = Elem<T>::kChunk;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (row < rows && k < D) {
    const T* p = P + row * D + k;
    if (k + C <= D && (D % C) == 0) {
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

template <typename T, int MODE, bool VECSTORE>
__global__ __launch_bounds__(kGenThreads, 2) void heads_kernel_generic(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    const int32_t* __restrict__ labels, float* __restrict__ stats, float* __restrict__ lab,
    int n_tt, int n_vt) {
  // The exit table is the first kernel argument; indexing it through the
  // kernarg segment pointer turns a per-exit lookup into one scalar load.
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int C = Elem<T>::kChunk;
  constexpr int BK = KStep<T>::v;
  constexpr int NTB = 2, NVB = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kGenStage];
  __shared__ float xmax[2][2][NTB * 32];
  __shared__ float xsum[2][2][NTB * 32][2];

  const int tid = threadIdx.x;
  int tt, vt;
  tile_coords(blockIdx.x, n_tt, n_vt, kGroupGen, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kGenTok;
  const int v0 = vt * kGenVoc;
  const auto L = lane_map<NTB, NVB>(tid, t0, v0, n, labels, MODE == kModeLoss);
  int a_row[NVB], a_x[NVB], b_row[NTB], b_x[NTB];
  operand_offsets(L, kGenVoc * kRowBytes, a_row, a_x, b_row, b_x);

  f32x16 acc[NTB][NVB];
  TeacherW32<NTB, NVB> wt_;   // teacher weights exp(l_M - m_M) (loss mode)

  for (int ei = 0; ei < n_exits; ++ei) {
    const int e = (MODE == kModeLoss) ? (ei == 0 ? n_exits - 1 : ei - 1) : ei;
    const bool teacher = (MODE == kModeLoss) && ei == 0;
    const int D = ex.d[e];
    const T* __restrict__ H = static_cast<const T*>(ex.h[e]);
    const T* __restrict__ W = static_cast<const T*>(ex.w[e]);
    zero_acc(acc);

    u32x4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qd = tid + kGenThreads * j;
        const int row = qd >> 3, c = qd & 7;
        ra[j] = load_chunk_zero<T>(W, v0 + row, vocab, k0 + c * C, D);
        rb[j] = load_chunk_zero<T>(H, t0 + row, n, k0 + c * C, D);
      }
    };
    auto sstore = [&](int buf) {
      uint8_t* A = lds + buf * kGenStage;
      uint8_t* B = A + kGenVoc * kRowBytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qd = tid + kGenThreads * j;
        const int row = qd >> 3, c = qd & 7;
        *reinterpret_cast<u32x4*>(A + row * kRowBytes + ((c ^ swz_a(row)) << 4)) = ra[j];
        *reinterpret_cast<u32x4*>(B + row * kRowBytes + ((c ^ swz_b(row)) << 4)) = rb[j];
      }
    };
    const int nk = (D + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk) gload((ks + 1) * BK);
      mfma_step<T, BK>(acc, lds + (ks & 1) * kGenStage, a_row, a_x, b_row, b_x, L.hl);
      if (ks + 1 < nk) sstore((ks + 1) & 1);
      __syncthreads();
    }
    if (v0 + kGenVoc > vocab) mask_tail(acc, L, vocab);
    if constexpr (MODE == kModeLoss)
      loss_epilogue<T, NTB, NVB, VECSTORE>(acc, wt_, L, teacher, e, n, vocab, t0, vt, n_vt,
                                           ex.out[e], stats, lab, xmax, xsum);
    else
      argmax_epilogue<NTB, NVB, VECSTORE>(acc, L, e, n, vocab, t0, vt, n_vt, ex.out[e], stats,
                                          xsum);
  }
}

template <typename T, int MODE>
hipError_t launch_heads(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                        const int32_t* labels, float* stats, float* lab, TileInfo* info,
                        hipStream_t s) {
  info->vtile = kGenVoc;
  info->teacher_w16 = false;
  if (n == 0) return hipSuccess;
  constexpr int C = Elem<T>::kChunk;
  const int n_tt = static_cast<int>((n + kGenTok - 1) / kGenTok);
  const int n_vt = (vocab + kGenVoc - 1) / kGenVoc;
  if (vocab % C == 0)
    hipLaunchKernelGGL((heads_kernel_generic<T, MODE, true>), dim3(n_tt * n_vt), dim3(kGenThreads),
                       0, s, ex, n_exits, n, vocab, labels, stats, lab, n_tt, n_vt);
  else
    hipLaunchKernelGGL((heads_kernel_generic<T, MODE, false>), dim3(n_tt * n_vt),
                       dim3(kGenThreads), 0, s, ex, n_exits, n, vocab, labels, stats, lab, n_tt,
                       n_vt);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_heads_loss(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                             const int32_t* labels, float* stats, float* lab, TileInfo* info,
                             hipStream_t s) {
  return launch_heads<T, kModeLoss>(n_exits, n, vocab, ex, labels, stats, lab, info, s);
}

template <typename T>
hipError_t launch_heads_argmax(int n_exits, int64_t n, int vocab, const ExitSet& ex, float* best,
                               TileInfo* info, hipStream_t s) {
  return launch_heads<T, kModeArgmax>(n_exits, n, vocab, ex, nullptr, best, nullptr, info, s);
}

template hipError_t launch_heads_loss<bf16_t>(int, int64_t, int, const ExitSet&, const int32_t*,
                                              float*, float*, TileInfo*, hipStream_t);
template hipError_t launch_heads_loss<float>(int, int64_t, int, const ExitSet&, const int32_t*,
                                             float*, float*, TileInfo*, hipStream_t);
template hipError_t launch_heads_argmax<bf16_t>(int, int64_t, int, const ExitSet&, float*, TileInfo*,
                                                hipStream_t);
template hipError_t launch_heads_argmax<float>(int, int64_t, int, const ExitSet&, float*, TileInfo*,
                                               hipStream_t);

}  // namespace nel
