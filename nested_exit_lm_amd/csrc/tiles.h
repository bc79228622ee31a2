// Tile geometry shared by the head-GEMM kernels (device side).
#pragma once
#include "common.h"

namespace nel {

constexpr float kMasked = -1.0e30f;   // logit of a vocabulary entry beyond V
// Loss epilogues: kModeLoss (row-major GEMM) forms the teacher-weighted sums
// in the epilogue; the packed GEMM's kModeLossPlain stores l - m in fp16 for
// every exit and kModeLossF16 the teacher's weights and the smaller exits'
// l - m in fp16 (sums formed by the gradient pass).
enum { kModeLoss = 0, kModeArgmax = 1, kModeLossPlain = 2, kModeLossF16 = 3 };

// A-row q of a 32-row MFMA block holds vocabulary entry vperm(q), chosen so
// that accumulator register r of lane half h is vocabulary entry 16h + r
// (the 32x32x16 accumulator puts rows 8(r/4) + 4h + r%4 in lane half h).
__device__ __forceinline__ int vperm(int q) { return ((q >> 2) & 1) * 16 + (q >> 3) * 4 + (q & 3); }
// Its inverse: the A-row that holds vocabulary entry p of the block.
__host__ __device__ inline int vperm_inv(int p) {
  return (((p >> 2) & 3) << 3) | (((p >> 4) & 1) << 2) | (p & 3);
}

// Workgroup id -> (token tile, vocabulary tile).  Consecutive ids are spread
// over the 8 XCDs, so ids are first regrouped per XCD; each XCD then walks
// groups of `group` token tiles across the vocabulary, so the workgroups
// resident on one XCD share a few token and vocabulary operand panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int n_tt, int n_vt, int group, int& tt,
                                            int& vt) {
  const int G = n_tt * n_vt;
  int L = bid;
  if ((G & 7) == 0) L = (bid & 7) * (G >> 3) + (bid >> 3);
  const int per_group = group * n_vt;
  const int g = L / per_group;
  const int first = g * group;
  const int gs = min(n_tt - first, group);
  const int r = L - g * per_group;
  tt = first + r % gs;
  vt = r / gs;
}

}  // namespace nel
