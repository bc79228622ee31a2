// Logit gradients of one 8-entry chunk of a token row, formed from the fp16
// scratch the packed loss GEMM leaves behind (device side; shared by the
// in-place gradient pass and the backward GEMMs that consume the gradient
// without it ever being stored).
//
// Loss ("Matryoshka Language Model Suites", distillation paragraph; teacher
// M = last exit under stop-gradient, p = softmax(l_M)): for a smaller exit
//     g_v = gs lambda (q_v - a p_v - (1 - a) [v = y]),   q = softmax(l)
// and for the teacher g_v = gs lambda_M (p_v - [v = y]).  The scratch holds,
// per 256-entry vocabulary tile with maximum m: the teacher's weights
// w = exp(l_M - m_M) and a smaller exit's s = l - m.  With the row constants
//     sc = exp(m_M - LSE_M),   c1 = (m - LSE) log2 e
// p_v = w_v sc and q_v = 2^(s_v log2 e + c1).
//
// Both callers must round identically, so the arithmetic is spelled out with
// explicit fused multiply-adds and nothing else may be contracted.
#pragma once
#include "common.h"

namespace nel {

// One 16-byte row constant record per (exit, vocabulary tile, token): the
// smaller exit's c1, the teacher's sc, the label as raw bits (NaN c1 and sc
// for a token whose label is outside the vocabulary).
struct GradRowConst {
  float c1, sc;
  int32_t y, pad;
};

// s, w: the chunk's 8 fp16 scratch entries of the exit and of the teacher;
// yi: the label's position in the chunk (y - first entry), acted on only
// when 0 <= yi < 8.  Returns the 8 gradients as bf16 pairs.
__device__ __forceinline__ u32x4 grad_chunk_student(const u32x4& s, const u32x4& w, float sc,
                                                    float c1, float ge, float alpha, int yi) {
#pragma clang fp contract(off)
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = Scratch<bf16_t>::get(w, i) * sc;
    const float q = __builtin_amdgcn_exp2f(fmaf(Scratch<bf16_t>::get(s, i), kLog2e, c1));
    g[i] = ge * fmaf(-alpha, p, q);
  }
  if (static_cast<unsigned>(yi) < 8u) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i == yi) g[i] = fmaf(-ge, 1.f - alpha, g[i]);
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(g[2 * j], g[2 * j + 1]);
  return o;
}

__device__ __forceinline__ u32x4 grad_chunk_teacher(const u32x4& w, float sc, float gt, int yi) {
#pragma clang fp contract(off)
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = gt * (Scratch<bf16_t>::get(w, i) * sc);
  if (static_cast<unsigned>(yi) < 8u) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i == yi) g[i] = g[i] - gt;
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(g[2 * j], g[2 * j + 1]);
  return o;
}

}  // namespace nel
