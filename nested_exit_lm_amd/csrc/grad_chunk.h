// Logit gradients of one 8-entry chunk of a token row, formed from the fp16
// scratch the packed loss GEMM leaves behind (device side; shared by the
// in-place gradient pass and the backward GEMMs that consume the gradient
// without it ever being stored).
//
// Loss ("Matryoshka Language Model Suites", distillation paragraph; teacher
// M = last exit under stop-gradient, p = softmax(l_M)): for a smaller exit
//     g_v = ge (q_v - a p_v - (1 - a) [v = y]),   q = softmax(l),
// and for the teacher g_v = ge_M (p_v - [v = y]), with ge = gs lambda_e (the
// upstream gradient times the exit's weight).  The scratch holds, per
// 256-entry vocabulary tile with maximum m: the teacher's weights
// w = exp(l_M - m_M) and a smaller exit's s = l - m, so with
// sc = exp(m_M - LSE_M) and c1 = (m - LSE) log2 e, p_v = w_v sc and
// q_v = 2^(s_v log2 e + c1).
//
// The magnitude |ge| is folded into three constants per (exit, tile, token):
//     c   = c1 + log2 |ge|     (the teacher: -inf, no softmax term of its own)
//     k   = -a |ge| sc         (the teacher: |ge| sc)
//     lab = -(1 - a) |ge|      (the teacher: -|ge|), added at the label
// so that |ge|-scaled gradients cost one exponential and two fused
// multiply-adds per entry:  g_v = fma(w_v, k, 2^fma(s_v, log2 e, c)) [+ lab].
// The sign of ge is applied to the bf16 results (an exact flip), so every
// consumer sees the same operand bits (a GEMM that negated its sums instead
// would not round like one that sums the negated gradients).
//
// Every caller must round identically, so the arithmetic is spelled out with
// explicit fused multiply-adds and nothing else may be contracted.
#pragma once
#include "common.h"

namespace nel {

// One 16-byte row constant record per (exit, vocabulary tile, token); NaN
// constants for a token whose label is outside the vocabulary.
struct GradRowConst {
  float c, k, lab;
  int32_t y;
};

// Per (exit, token): gabs = |gs lambda_e| (NaN for a bad label).
struct GradExitRow {
  float lg, ka, lab;   // log2 gabs; k / sc; the label's term
};

__device__ __forceinline__ GradExitRow grad_exit_row(bool teacher, float gabs, float alpha) {
#pragma clang fp contract(off)
  GradExitRow r;
  r.lg = log2f(gabs);
  r.ka = teacher ? gabs : -alpha * gabs;
  r.lab = teacher ? -gabs : -((1.f - alpha) * gabs);
  return r;
}

// The tile constants from the exit's tile maximum mt and LSE, and the
// teacher's sc of the same tile.
__device__ __forceinline__ float grad_tile_c(bool teacher, const GradExitRow& r, float mt,
                                             float lse) {
#pragma clang fp contract(off)
  return teacher ? -INFINITY : fmaf(mt - lse, kLog2e, r.lg);
}
__device__ __forceinline__ float grad_tile_k(const GradExitRow& r, float sc) {
#pragma clang fp contract(off)
  return r.ka * sc;
}

// The label's position relative to a chunk's first entry v0, wrapping for
// any label (a bad one included) instead of overflowing.
__device__ __forceinline__ int label_offset(uint32_t y, int v0) {
  return static_cast<int>(y - static_cast<uint32_t>(v0));
}
__device__ __forceinline__ int label_offset(int32_t y, int v0) {
  return label_offset(static_cast<uint32_t>(y), v0);
}

// s, w: the chunk's 8 fp16 scratch entries of the exit and of the teacher
// (the teacher passes its own w as s, with c = -inf so that 2^-inf = +0 and
// g = fma(w, k, +0) = w k rounded once); yi: the label's position in the
// chunk (y - first entry), acted on only when 0 <= yi < 8, which holds for
// one chunk of a row, so the wavefront skips that step unless one of its
// lanes needs it.  neg: 0x80008000 to store -g (the sign of ge), else 0.
// Every lane of the wavefront that is active at the call must call it.
__device__ __forceinline__ u32x4 grad_chunk(const u32x4& s, const u32x4& w, float c, float k,
                                            float lab, int yi, uint32_t neg = 0u) {
#pragma clang fp contract(off)
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = __builtin_amdgcn_exp2f(fmaf(Scratch<bf16_t>::get(s, i), kLog2e, c));
    g[i] = fmaf(Scratch<bf16_t>::get(w, i), k, q);
  }
  const bool here = static_cast<unsigned>(yi) < 8u;
  if (__builtin_amdgcn_ballot_w64(here) != 0) {
    asm volatile("");   // keeps the block a branch (not speculated into selects)
    if (here) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i == yi) g[i] = g[i] + lab;
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(g[2 * j], g[2 * j + 1]) ^ neg;
  return o;
}

// The teacher's chunk without the exponential: bit for bit grad_chunk(w, w,
// -inf, k, lab, yi, neg).
__device__ __forceinline__ u32x4 grad_chunk_teacher(const u32x4& w, float k, float lab, int yi,
                                                    uint32_t neg = 0u) {
#pragma clang fp contract(off)
  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = fmaf(Scratch<bf16_t>::get(w, i), k, 0.f);
  const bool here = static_cast<unsigned>(yi) < 8u;
  if (__builtin_amdgcn_ballot_w64(here) != 0) {
    asm volatile("");   // keeps the block a branch (not speculated into selects)
    if (here) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i == yi) g[i] = g[i] + lab;
    }
  }
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(g[2 * j], g[2 * j + 1]) ^ neg;
  return o;
}

}  // namespace nel
