// Row merge of the head GEMM's per-tile statistics, the token means, the
// in-place logit-gradient finalisation, the argmax merge and greedy
// acceptance.
//
// Loss ("Matryoshka Language Model Suites", distillation and limitations
// paragraphs; follow-up 4 of "Is nesting the cheapest way to build a model
// suite?" for the 0.7 / 0.3 mix), teacher M = last exit, p = softmax(l_M):
//     CE_m = LSE_m - l_m[y],  Dist_m = LSE_m - sum_v p_v l_m,v   (m < M)
//     L_m = (1 - a) CE_m + a Dist_m (m < M),  L_M = CE_M,  total = sum_m L_m
// From the tiles: LSE = online log-sum-exp of (m_tile, sigma_tile) and
// sum_v p_v l_m,v = sum_tiles exp(m_M,tile - LSE_M) S_m,tile.
// Gradient (teacher under stop-gradient), written over the tile-shifted
// logits s = l - m_tile the GEMM left in the caller's buffers:
//     m < M: gs (exp(s_m + m_m,tile - LSE_m) - a p - (1 - a) [v = y])
//     M:     gs (p - [v = y]),   p = exp(s_M + m_M,tile - LSE_M)
// Exit weights lambda (limitations paragraph: reweighting the per-exit
// losses) scale exit m's gradient and its share of the total.
// Other divergences D(p, q) in place of the cross-entropy to the teacher
// (follow-up 4: reverse KL, Jensen-Shannon, an acceptance loss read as the
// total variation 1 - sum min(p, q)) need p and q per entry after the row's
// LSE is known: div_stats_kernel reads the stored s of the teacher and each
// student and reduces D and the gradient's row constant K = sum_v q_v r_v,
// r = dD/dq; the student gradient is then
//     gs lambda_m ((1 - a)(q - [v = y]) + a q (r - K)).
#include <limits.h>

#include "common.h"
#include "grad_chunk.h"
#include "internal.h"

namespace nel {

namespace {

// ---------------------------------------------------------------- loss merge
// 1024 threads = 64 tokens x kMergeGroups tile groups (group g takes tiles
// g, g + kMergeGroups, ...); the groups are merged in LDS in a fixed order,
// so results do not depend on scheduling.  The first wavefront
// (one lane per token) also reduces the workgroup's per-token values into
// fp64 partial sums of the reported means, in a fixed butterfly order:
// partials[block][q], q = CE_0.., Dist_0.., L_0.., total.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

constexpr int kMergeGroups = 16;
constexpr int kMergeBatch = 8;    // tiles whose loads a merge thread issues together

template <int N>
__device__ __forceinline__ float group_tree(const float (*sh)[64][2], int tl) {
  if constexpr (N == 1)
    return sh[0][tl][0];
  else
    return group_tree<N / 2>(sh, tl) + group_tree<N / 2>(sh + N / 2, tl);
}

__global__ __launch_bounds__(1024) void loss_merge_kernel(int M, int64_t n, int vocab,
                                                         const int32_t* __restrict__ labels,
                                                         float alpha,
                                                         const float* __restrict__ stats,
                                                         const float* __restrict__ lab,
                                                         float* __restrict__ lse_out,
                                                         float* __restrict__ tokloss,
                                                         double* __restrict__ partials,
                                                         int32_t* __restrict__ flags, int n_vt,
                                                         ExitW lam, int skip_dist) {
  __shared__ float sh[kMergeGroups][64][2];
  const int tl = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMergeTok + tl;
  const bool valid = t < n;
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const int y = valid ? labels[t] : 0;
  const bool bad = y < 0 || y >= vocab;
  if (g == 0 && valid && bad && flags) atomicOr(flags, 2 /*NEL_FLAG_BAD_LABEL*/);
  double* part = partials + static_cast<int64_t>(blockIdx.x) * (3 * M + 1);
  const float* stT = stats + static_cast<int64_t>(M - 1) * 3 * plane + t;
  float lseT = 0.f;
  double total = 0.0;
  for (int ei = 0; ei < M; ++ei) {
    const int e = ei == 0 ? M - 1 : ei - 1;
    const float* st = stats + static_cast<int64_t>(e) * 3 * plane + t;
    // a thread's tiles vt = g + kMergeGroups i in ascending order, their
    // loads issued kMergeBatch at a time (past the last tile: re-reads, unused)
    float m = -INFINITY, s = 0.f;
    if (valid)
      for (int vt0 = g; vt0 < n_vt; vt0 += kMergeBatch * kMergeGroups) {
        float mm[kMergeBatch], ss[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          const int64_t o = static_cast<int64_t>(min(vt0 + k * kMergeGroups, n_vt - 1)) * n;
          mm[k] = st[o];
          ss[k] = st[plane + o];
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k)
          if (vt0 + k * kMergeGroups < n_vt) lse_merge(m, s, mm[k], ss[k]);
      }
    sh[g][tl][0] = m;
    sh[g][tl][1] = s;
    __syncthreads();
    float Mx = -INFINITY, Sx = 0.f;
#pragma unroll
    for (int gg = 0; gg < kMergeGroups; ++gg) lse_merge(Mx, Sx, sh[gg][tl][0], sh[gg][tl][1]);
    __syncthreads();
    const float L = Mx + flog(Sx);
    if (ei == 0) lseT = L;
    float dist = 0.f;
    if (ei > 0 && !skip_dist) {   // (otherwise div_finish_kernel supplies Dist)
      float a = 0.f;
      if (valid)
        for (int vt0 = g; vt0 < n_vt; vt0 += kMergeBatch * kMergeGroups) {
          float mt[kMergeBatch], ws[kMergeBatch];
#pragma unroll
          for (int k = 0; k < kMergeBatch; ++k) {
            const int64_t o = static_cast<int64_t>(min(vt0 + k * kMergeGroups, n_vt - 1)) * n;
            mt[k] = stT[o];
            ws[k] = st[2 * plane + o];
          }
#pragma unroll
          for (int k = 0; k < kMergeBatch; ++k)
            if (vt0 + k * kMergeGroups < n_vt) a = fmaf(fexp(mt[k] - lseT), ws[k], a);
        }
      sh[g][tl][0] = a;
      __syncthreads();
      const float T = group_tree<kMergeGroups>(sh, tl);
      __syncthreads();
      dist = L - T;
    }
    if (g == 0) {   // wavefront-uniform branch: the 64 token lanes
      float ce = L - ((bad || !valid) ? 0.f : lab[static_cast<int64_t>(e) * n + t]);
      float lm = (ei == 0) ? ce : (1.f - alpha) * ce + alpha * dist;
      float lse = L;
      if (bad) ce = dist = lm = lse = __builtin_nanf("");
      if (valid) {
        lse_out[static_cast<int64_t>(e) * n + t] = lse;
        tokloss[(static_cast<int64_t>(e) * 3 + 0) * n + t] = ce;
        tokloss[(static_cast<int64_t>(e) * 3 + 1) * n + t] = dist;
        tokloss[(static_cast<int64_t>(e) * 3 + 2) * n + t] = lm;
      }
      const double sce = wave_sum_f64(valid ? static_cast<double>(ce) : 0.0);
      const double sdi = wave_sum_f64(valid ? static_cast<double>(dist) : 0.0);
      const double slm = wave_sum_f64(valid ? static_cast<double>(lm) : 0.0);
      total += valid ? static_cast<double>(lam.w[e]) * lm : 0.0;
      if (tl == 0) {
        part[e] = sce;
        part[M + e] = sdi;
        part[2 * M + e] = slm;
      }
    }
  }
  if (g == 0) {
    const double st = wave_sum_f64(total);
    if (tl == 0) part[3 * M] = st;
  }
}

// ---------------------------------------------------------------- means
// Means from the merge's partial sums: thread i of the workgroup adds the
// partials of blocks i, i + 256, ... and the 256 results are combined in a
// fixed tree, so the means do not depend on scheduling.
__global__ __launch_bounds__(256) void loss_means_kernel(int M, int64_t n, int64_t nblk,
                                                         const double* __restrict__ partials,
                                                         float* __restrict__ means) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int qi = 0; qi <= 3 * M; ++qi) {
    double a = 0.0;
    for (int64_t b = tid; b < nblk; b += 256) a += partials[b * (3 * M + 1) + qi];
    a = wave_sum_f64(a);
    if (lane == 0) red[wave] = a;
    __syncthreads();
    if (tid == 0)
      means[qi] = n > 0 ? static_cast<float>(((red[0] + red[1]) + (red[2] + red[3])) /
                                             static_cast<double>(n))
                        : 0.f;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- divergences
// The exits' gradient buffers (dlogits), by value.
struct DlPtrs {
  void* p[kMaxExits];
};

// Per entry of one token row, given the teacher's and a student's log-probs
// (lp, lq) and probabilities (p, q): the divergence term d and q_v r_v.
// log m, m = (p + q) / 2, for the Jensen-Shannon terms: from the
// probabilities while their sum is a normal float (one logarithm), else from
// the log-probabilities, which stays finite where both underflow.
__device__ __forceinline__ float js_log_mix(float lp, float lq, float p, float q) {
  const float s = p + q;
  if (s >= 0x1p-100f) return flog(s) - kLn2;
  const float hi = fmaxf(lp, lq), lo = fminf(lp, lq);
  return hi + flog(1.f + fexp(lo - hi)) - kLn2;
}

template <int DIV>
__device__ __forceinline__ void div_terms(float lp, float lq, float p, float q, float& d,
                                          float& qr) {
  if constexpr (DIV == kDivReverseKL) {
    d = q * (lq - lp);   // r = log q - log p (+ 1, which K cancels)
    qr = d;
  } else if constexpr (DIV == kDivJS) {
    const float lm = js_log_mix(lp, lq, p, q);
    d = 0.5f * (p * (lp - lm) + q * (lq - lm));
    qr = 0.5f * q * (lq - lm);
  } else {   // kDivTV
    d = 0.5f * fabsf(p - q);
    qr = q > p ? 0.5f * q : (q < p ? -0.5f * q : 0.f);
  }
}

template <int DIV>
__device__ __forceinline__ float div_r(float lp, float lq, float p, float q) {
  if constexpr (DIV == kDivReverseKL) {
    return lq - lp;
  } else if constexpr (DIV == kDivJS) {
    return 0.5f * (lq - js_log_mix(lp, lq, p, q));
  } else {
    return q > p ? 0.5f : (q < p ? -0.5f : 0.f);
  }
}

// One workgroup per token row (grid-stride): for every student e < M - 1,
// dv[e][t] = D(p, q_e) and kv[e][t] = K, each a per-thread fp32 sum in
// vocabulary order combined in a fixed tree.  The stored s are read, not
// modified (the teacher's as shifted logits: never the fp16 weight form).
template <typename T, int DIV>
__global__ __launch_bounds__(256) void div_stats_kernel(int M, int64_t n, int vocab, int vtile,
                                                        const float* __restrict__ stats,
                                                        const float* __restrict__ lse, DlPtrs dl,
                                                        int n_vt, float* __restrict__ dv,
                                                        float* __restrict__ kv) {
  constexpr int C = Elem<T>::kChunk;
  __shared__ float red[4][2 * (kMaxExits - 1)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const int S = M - 1;
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x) {
    float D[kMaxExits - 1], K[kMaxExits - 1];
#pragma unroll
    for (int e = 0; e < kMaxExits - 1; ++e) D[e] = K[e] = 0.f;
    auto off = [&](int e, int tile) {
      return stats[static_cast<int64_t>(e) * 3 * plane + static_cast<int64_t>(tile) * n + t] -
             lse[static_cast<int64_t>(e) * n + t];
    };
    if (vocab % C == 0) {
      const int64_t cpr = vocab / C;
      for (int64_t c = tid; c < cpr; c += 256) {
        const int tile = static_cast<int>(c * C) / vtile;
        const u32x4 tr = reinterpret_cast<const u32x4*>(static_cast<const T*>(dl.p[M - 1]) + t * vocab)[c];
        const float oT = off(M - 1, tile);
        float lp[C], p[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
          lp[i] = Scratch<T>::get(tr, i) + oT;
          p[i] = fexp(lp[i]);
        }
#pragma unroll
        for (int e = 0; e < kMaxExits - 1; ++e) {
          if (e >= S) break;
          const u32x4 sr = reinterpret_cast<const u32x4*>(static_cast<const T*>(dl.p[e]) + t * vocab)[c];
          const float oe = off(e, tile);
#pragma unroll
          for (int i = 0; i < C; ++i) {
            const float lq = Scratch<T>::get(sr, i) + oe;
            float d, qr;
            div_terms<DIV>(lp[i], lq, p[i], fexp(lq), d, qr);
            D[e] += d;
            K[e] += qr;
          }
        }
      }
    } else {
      for (int v = tid; v < vocab; v += 256) {
        const int tile = v / vtile;
        const float lp = Scratch<T>::load(static_cast<const T*>(dl.p[M - 1]) + t * vocab + v) + off(M - 1, tile);
        const float p = fexp(lp);
        for (int e = 0; e < S; ++e) {
          const float lq = Scratch<T>::load(static_cast<const T*>(dl.p[e]) + t * vocab + v) + off(e, tile);
          float d, qr;
          div_terms<DIV>(lp, lq, p, fexp(lq), d, qr);
          D[e] += d;
          K[e] += qr;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kMaxExits - 1; ++e) {
      if (e >= S) break;
      const float a = wave_sum(D[e]), b = wave_sum(K[e]);
      if (lane == 0) {
        red[wave][2 * e] = a;
        red[wave][2 * e + 1] = b;
      }
    }
    __syncthreads();
    if (tid < 2 * S) {
      const float x = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
      ((tid & 1) ? kv : dv)[static_cast<int64_t>(tid >> 1) * n + t] = x;
    }
    __syncthreads();   // red is reused by the next row
  }
}

// Losses and mean partials once D is known (the merge's tail with Dist from
// dv): one wavefront per kMergeTok tokens, the same partial layout and order.
__global__ __launch_bounds__(64) void div_finish_kernel(int M, int64_t n, float alpha,
                                                        const float* __restrict__ dv,
                                                        float* __restrict__ tokloss,
                                                        double* __restrict__ partials, ExitW lam) {
  const int tl = threadIdx.x;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kMergeTok + tl;
  const bool valid = t < n;
  double* part = partials + static_cast<int64_t>(blockIdx.x) * (3 * M + 1);
  double total = 0.0;
  for (int ei = 0; ei < M; ++ei) {
    const int e = ei == 0 ? M - 1 : ei - 1;
    float ce = 0.f, dist = 0.f, lm = 0.f;
    if (valid) {
      ce = tokloss[(static_cast<int64_t>(e) * 3 + 0) * n + t];
      dist = ei == 0 ? 0.f : dv[static_cast<int64_t>(e) * n + t];
      if (ce != ce) dist = ce;   // a bad label (NaN) stays NaN
      lm = ei == 0 ? ce : (1.f - alpha) * ce + alpha * dist;
      tokloss[(static_cast<int64_t>(e) * 3 + 1) * n + t] = dist;
      tokloss[(static_cast<int64_t>(e) * 3 + 2) * n + t] = lm;
    }
    const double sce = wave_sum_f64(valid ? static_cast<double>(ce) : 0.0);
    const double sdi = wave_sum_f64(valid ? static_cast<double>(dist) : 0.0);
    const double slm = wave_sum_f64(valid ? static_cast<double>(lm) : 0.0);
    total += valid ? static_cast<double>(lam.w[e]) * lm : 0.0;
    if (tl == 0) {
      part[e] = sce;
      part[M + e] = sdi;
      part[2 * M + e] = slm;
    }
  }
  const double st = wave_sum_f64(total);
  if (tl == 0) part[3 * M] = st;
}

// ---------------------------------------------------------------- finalize

// 16-byte chunk path (vocab a multiple of the chunk).  Each workgroup
// iteration covers 256 consecutive chunks of one token row for all exits.
template <typename T, int DIV>
__global__ __launch_bounds__(256) void finalize_vec(int M, int64_t n, int vocab, int vtile,
                                                    const int32_t* __restrict__ labels, float alpha,
                                                    float gs, const float* __restrict__ stats,
                                                    const float* __restrict__ lse, DlPtrs dl,
                                                    int n_vt, int segs_per_row,
                                                    const float* __restrict__ kv, ExitW lam) {
  constexpr int C = Elem<T>::kChunk;
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const int64_t cpr = vocab / C;
  const int64_t nseg = n * segs_per_row;
  for (int64_t seg = blockIdx.x; seg < nseg; seg += gridDim.x) {
    const int64_t t = seg / segs_per_row;
    const int64_t c = static_cast<int64_t>(seg - t * segs_per_row) * 256 + threadIdx.x;
    if (c >= cpr) continue;
    const int v0 = static_cast<int>(c * C);
    const int tile = v0 / vtile;
    const int y = labels[t];
    const bool bad = y < 0 || y >= vocab;
    u32x4 raw[kMaxExits];
#pragma unroll
    for (int e = 0; e < kMaxExits; ++e)
      if (e < M) raw[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                             static_cast<const T*>(dl.p[e]) + t * vocab) + c);
    // The teacher's chunk in a vector of its own: every element index below is
    // a compile-time constant (no indexing of raw[] by the run-time M - 1).
    const u32x4 traw = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const T*>(dl.p[M - 1]) + t * vocab) + c);
    float p[C], lp[C];
    {
      const int e = M - 1;
      const float off = stats[static_cast<int64_t>(e) * 3 * plane + static_cast<int64_t>(tile) * n + t] -
                        lse[static_cast<int64_t>(e) * n + t];
#pragma unroll
      for (int i = 0; i < C; ++i) {
        lp[i] = Scratch<T>::get(traw, i) + off;
        p[i] = fexp(lp[i]);
      }
    }
#pragma unroll
    for (int e = 0; e < kMaxExits; ++e) {
      if (e >= M) break;
      const bool teacher = e == M - 1;
      const float off = stats[static_cast<int64_t>(e) * 3 * plane + static_cast<int64_t>(tile) * n + t] -
                        lse[static_cast<int64_t>(e) * n + t];
      const float hot = teacher ? 1.f : 1.f - alpha;
      const float ge = gs * lam.w[e];
      float kc = 0.f;
      if constexpr (DIV != kDivForward)
        if (!teacher) kc = kv[static_cast<int64_t>(e) * n + t];
      float g[C];
#pragma unroll
      for (int i = 0; i < C; ++i) {
        float val;
        if (teacher) {
          val = p[i];
        } else {
          const float lq = Scratch<T>::get(raw[e], i) + off;
          const float q = fexp(lq);
          if constexpr (DIV == kDivForward)
            val = q - alpha * p[i];
          else
            val = (1.f - alpha) * q + alpha * q * (div_r<DIV>(lp[i], lq, p[i], q) - kc);
        }
        if (v0 + i == y) val -= hot;
        g[i] = bad ? __builtin_nanf("") : ge * val;
      }
      u32x4 o;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(g[2 * j], g[2 * j + 1]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(g[j]);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<T*>(dl.p[e]) + t * vocab) + c);
    }
  }
}

// Packed path with fp16 scratch: the teacher's buffer holds its fp16 weights
// w = exp(l_M - m), each smaller exit's its fp16 l - m (m the 256-entry tile
// maximum).  One workgroup per token row (grid-stride) writes every exit's
// gradient in place, as finalize_vec, and reduces per smaller exit
// sum_v p_v l_m,v in a fixed order (per-thread fp32 in vocabulary order, then
// a fixed tree): dv[e][t] = LSE_e - that sum, the cross-entropy to the teacher.
// Per 16-byte chunk (8 entries, one tile): p = w exp(m_M - LSE_M),
// q = exp2(s log2 e + (m_e - LSE_e) log2 e), g_e = lambda_e gs (q - a p) and
// g_M = lambda_M gs p, with the label's entry corrected only in the chunk that
// holds it; sum_v p l_e over the chunk is sum p s + m_e sum p.  A bad label
// makes the scale NaN, which turns the whole row into NaN.  The gradients
// come from grad_chunk.h (grad_exit_row per row, grad_tile_c / grad_tile_k
// per tile), shared with the backward GEMMs that form them without storing
// them; WRITE_G = false keeps the buffers as they are and computes dv only
// (for those GEMMs).
template <int MS, bool WRITE_G>   // MS: the most smaller exits the loops are unrolled for
__global__ __launch_bounds__(256) void finalize_rows_f16(int M, int64_t n, int vocab, int vshift,
                                                         const int32_t* __restrict__ labels,
                                                         float alpha, float gs,
                                                         const float* __restrict__ stats,
                                                         const float* __restrict__ lse, DlPtrs dl,
                                                         int n_vt, float* __restrict__ dv,
                                                         ExitW lam) {
  __shared__ float red[4][kMaxExits];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const int64_t cpr = vocab / 8;
  const int S = M - 1;
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x) {
    const int y = labels[t];
    const bool bad = y < 0 || y >= vocab;
    const float nanv = __builtin_nanf("");
    const float lseT = lse[static_cast<int64_t>(M - 1) * n + t];
    const float geT = gs * lam.w[M - 1];
    const GradExitRow rT = grad_exit_row(true, bad ? nanv : fabsf(geT), alpha);
    const uint32_t negT = geT < 0.f ? 0x80008000u : 0u;
    GradExitRow rE[MS];
    uint32_t negE[MS];
    float lseE[MS], acc[MS];
#pragma unroll
    for (int e = 0; e < MS; ++e) {
      acc[e] = 0.f;
      lseE[e] = 0.f;
      negE[e] = 0u;
      if (e < S) {
        const float ge = gs * lam.w[e];
        rE[e] = grad_exit_row(false, bad ? nanv : fabsf(ge), alpha);
        negE[e] = ge < 0.f ? 0x80008000u : 0u;
        lseE[e] = lse[static_cast<int64_t>(e) * n + t];
      }
    }
    // four chunks per thread per round (chunks c0 + 256 k): every exit's
    // loads of the round, and the tile statistics they need, are issued
    // before any of them is used (12 16-byte loads in flight per thread for
    // three exits).  No load sits under a condition: chunks past the row end
    // re-read its last chunk and exit slots beyond the smaller exits re-read
    // the teacher's row, and neither is used, so the compiler keeps every
    // load of the round in flight at once.
    const bf16_t* rowT = static_cast<const bf16_t*>(dl.p[M - 1]) + t * vocab;
    const float* stTp = stats + static_cast<int64_t>(M - 1) * 3 * plane + t;
    const bf16_t* rowE[MS];
    const float* stEp[MS];
#pragma unroll
    for (int e = 0; e < MS; ++e) {
      rowE[e] = static_cast<const bf16_t*>(dl.p[e < S ? e : M - 1]) + t * vocab;
      stEp[e] = stats + static_cast<int64_t>(e < S ? e : M - 1) * 3 * plane + t;
    }
    for (int64_t c0 = tid; c0 < cpr; c0 += 4 * 256) {
      u32x4 tw[4], sr[MS][4];
      float mT[4], mE[MS][4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t cl = min(c0 + 256 * k, cpr - 1);
        const int64_t tile = (cl * 8) >> vshift;   // the tile width is a power of 2
        tw[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowT) + cl);
#pragma unroll
        for (int e = 0; e < MS; ++e)
          sr[e][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowE[e]) + cl);
        mT[k] = stTp[tile * n];
#pragma unroll
        for (int e = 0; e < MS; ++e) mE[e][k] = stEp[e][tile * n];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t c = c0 + 256 * k;
        if (c >= cpr) break;
        const int v0 = static_cast<int>(c * 8);
        const float scT = fexp(mT[k] - lseT);
        const int yi = label_offset(y, v0);   // the label's entry in this chunk when 0 <= yi < 8
        float p[8];
        float sp = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = Scratch<bf16_t>::get(tw[k], i) * scT;
          sp += p[i];
        }
#pragma unroll
        for (int e = 0; e < MS; ++e) {
          if (e >= S) break;
          const float mt = mE[e][k];
          float ps = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) ps = fmaf(p[i], Scratch<bf16_t>::get(sr[e][k], i), ps);
          acc[e] += fmaf(mt, sp, ps);
          if constexpr (WRITE_G)
            __builtin_nontemporal_store(
                grad_chunk(sr[e][k], tw[k], grad_tile_c(false, rE[e], mt, lseE[e]),
                           grad_tile_k(rE[e], scT), rE[e].lab, yi, negE[e]),
                reinterpret_cast<u32x4*>(static_cast<bf16_t*>(dl.p[e]) + t * vocab) + c);
        }
        if constexpr (WRITE_G)
          __builtin_nontemporal_store(
              grad_chunk_teacher(tw[k], grad_tile_k(rT, scT), rT.lab, yi, negT),
              reinterpret_cast<u32x4*>(static_cast<bf16_t*>(dl.p[M - 1]) + t * vocab) + c);
      }
    }
#pragma unroll
    for (int e = 0; e < MS; ++e) {
      if (e >= S) break;
      const float a = wave_sum(acc[e]);
      if (lane == 0) red[wave][e] = a;
    }
    __syncthreads();
    if (tid < S)
      dv[static_cast<int64_t>(tid) * n + t] = lse[static_cast<int64_t>(tid) * n + t] -
                                              ((red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]));
    __syncthreads();   // red is reused by the next row
  }
}

// Row constants of the gradients that the backward GEMMs form from the fp16
// scratch (grad_chunk.h), per (exit, vocabulary tile, token) over the plane,
// from the same expressions as finalize_rows_f16: |gs lambda_e| NaN for a bad
// label, which makes every gradient of that token NaN, as the in-place pass
// does.  The signs of gs lambda_e are left to the GEMMs.
__global__ __launch_bounds__(256) void grad_consts_kernel(int M, int64_t n, int vocab, int n_vt,
                                                          const int32_t* __restrict__ labels,
                                                          float alpha, float gs, ExitW lam,
                                                          const float* __restrict__ stats,
                                                          const float* __restrict__ lse,
                                                          GradRowConst* __restrict__ out) {
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < plane;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t tile = i / n, t = i - tile * n;
    const int y = labels[t];
    const bool bad = y < 0 || y >= vocab;
    const float nanv = __builtin_nanf("");
    const float lseT = lse[static_cast<int64_t>(M - 1) * n + t];
    const float scT = fexp(stats[static_cast<int64_t>(M - 1) * 3 * plane + tile * n + t] - lseT);
    for (int e = 0; e < M; ++e) {
      const bool teacher = e == M - 1;
      const GradExitRow r = grad_exit_row(teacher, bad ? nanv : fabsf(gs * lam.w[e]), alpha);
      float c = -INFINITY;
      if (!teacher)
        c = grad_tile_c(false, r, stats[static_cast<int64_t>(e) * 3 * plane + tile * n + t],
                        lse[static_cast<int64_t>(e) * n + t]);
      u32x4 v;
      v[0] = __float_as_uint(c);
      v[1] = __float_as_uint(grad_tile_k(r, scT));
      v[2] = __float_as_uint(r.lab);
      v[3] = static_cast<uint32_t>(y);
      *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(e) * plane + i) = v;
    }
  }
}

// Element path for any vocabulary size.
template <typename T, int DIV>
__global__ __launch_bounds__(256) void finalize_elem(int M, int64_t n, int vocab, int vtile,
                                                     const int32_t* __restrict__ labels,
                                                     float alpha, float gs,
                                                     const float* __restrict__ stats,
                                                     const float* __restrict__ lse, DlPtrs dl,
                                                     int n_vt, const float* __restrict__ kv,
                                                     ExitW lam) {
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const int64_t total = n * vocab;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = i / vocab;
    const int v = static_cast<int>(i - t * vocab);
    const int tile = v / vtile;
    const int y = labels[t];
    const bool bad = y < 0 || y >= vocab;
    const int eT = M - 1;
    T* pt = static_cast<T*>(dl.p[eT]) + i;
    const float lp = Scratch<T>::load(pt) +
                     stats[static_cast<int64_t>(eT) * 3 * plane + static_cast<int64_t>(tile) * n + t] -
                     lse[static_cast<int64_t>(eT) * n + t];
    const float p = fexp(lp);
    for (int e = 0; e < M; ++e) {
      T* pe = static_cast<T*>(dl.p[e]) + i;
      float val;
      if (e == eT) {
        val = p - (v == y ? 1.f : 0.f);
      } else {
        const float lq = Scratch<T>::load(pe) +
                         stats[static_cast<int64_t>(e) * 3 * plane + static_cast<int64_t>(tile) * n + t] -
                         lse[static_cast<int64_t>(e) * n + t];
        const float q = fexp(lq);
        if constexpr (DIV == kDivForward)
          val = q - alpha * p;
        else
          val = (1.f - alpha) * q +
                alpha * q * (div_r<DIV>(lp, lq, p, q) - kv[static_cast<int64_t>(e) * n + t]);
        if (v == y) val -= 1.f - alpha;
      }
      *pe = Elem<T>::from_f32(bad ? __builtin_nanf("") : gs * lam.w[e] * val);
    }
  }
}

// ---------------------------------------------------------------- argmax merge
// One wavefront per (exit, token): lane l takes tiles l, l + 64, ... in
// ascending order (strict > keeps a tile's lower index on ties), then the
// lanes' winners are combined by value, the lower index on ties.
__global__ __launch_bounds__(256) void argmax_merge_kernel(int E, int64_t n,
                                                           const float* __restrict__ best,
                                                           int32_t* __restrict__ argmax, int n_vt) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= E * n) return;   // wavefront-uniform
  const int64_t e = i / n, t = i - e * n;
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const float* b = best + e * 2 * plane + t;
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int vt = lane; vt < n_vt; vt += 64) {
    const float v = b[static_cast<int64_t>(vt) * n];
    if (v > bv) {
      bv = v;
      bi = __float_as_int(b[plane + static_cast<int64_t>(vt) * n]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) argmax[i] = bi;
}

// ---------------------------------------------------------------- acceptance
__global__ __launch_bounds__(256) void accept_kernel(int B, int P, int dlen,
                                                     const int32_t* __restrict__ d,
                                                     const int32_t* __restrict__ v,
                                                     int32_t* __restrict__ acc) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int64_t base = static_cast<int64_t>(b) * P;
  int k = 0;
  while (k < dlen && d[base + k] == v[base + k]) ++k;
  acc[b] = k;
}

__global__ void clear_flags_kernel(int32_t* f) { *f = 0; }

}  // namespace

hipError_t launch_loss_merge(int n_exits, int64_t n, int vocab, int vtile, const int32_t* labels,
                             float alpha, const float* stats, const float* lab, float* lse,
                             float* tokloss, double* partials, int32_t* flags, const ExitW& lam,
                             bool skip_dist, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(loss_merge_kernel, dim3(static_cast<unsigned>(n_merge_blocks(n))), dim3(1024), 0,
                     s, n_exits, n, vocab, labels, alpha, stats, lab, lse, tokloss, partials, flags,
                     (vocab + vtile - 1) / vtile, lam, skip_dist ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_loss_finish(int n_exits, int64_t n, float alpha, const float* dv,
                              float* tokloss, double* partials, const ExitW& lam, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(div_finish_kernel, dim3(static_cast<unsigned>(n_merge_blocks(n))), dim3(64), 0,
                     s, n_exits, n, alpha, dv, tokloss, partials, lam);
  return hipGetLastError();
}

hipError_t launch_finalize_rows(int n_exits, int64_t n, int vocab, const TileInfo& info,
                                const int32_t* labels, float alpha, float grad_scale,
                                const float* stats, const float* lse, void* const* dlogits,
                                float* dv, const ExitW& lam, bool write_g, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (!info.teacher_w16 || vocab % 8 != 0 || (info.vtile & (info.vtile - 1)) != 0)
    return hipErrorInvalidValue;
  const int vshift = __builtin_ctz(static_cast<unsigned>(info.vtile));
  DlPtrs dl{};
  for (int e = 0; e < n_exits; ++e) dl.p[e] = dlogits[e];
  // one workgroup per row up to 65536 rows (grid-stride beyond)
  const unsigned grid = static_cast<unsigned>(n < 65536 ? n : 65536);
  const int n_vt = (vocab + info.vtile - 1) / info.vtile;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, n_exits, n, vocab, vshift, labels, alpha,
                       grad_scale, stats, lse, dl, n_vt, dv, lam);
  };
  // unrolled for exactly the smaller exits there are (up to three), so that no
  // load of an unused exit slot is issued
  if (n_exits <= 2)
    write_g ? go(finalize_rows_f16<1, true>) : go(finalize_rows_f16<1, false>);
  else if (n_exits == 3)
    write_g ? go(finalize_rows_f16<2, true>) : go(finalize_rows_f16<2, false>);
  else if (n_exits == 4)
    write_g ? go(finalize_rows_f16<3, true>) : go(finalize_rows_f16<3, false>);
  else
    write_g ? go(finalize_rows_f16<kMaxExits - 1, true>)
            : go(finalize_rows_f16<kMaxExits - 1, false>);
  return hipGetLastError();
}

hipError_t launch_grad_consts(int n_exits, int64_t n, int vocab, const TileInfo& info,
                              const int32_t* labels, float alpha, float grad_scale,
                              const ExitW& lam, const float* stats, const float* lse, void* out,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (!info.teacher_w16) return hipErrorInvalidValue;   // constants of the fp16 scratch only
  const int n_vt = (vocab + info.vtile - 1) / info.vtile;
  const int64_t plane = static_cast<int64_t>(n_vt) * n;
  const int64_t blocks = (plane + 255) / 256;
  hipLaunchKernelGGL(grad_consts_kernel, dim3(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)),
                     dim3(256), 0, s, n_exits, n, vocab, n_vt, labels, alpha, grad_scale, lam,
                     stats, lse, static_cast<GradRowConst*>(out));
  return hipGetLastError();
}

template <typename T>
hipError_t launch_divergence(int n_exits, int64_t n, int vocab, const TileInfo& info, int div,
                             float alpha, const float* stats, const float* lse,
                             void* const* dlogits, float* dv, float* kv, float* tokloss,
                             double* partials, const ExitW& lam, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (info.teacher_w16)
    return hipErrorInvalidValue;   // needs every exit's shifted logits
  DlPtrs dl{};
  for (int e = 0; e < n_exits; ++e) dl.p[e] = dlogits[e];
  const int n_vt = (vocab + info.vtile - 1) / info.vtile;
  if (n_exits > 1) {
    const unsigned grid = static_cast<unsigned>(n < 256 * 16 ? n : 256 * 16);
    switch (div) {
      case kDivReverseKL:
        hipLaunchKernelGGL((div_stats_kernel<T, kDivReverseKL>), dim3(grid), dim3(256), 0, s,
                           n_exits, n, vocab, info.vtile, stats, lse, dl, n_vt, dv, kv);
        break;
      case kDivJS:
        hipLaunchKernelGGL((div_stats_kernel<T, kDivJS>), dim3(grid), dim3(256), 0, s, n_exits, n,
                           vocab, info.vtile, stats, lse, dl, n_vt, dv, kv);
        break;
      case kDivTV:
        hipLaunchKernelGGL((div_stats_kernel<T, kDivTV>), dim3(grid), dim3(256), 0, s, n_exits, n,
                           vocab, info.vtile, stats, lse, dl, n_vt, dv, kv);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  return launch_loss_finish(n_exits, n, alpha, dv, tokloss, partials, lam, s);
}

template hipError_t launch_divergence<bf16_t>(int, int64_t, int, const TileInfo&, int, float,
                                              const float*, const float*, void* const*, float*,
                                              float*, float*, double*, const ExitW&, hipStream_t);
template hipError_t launch_divergence<float>(int, int64_t, int, const TileInfo&, int, float,
                                             const float*, const float*, void* const*, float*,
                                             float*, float*, double*, const ExitW&, hipStream_t);

hipError_t launch_loss_means(int n_exits, int64_t n, const double* partials, float* means,
                             hipStream_t s) {
  hipLaunchKernelGGL(loss_means_kernel, dim3(1), dim3(256), 0, s, n_exits, n, n_merge_blocks(n),
                     partials, means);
  return hipGetLastError();
}

template <typename T, int DIV>
static void finalize_div(int n_exits, int64_t n, int vocab, const TileInfo& info,
                         const int32_t* labels, float alpha, float grad_scale, const float* stats,
                         const float* lse, const DlPtrs& dl, const float* kv, const ExitW& lam,
                         hipStream_t s) {
  constexpr int C = Elem<T>::kChunk;
  const int vtile = info.vtile;
  const int n_vt = (vocab + vtile - 1) / vtile;
  if (vocab % C == 0) {
    const int64_t cpr = vocab / C;
    const int segs = static_cast<int>((cpr + 255) / 256);
    const int64_t nseg = n * segs;
    const unsigned grid = static_cast<unsigned>(nseg < 256 * 16 ? nseg : 256 * 16);
    hipLaunchKernelGGL((finalize_vec<T, DIV>), dim3(grid), dim3(256), 0, s, n_exits, n,
                       vocab, vtile, labels, alpha, grad_scale, stats, lse, dl, n_vt, segs, kv,
                       lam);
  } else {
    const int64_t total = n * vocab;
    const int64_t blocks = (total + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 256 * 16 ? blocks : 256 * 16);
    hipLaunchKernelGGL((finalize_elem<T, DIV>), dim3(grid), dim3(256), 0, s, n_exits, n, vocab,
                       vtile, labels, alpha, grad_scale, stats, lse, dl, n_vt, kv, lam);
  }
}

template <typename T>
hipError_t launch_finalize(int n_exits, int64_t n, int vocab, const TileInfo& info,
                           const int32_t* labels, float alpha, float grad_scale,
                           const float* stats, const float* lse, void* const* dlogits, int div,
                           const float* kv, const ExitW& lam, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (info.teacher_w16)
    return hipErrorInvalidValue;   // teacher weights: finalize_rows reads them
  DlPtrs dl{};
  for (int e = 0; e < n_exits; ++e) dl.p[e] = dlogits[e];
  switch (div) {
    case kDivForward:
      finalize_div<T, kDivForward>(n_exits, n, vocab, info, labels, alpha, grad_scale, stats, lse,
                                   dl, kv, lam, s);
      break;
    case kDivReverseKL:
      finalize_div<T, kDivReverseKL>(n_exits, n, vocab, info, labels, alpha, grad_scale, stats,
                                     lse, dl, kv, lam, s);
      break;
    case kDivJS:
      finalize_div<T, kDivJS>(n_exits, n, vocab, info, labels, alpha, grad_scale, stats, lse, dl,
                              kv, lam, s);
      break;
    case kDivTV:
      finalize_div<T, kDivTV>(n_exits, n, vocab, info, labels, alpha, grad_scale, stats, lse, dl,
                              kv, lam, s);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_finalize<bf16_t>(int, int64_t, int, const TileInfo&, const int32_t*,
                                            float, float, const float*, const float*,
                                            void* const*, int, const float*, const ExitW&,
                                            hipStream_t);
template hipError_t launch_finalize<float>(int, int64_t, int, const TileInfo&, const int32_t*,
                                           float, float, const float*, const float*, void* const*,
                                           int, const float*, const ExitW&, hipStream_t);

hipError_t launch_argmax_merge(int n_exits, int64_t n, int vocab, int vtile, const float* best,
                               int32_t* argmax, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t total = n_exits * n;
  hipLaunchKernelGGL(argmax_merge_kernel, dim3(static_cast<unsigned>((total + 3) / 4)),
                     dim3(256), 0, s, n_exits, n, best, argmax, (vocab + vtile - 1) / vtile);
  return hipGetLastError();
}

hipError_t launch_accept(int batch, int positions, int draft_len, const int32_t* draft,
                         const int32_t* verify, int32_t* accepted, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(accept_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, batch, positions,
                     draft_len, draft, verify, accepted);
  return hipGetLastError();
}

hipError_t launch_clear_flags(int32_t* flags, hipStream_t s) {
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, s, flags);
  return hipGetLastError();
}

}  // namespace nel
