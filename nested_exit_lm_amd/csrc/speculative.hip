// Sampled speculative verification from the draft and verifying exits' fp32
// logits (follow-up 4 on "Is nesting the cheapest way to build a model
// suite?": a drafted token is accepted with probability
// beta = sum_v min(p_v, q_v); "Matryoshka Language Model Suites",
// speculative-decoding paragraph: the nested draft / verifier pair under
// nucleus sampling).
//
// Per position the sampling distribution of an exit is softmax(l / T)
// restricted to its nucleus (the most probable entries reaching top_p, every
// entry tied with the last one needed included) and renormalised.  Per
// sequence: drafted token x_i (i < L) is accepted iff u_i p(x_i) < q(x_i);
// after the first rejection at k the next token is drawn from max(0, q_k - p_k)
// (q_k if that is all zero), after L acceptances from q at position L; draws
// are inverse-CDF in vocabulary order with the caller's uniform.
//
// Kernels: (1) per exit and position (a 1024-thread workgroup), the row
// maximum, the softmax sum and the nucleus threshold, found exactly by a
// bisection on order-preserving integer keys of the unnormalised
// probabilities (30 steps: the two top bits are fixed; every step a
// fixed-order workgroup reduction in fp64, so every thread takes the same
// decision);
// (2) beta per drafted position; (3) per sequence, the acceptance chain and
// the draw from weights staged in LDS, whose running sums are fp64.
// Probabilities themselves are fp32.
// A row lives in registers (V <= kStatThreads x kPer).
#include "common.h"
#include "internal.h"

namespace nel {

namespace {

constexpr int kStatThreads = 1024;   // threads per row of the statistics kernel
constexpr int kPer = 32;             // row entries per thread: V <= 32768
constexpr int kMaxVocab = kStatThreads * kPer;

// Unnormalised probability exp(l / T - max) of a raw logit.  Multiply and
// subtract are kept separate (no contraction) so that every kernel derives
// bit-identical values, and with them identical nucleus membership.
__device__ __forceinline__ float scaled(float l, float inv_t) { return __fmul_rn(l, inv_t); }
__device__ __forceinline__ float unnorm(float l, float inv_t, float mx) {
  return fexp(__fsub_rn(scaled(l, inv_t), mx));
}

// Reductions over a workgroup of NW wavefronts in a fixed order (wavefront
// results combined as a balanced tree); every thread gets the result.
template <int NW, typename T>
__device__ __forceinline__ T tree_sum(const T* r) {
  if constexpr (NW == 1)
    return r[0];
  else
    return tree_sum<NW / 2>(r) + tree_sum<NW / 2>(r + NW / 2);
}
template <int NW>
__device__ __forceinline__ float tree_max(const float* r) {
  if constexpr (NW == 1)
    return r[0];
  else
    return fmaxf(tree_max<NW / 2>(r), tree_max<NW / 2>(r + NW / 2));
}
template <int NW = 4>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return tree_sum<NW>(red);
}
template <int NW = 4>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return tree_sum<NW>(red);
}
// The same sum with one barrier instead of two, for a sequence of reductions
// that alternate between two slot arrays: the barrier of one reduction also
// orders every read of the other array (by the reduction before it) ahead of
// the next write to it.
template <int NW>
__device__ __forceinline__ double block_sum_f64_alt(double v, double (&red)[2][NW], int& parity) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double* r = red[parity];
  parity ^= 1;
  if (lane == 0) r[wave] = v;
  __syncthreads();
  return tree_sum<NW>(r);
}
template <int NW = 4>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return tree_max<NW>(red);
}

// Row statistics of one (exit, position): stats = {max of l/T, nucleus sum
// sum_{kept} exp(l/T - max), threshold (the smallest kept value), softmax sum}.
// Thread t holds entries t + kStatThreads j; each thread's sums run over four
// interleaved partial sums (independent add chains) combined in a fixed order.
// Eight wavefronts per SIMD (64 registers per lane, a few values spilled) let
// two workgroups share a CU, so one's reductions overlap the other's
// arithmetic; measured faster than one workgroup per CU at 68 registers.
__global__ __launch_bounds__(kStatThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void nucleus_stats_kernel(
    const float* __restrict__ draft, const float* __restrict__ verify, int positions, int rows_per_seq,
    int vocab, float inv_t, float top_p, float4* __restrict__ stats) {
  constexpr int NW = kStatThreads / 64;
  __shared__ float red[NW];
  __shared__ double red64[2][NW];
  int parity = 0;
  const int tid = threadIdx.x;
  const int nrows = gridDim.x / 2;
  const int exit = blockIdx.x / nrows, r = blockIdx.x % nrows;   // r = b * rows_per_seq + i
  const int b = r / rows_per_seq, i = r % rows_per_seq;
  const float* row = (exit == 0 ? draft : verify) + (static_cast<int64_t>(b) * positions + i) * vocab;
  float x[kPer];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int v = tid + kStatThreads * j;
    x[j] = v < vocab ? row[v] : -INFINITY;
    if (v < vocab) mx = fmaxf(mx, scaled(x[j], inv_t));
  }
  mx = block_max<NW>(mx, red);
  // From here the row is held as its unnormalised probabilities, in place of
  // the logits.  They are all >= 0, so their bit patterns order like their
  // values, and the order key of a value is its bits with bit 31 set: a key
  // K >= 2^31 selects the values whose bits are >= K - 2^31, and K = 0 all.
  float sp[4] = {0.f, 0.f, 0.f, 0.f};   // this thread's share of the softmax sum
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int v = tid + kStatThreads * j;
    x[j] = v < vocab ? unnorm(x[j], inv_t, mx) : 0.f;
    sp[j & 3] += x[j];
  }
  auto mass = [&](uint32_t K) {   // this thread's mass of keys >= K
    const uint32_t lo = K & 0x7fffffffu;
    float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kPer; ++j) m[j & 3] += __float_as_uint(x[j]) >= lo ? x[j] : 0.f;
    return (m[0] + m[1]) + (m[2] + m[3]);
  };
  // largest key K with mass(key >= K) >= top_p.  Each thread's 32 terms are
  // summed in fp32, the workgroup's 1024 partial sums in fp64.
  const double s64 = block_sum_f64_alt<NW>((sp[0] + sp[1]) + (sp[2] + sp[3]), red64, parity);
  uint32_t K = 0;
  if (top_p < 1.f) {
    const double need = static_cast<double>(top_p) * s64;
    // The two top bits are decided without a reduction.  Bit 31: every key
    // has it (all values are >= 0), and the mass of all keys is s64 itself
    // (the same fp32 terms added in the same order), which is >= need.
    // Bit 30: keys with it hold values >= 2, and no value exceeds exp(0) = 1,
    // so that mass is 0 < need.
    K = 0x80000000u;
    for (int bit = 29; bit >= 0; --bit) {
      const uint32_t cand = K | (1u << bit);
      if (block_sum_f64_alt<NW>(mass(cand), red64, parity) >= need) K = cand;
    }
  }
  const float sn = static_cast<float>(block_sum_f64_alt<NW>(mass(K), red64, parity));
  // the threshold as a value: the smallest kept e (K without its order bit;
  // 0 keeps every entry when top_p = 1)
  if (tid == 0)
    stats[blockIdx.x] = make_float4(mx, sn, __uint_as_float(K & 0x7fffffffu), static_cast<float>(s64));
}

// Nucleus probability of entry value l (raw logit) under row stats st.
__device__ __forceinline__ float nprob(float l, float inv_t, float4 st) {
  const float e = unnorm(l, inv_t, st.x);
  // e >= 0, so comparing bit patterns compares values
  return __float_as_uint(e) >= __float_as_uint(st.z) ? e / st.y : 0.f;
}

__global__ __launch_bounds__(256) void beta_kernel(const float* __restrict__ draft,
                                                   const float* __restrict__ verify, int positions,
                                                   int rows_per_seq, int draft_len, int vocab,
                                                   float inv_t, const float4* __restrict__ stats,
                                                   float* __restrict__ beta) {
  __shared__ float red[4];
  const int b = blockIdx.x / draft_len, i = blockIdx.x % draft_len;
  const int nrows = gridDim.x / draft_len * rows_per_seq;
  const int r = b * rows_per_seq + i;
  const float4 sp = stats[r], sq = stats[nrows + r];
  const int64_t off = (static_cast<int64_t>(b) * positions + i) * vocab;
  // eight entries per thread per round, their loads issued together; the
  // sum runs over them in vocabulary order
  float acc = 0.f;
  for (int base = 0; base < vocab; base += 256 * 8) {
    float dv[8], qv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = base + static_cast<int>(threadIdx.x) + 256 * u;
      dv[u] = v < vocab ? draft[off + v] : 0.f;
      qv[u] = v < vocab ? verify[off + v] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int v = base + static_cast<int>(threadIdx.x) + 256 * u;
      if (v < vocab) acc += fminf(nprob(dv[u], inv_t, sp), nprob(qv[u], inv_t, sq));
    }
  }
  acc = block_sum(acc, red);
  if (threadIdx.x == 0) beta[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void accept_draw_kernel(
    const float* __restrict__ draft, const float* __restrict__ verify, int positions,
    int rows_per_seq, int draft_len, int vocab, float inv_t, const float4* __restrict__ stats,
    const int32_t* __restrict__ tokens, const float* __restrict__ u_accept,
    const float* __restrict__ u_next, int32_t* __restrict__ accepted,
    int32_t* __restrict__ next_token, int32_t* __restrict__ flags) {
  const int tid = threadIdx.x, b = blockIdx.x;
  const int nrows = gridDim.x * rows_per_seq;
  // acceptance chain (every thread computes it identically)
  int k = 0;
  bool bad = false;
  for (; k < draft_len; ++k) {
    const int64_t pos = static_cast<int64_t>(b) * positions + k;
    const int x = tokens[pos];
    if (x < 0 || x >= vocab) {
      bad = true;
      break;
    }
    const int r = b * rows_per_seq + k;
    const float p = nprob(draft[pos * vocab + x], inv_t, stats[r]);
    const float q = nprob(verify[pos * vocab + x], inv_t, stats[nrows + r]);
    if (!(u_accept[pos] * p < q)) break;
  }
  if (bad && tid == 0 && flags) atomicOr(flags, 1 /*NEL_FLAG_BAD_ID*/);
  // the distribution of the next token: residual at k, or q at position L
  const int r = b * rows_per_seq + k;
  const float4 sp = stats[r], sq = stats[nrows + r];
  const int64_t off = (static_cast<int64_t>(b) * positions + k) * vocab;
  const bool residual = k < draft_len;
  // this thread's contiguous chunk of the vocabulary
  const int per = (vocab + 255) / 256;
  const int v0 = tid * per, v1 = min(v0 + per, vocab);
  // The row's weights are computed once, with coalesced reads, into LDS; one
  // pad word per 128 entries keeps the chunk-wise reads below free of bank
  // conflicts when chunks are 128 entries long (V = 32768).
  __shared__ float wl[kMaxVocab + kMaxVocab / 128];
  // eight entries per thread per round, their loads issued together
  auto stage = [&](bool res) {
    for (int base = 0; base < vocab; base += 256 * 8) {
      float qv[8], dv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = base + tid + 256 * u;
        qv[u] = v < vocab ? verify[off + v] : 0.f;
        dv[u] = v < vocab && res ? draft[off + v] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = base + tid + 256 * u;
        if (v < vocab) {
          const float q = nprob(qv[u], inv_t, sq);
          wl[v + (v >> 7)] = res ? fmaxf(q - nprob(dv[u], inv_t, sp), 0.f) : q;
        }
      }
    }
    __syncthreads();
  };
  auto w_at = [&](int v) { return wl[v + (v >> 7)]; };
  // running sums of the draw in fp64: chunk sums, their exclusive prefix in
  // thread order, then the crossing inside the one chunk that holds it
  __shared__ double red64[4];
  __shared__ double excl[256];
  __shared__ double red_lane[64];
  __shared__ double seq_total;
  __shared__ int firstpick, lastpos;
  stage(residual);
  double part = 0.0;
  for (int v = v0; v < v1; ++v) part += w_at(v);
  if (residual && !(block_sum_f64(part, red64) > 0.0)) {   // q == p on the nucleus: draw from q
    __syncthreads();
    stage(false);
    part = 0.0;
    for (int v = v0; v < v1; ++v) part += w_at(v);
  }
  __syncthreads();
  excl[tid] = part;
  if (tid == 0) {
    firstpick = 0x7fffffff;
    lastpos = -1;
  }
  __syncthreads();
  // exclusive prefix of the 256 chunk sums by wavefront 0: each lane adds
  // four consecutive chunks in order, lane 0 runs over the 64 lane totals,
  // each lane then offsets its four (a fixed order, so the result is
  // reproducible)
  if (tid < 64) {
    const double c0 = excl[4 * tid], c1 = excl[4 * tid + 1], c2 = excl[4 * tid + 2],
                 c3 = excl[4 * tid + 3];
    const double s1 = c0 + c1, s2 = s1 + c2, s3 = s2 + c3;
    red_lane[tid] = s3;
    wave_lds_sync();
    if (tid == 0) {
      double run = 0.0;
      for (int t = 0; t < 64; ++t) {
        const double c = red_lane[t];
        red_lane[t] = run;
        run += c;
      }
      seq_total = run;
    }
    wave_lds_sync();
    const double base = red_lane[tid];
    excl[4 * tid] = base;
    excl[4 * tid + 1] = base + c0;
    excl[4 * tid + 2] = base + s1;
    excl[4 * tid + 3] = base + s2;
  }
  __syncthreads();
  const double target = static_cast<double>(u_next[b]) * seq_total;
  // the last entry of positive weight is the fallback when rounding leaves
  // the target uncrossed
  double run = excl[tid];
  int pick = -1, last_pos = -1;
  for (int v = v0; v < v1; ++v) {
    const float w = w_at(v);
    if (w > 0.f) last_pos = v;
    if (pick < 0 && w > 0.f && run + w > target) pick = v;
    run += w;
  }
  if (pick >= 0) atomicMin(&firstpick, pick);
  if (last_pos >= 0) atomicMax(&lastpos, last_pos);
  __syncthreads();
  if (tid == 0) {
    accepted[b] = k;
    next_token[b] = firstpick != 0x7fffffff ? firstpick : lastpos;
  }
}

}  // namespace

size_t speculative_ws_bytes(int batch, int draft_len) {
  return sizeof(float4) * 2 * static_cast<size_t>(batch) * (draft_len + 1);
}

hipError_t launch_speculative_verify(int batch, int positions, int draft_len, int vocab,
                                     const float* draft, const float* verify,
                                     const int32_t* tokens, const float* u_accept,
                                     const float* u_next, float temperature, float top_p,
                                     float* beta, int32_t* accepted, int32_t* next_token,
                                     int32_t* flags, void* workspace, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const int rows_per_seq = draft_len + 1;
  const float inv_t = 1.f / temperature;
  float4* stats = static_cast<float4*>(workspace);
  hipLaunchKernelGGL(nucleus_stats_kernel, dim3(2 * batch * rows_per_seq), dim3(kStatThreads), 0, s, draft,
                     verify, positions, rows_per_seq, vocab, inv_t, top_p, stats);
  if (beta && draft_len > 0)
    hipLaunchKernelGGL(beta_kernel, dim3(batch * draft_len), dim3(256), 0, s, draft, verify,
                       positions, rows_per_seq, draft_len, vocab, inv_t, stats, beta);
  hipLaunchKernelGGL(accept_draw_kernel, dim3(batch), dim3(256), 0, s, draft, verify, positions,
                     rows_per_seq, draft_len, vocab, inv_t, stats, tokens, u_accept, u_next,
                     accepted, next_token, flags);
  return hipGetLastError();
}

}  // namespace nel
