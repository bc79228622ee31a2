// Multi-exit LM-head GEMM on MFMA-tiled head weights (bf16, gfx950).
//
// Same contraction and epilogues as the row-major head GEMM: every exit m's
// logits l_m = h_m W^m^T (copyedit of Sec. 2 "Modeling") in fp32 registers,
// turned into per-tile loss statistics for the distillation loss
// ("Matryoshka Language Model Suites", distillation paragraph) or into a
// per-tile greedy argmax; no fp32 logit tensor is written for the loss.
//
// Why a second weight layout.  A wavefront that keeps its whole vocabulary
// slice of W in registers needs no LDS for W at all, which removes most of the
// LDS traffic that limits an LDS-staged GEMM on this chip; but the MFMA
// operand layout puts 32 different W rows in consecutive lanes, and such
// strided row loads run at a third of the rate of contiguous ones.  So W is
// first rewritten (nel_pack_weights, one HBM-bound pass) into 1 KB blocks
// that are exactly one MFMA A operand each:
//     block (rb, kp), rb < V/32, kp < D/16, at element offset (rb * D/16 + kp) * 512;
//     lane l's 8 elements at l * 8 are W[32 rb + vperm(l % 32)][16 kp + 8 (l / 32) + j],
// so every operand load is one contiguous 1 KB read.
//
// Workgroup: 4 wavefronts, tile 128 tokens x 256 vocabulary entries, two
// workgroups per CU; the main loop (packed_core.h) streams W (the packed A
// operand) straight into registers and stages the token slice of h (the B
// operand) through LDS.  Wavefront w owns vocabulary entries [64w, 64w + 64)
// of the tile for all 128 tokens (4 x 2 accumulator blocks of 32 x 32).
//
// Loss epilogue: per (token, tile) the row maximum m, sum exp(l - m) and the
// label's logit, and one 16-bit copy of the tile in the exit's gradient
// buffer, in fp16 (relative rounding 2^-11).  kModeLossF16 (the
// cross-entropy to the teacher): the teacher (last exit, run first) stores its
// weights w = exp(l_M - m), the smaller exits l - m; the row-wise gradient
// pass forms the teacher-weighted sums sum_v p_v l_m,v from them.
// kModeLossPlain (the other divergences, whose pass reads every exit's
// l - m) stores l - m for every exit.  No epilogue reads another exit's tile
// back.
#include <limits.h>

#include "common.h"
#include "internal.h"
#include "packed_core.h"
#include "tiles.h"

namespace nel {

namespace {

constexpr int kPkTok = kPkBRows;   // tokens per workgroup (the B rows)
constexpr int kPkVoc = kPkARows;   // vocabulary entries per workgroup (the A rows)
constexpr int kPkGroup = 8;        // token tiles per tile group (see tile_coords)

// ---------------------------------------------------------------- packing
// One thread per 16-byte chunk of W, visited as (row block rb, 64-column
// group kc, row in block, chunk in the 128-byte row piece) with the chunk
// fastest: the reads are whole 128-byte row pieces, the writes of a
// workgroup fill four whole 1 KB blocks.
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ w,
                                                   bf16_t* __restrict__ p, int vocab, int d) {
  const int64_t chunks = static_cast<int64_t>(vocab) * d / 8;
  const int cpr = d / 64;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < chunks;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t grp = i >> 8;
    const int x = static_cast<int>(i & 255), row = x >> 3, ch = x & 7;
    const int64_t rb = grp / cpr;
    const int kc = static_cast<int>(grp - rb * cpr);
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + (rb * 32 + row) * d + kc * 64 + ch * 8);
    const int kp = kc * 4 + (ch >> 1);
    const int l = (ch & 1) * 32 + vperm_inv(row);
    *reinterpret_cast<u32x4*>(p + ((rb * (d / 16) + kp) * 64 + l) * 8) = v;
  }
}

// ---------------------------------------------------------------- GEMM
template <int MODE>
__global__ __launch_bounds__(kPkThreads, 2) void heads_kernel_packed(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    const int32_t* __restrict__ labels, float* __restrict__ stats, float* __restrict__ lab,
    int n_tt, int n_vt) {
  // The exit table is the first kernel argument; indexing it through the
  // kernarg segment pointer keeps per-exit lookups scalar.
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int NTB = kPkNTB, NVB = kPkNAB;
  __shared__ u32x4 hs[2][8 * kPkTok];
  __shared__ float xmax[4][kPkTok];
  __shared__ float xsum[4][kPkTok][2];

  const int tid = threadIdx.x, lane = tid & 63, q = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Loss modes: every exit in one workgroup (the teacher first).  Argmax: one
  // exit per workgroup, the widest exit's tiles first, so that at small token
  // counts the narrow exits' short workgroups fill the last round.
  int ei0 = 0, ei1 = n_exits, bid = blockIdx.x;
  if constexpr (MODE == kModeArgmax) {
    const int k = blockIdx.x / (n_tt * n_vt);
    ei0 = n_exits - 1 - k;
    ei1 = ei0 + 1;
    bid = blockIdx.x - k * (n_tt * n_vt);
  }
  int tt, vt;
  tile_coords(bid, n_tt, n_vt, kPkGroup, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kPkTok;
  const int vw = vt * kPkVoc + wave * (NVB * 32);   // this wavefront's first vocabulary entry
  const int64_t tq = t0 + q;                        // token of this lane in token block 0

  int ylab[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
    ylab[tb] = (MODE != kModeArgmax && tq + tb * 32 < n) ? labels[tq + tb * 32] : -1;
  const int vlane = vw + 16 * hl;   // first of this lane's 16 consecutive entries in block 0
  // W row block of the loads for block 0 and block 1, clamped: rows beyond V are never stored
  const int rb0 = min(vw >> 5, vocab / 32 - 1), rb1 = min((vw >> 5) + 1, vocab / 32 - 1);
  const PackedLanes pl = packed_lanes(tid);
  uint32_t hoff[4];   // byte offsets of this thread's h chunks from row t0 (rows beyond n clamped)

  f32x16 acc[NTB][NVB];
  for (int ei = ei0; ei < ei1; ++ei) {
    const int e = (MODE != kModeArgmax) ? (ei == 0 ? n_exits - 1 : ei - 1) : ei;
    const bool teacher = MODE == kModeLossF16 && ei == 0;
    const int D = ex.d[e];
    // wave-uniform bases; per-lane 32-bit byte offsets
    const char* __restrict__ Hb = static_cast<const char*>(ex.h[e]) + t0 * D * 2;
    const char* __restrict__ P = static_cast<const char*>(ex.w[e]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = min(t0 + pl.brow + 32 * j, n - 1) - t0;
      hoff[j] = static_cast<uint32_t>((row * D + pl.bchunk * 8) * 2);
    }
    packed_tile_gemm<NTB, NVB>(acc, hs, P + static_cast<int64_t>(rb0) * 64 * D,
                               P + static_cast<int64_t>(rb1) * 64 * D, Hb, hoff, pl, D / kPkBK);

    // vocabulary entries beyond V (last tile only) vanish under exp and never win a max
    if (vt * kPkVoc + kPkVoc > vocab) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vlane + 32 * vb + r >= vocab) acc[tb][vb][r] = kMasked;
    }

    const int64_t plane = static_cast<int64_t>(n_vt) * n;
    if constexpr (MODE != kModeArgmax) {
      // (1) row maximum over the tile's 256 entries: registers, lane 32 apart, 4 wavefronts
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
        if (hl == 0) xmax[wave][tb * 32 + q] = m;
      }
      __syncthreads();
      float M[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int j = tb * 32 + q;
        M[tb] = fmaxf(fmaxf(xmax[0][j], xmax[1][j]), fmaxf(xmax[2][j], xmax[3][j]));
      }
      // (2) sums, teacher weights / shifted logits, label logit
      bf16_t* __restrict__ O = static_cast<bf16_t*>(ex.out[e]);
      // The 16-bit copies leave through LDS, one 32-token block at a time: a
      // lane holds 32 bytes of one token row, but the wavefront's 64 entries
      // of a row are one aligned 128-byte line, so after a wave-local
      // transpose eight lanes store a whole line (the MFMA lanes would write
      // 32 rows x 2 pieces per store instead).  The wavefront uses its own
      // 4 KB of the B stage, which no wavefront reads again before the barrier
      // that ends this block.  Row r, 16-byte chunk c sits at slot
      // 8 r + (c ^ ((r / 2) mod 8)): writes and reads cover all 64 banks.
      char* const stage = reinterpret_cast<char*>(&hs[0][0]) + wave * 4096;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const float ml = M[tb] * kLog2e;
        const int64_t tok = tq + 32 * tb;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          // V is a multiple of 32, so a lane's 16 entries are all inside or all beyond V
          const int vbase = vlane + 32 * vb;
          if (teacher) {
            u32x4 pk[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float x0 = __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][r], kLog2e, -ml));
              const float x1 = __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][r + 1], kLog2e, -ml));
              s0 += x0;
              s1 += x1;
              pk[r >> 3][(r >> 1) & 3] = pack_f16x2(x0, x1);
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              *reinterpret_cast<u32x4*>(stage +
                                        (8 * q + ((4 * vb + 2 * hl + h2) ^ ((q >> 1) & 7))) * 16) =
                  pk[h2];
          } else {
            u32x4 pk[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float a0 = acc[tb][vb][r], a1 = acc[tb][vb][r + 1];
              s0 += __builtin_amdgcn_exp2f(fmaf(a0, kLog2e, -ml));
              s1 += __builtin_amdgcn_exp2f(fmaf(a1, kLog2e, -ml));
              pk[r >> 3][(r >> 1) & 3] = pack_f16x2(a0 - M[tb], a1 - M[tb]);
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              *reinterpret_cast<u32x4*>(stage +
                                        (8 * q + ((4 * vb + 2 * hl + h2) ^ ((q >> 1) & 7))) * 16) =
                  pk[h2];
          }
          const int dd = ylab[tb] - vbase;
          if (static_cast<unsigned>(dd) < 16u && ylab[tb] < vocab) {
            float val = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) val = (r == dd) ? acc[tb][vb][r] : val;
            lab[static_cast<int64_t>(e) * n + tok] = val;
          }
        }
        wave_lds_sync();
        {
          // wave-uniform row base, 32-bit lane offsets (a block is 32 rows of 2 V bytes)
          const int ch = lane & 7;
          const uint32_t loff = (static_cast<uint32_t>(lane >> 3) * static_cast<uint32_t>(vocab) +
                                 8u * static_cast<uint32_t>(ch)) * 2u;
          const bool col_ok = vw + 8 * ch < vocab;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 8 * j + (lane >> 3);
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(stage + (8 * row + (ch ^ ((row >> 1) & 7))) * 16);
            char* rb = reinterpret_cast<char*>(O) + ((t0 + 32 * tb + 8 * j) * vocab + vw) * 2;
            // whole lines, not read again before the gradient pass: nontemporal
            if (col_ok && t0 + 32 * tb + row < n)
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(rb + loff));
          }
        }
        wave_lds_sync();
        float s = s0 + s1;
        s += __shfl_xor(s, 32, 64);
        if (hl == 0) xsum[wave][tb * 32 + q][0] = s;
      }
      __syncthreads();
      // (3) wavefront w writes the statistics of token block w
      float Mw = M[0];
#pragma unroll
      for (int tb = 1; tb < NTB; ++tb) Mw = (tb == wave) ? M[tb] : Mw;
      const int j = wave * 32 + q;
      const int64_t tk = t0 + j;
      if (hl == 0 && tk < n) {
        float* st = stats + (static_cast<int64_t>(e) * 3 * n_vt + vt) * n + tk;
        st[0] = Mw;
        st[plane] = (xsum[0][j][0] + xsum[1][j][0]) + (xsum[2][j][0] + xsum[3][j][0]);
      }
    } else {
      // per token the tile's (max, lowest index); optional fp32 logits
      float* __restrict__ O = static_cast<float*>(ex.out[e]);
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
              bi = vlane + 32 * vb + r;
            }
        const float ov = __shfl_xor(bv, 32, 64);
        const int oi = __shfl_xor(bi, 32, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
        const int64_t tok = tq + 32 * tb;
        if (O != nullptr && tok < n) {
#pragma unroll
          for (int vb = 0; vb < NVB; ++vb) {
            const int vbase = vlane + 32 * vb;
            if (vbase >= vocab) continue;
            u32x4* dst = reinterpret_cast<u32x4*>(O + tok * vocab + vbase);
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4) {
              u32x4 pk;
#pragma unroll
              for (int k = 0; k < 4; ++k) pk[k] = __float_as_uint(acc[tb][vb][4 * h4 + k]);
              dst[h4] = pk;
            }
          }
        }
        if (hl == 0) {
          xsum[wave][tb * 32 + q][0] = bv;
          xsum[wave][tb * 32 + q][1] = __int_as_float(bi);
        }
      }
      __syncthreads();
      const int j = wave * 32 + q;
      const int64_t tk = t0 + j;
      if (hl == 0 && tk < n) {
        float bv = xsum[0][j][0];
        int bi = __float_as_int(xsum[0][j][1]);
#pragma unroll
        for (int w = 1; w < 4; ++w)   // later wavefronts hold higher indices: ties keep the first
          if (xsum[w][j][0] > bv) {
            bv = xsum[w][j][0];
            bi = __float_as_int(xsum[w][j][1]);
          }
        float* b = stats + (static_cast<int64_t>(e) * 2 * n_vt + vt) * n + tk;
        b[0] = bv;
        b[plane] = __int_as_float(bi);
      }
    }
    // xmax / xsum are next written after this exit's main loop, behind its barriers
  }
}

template <int MODE>
hipError_t launch_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                         const int32_t* labels, float* stats, float* lab, TileInfo* info,
                         hipStream_t s) {
  info->vtile = kPkVoc;
  info->teacher_w16 = MODE == kModeLossF16;
  if (n == 0) return hipSuccess;
  const int n_tt = static_cast<int>((n + kPkTok - 1) / kPkTok);
  const int n_vt = (vocab + kPkVoc - 1) / kPkVoc;
  const int splits = MODE == kModeArgmax ? n_exits : 1;   // argmax: a workgroup per exit
  hipLaunchKernelGGL((heads_kernel_packed<MODE>), dim3(n_tt * n_vt * splits), dim3(kPkThreads), 0,
                     s, ex, n_exits, n, vocab, labels, stats, lab, n_tt, n_vt);
  return hipGetLastError();
}

}  // namespace

// d below 2^24 keeps the 32-bit byte offsets of a 128-token slice of h in range.
bool packed_shape_ok(int vocab, int d) {
  return vocab >= 32 && vocab % 32 == 0 && d >= 64 && d % 64 == 0 && d < (1 << 24);
}

hipError_t launch_pack_weights(int vocab, int d, const void* w, void* packed, hipStream_t s) {
  const int64_t chunks = static_cast<int64_t>(vocab) * d / 8;
  const int64_t blocks = (chunks + 255) / 256;
  const int grid = static_cast<int>(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, static_cast<const bf16_t*>(w),
                     static_cast<bf16_t*>(packed), vocab, d);
  return hipGetLastError();
}

hipError_t launch_heads_loss_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                                    const int32_t* labels, float* stats, float* lab, bool plain,
                                    TileInfo* info, hipStream_t s) {
  if (plain)
    return launch_packed<kModeLossPlain>(n_exits, n, vocab, ex, labels, stats, lab, info, s);
  return launch_packed<kModeLossF16>(n_exits, n, vocab, ex, labels, stats, lab, info, s);
}

hipError_t launch_heads_argmax_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                                      float* best, TileInfo* info, hipStream_t s) {
  return launch_packed<kModeArgmax>(n_exits, n, vocab, ex, nullptr, best, nullptr, info, s);
}

}  // namespace nel
