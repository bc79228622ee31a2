// Main loop of the bf16 GEMMs whose A operand is in the MFMA-tiled layout
// (device side; shared by the head GEMM and the head-backward GEMMs).
//
// A workgroup of 4 wavefronts computes a 128 x 256 tile of C = B A^T:
//  * A: 256 rows (64 per wavefront, two 32-row blocks), packed so that every
//    MFMA A operand is one contiguous 1 KB block: row block rb, K block kp
//    (16 columns) at byte (rb * K / 16 + kp) * 1024, lane l's 16 bytes at
//    l * 16 holding row 32 rb + vperm(l % 32), columns 16 kp + 8 (l / 32) ...+7.
//    Each wavefront loads its blocks straight into registers, one K step
//    (64 columns, 4 blocks per row block) ahead of the MFMAs.
//  * B: 128 rows, row-major with K contiguous.  The workgroup loads each
//    128 x 64 slice once and publishes it in LDS (double-buffered) for all
//    four wavefronts.  LDS holds the slice chunk-major: row t, 16-byte chunk c
//    in slot 128 c + (t ^ 2c), so the reads of 16 consecutive rows and the
//    writes of 2 rows x 8 chunks both cover all 64 banks once per 16-lane pass.
//  * C: accumulator acc[tb][ab] is the 32 x 32 block (B rows 32 tb.., A rows
//    32 ab..) of the wavefront; lane (q, h) holds B row 32 tb + q and the 16
//    consecutive A rows 32 ab + 16 h + r, r = acc register.
#pragma once
#include "common.h"

namespace nel {

constexpr int kPkThreads = 256;   // 4 wavefronts
constexpr int kPkBRows = 128;     // B rows per workgroup
constexpr int kPkARows = 256;     // A rows per workgroup
constexpr int kPkBK = 64;         // K per step
constexpr int kPkNTB = 4;         // B blocks of 32 rows per wavefront
constexpr int kPkNAB = 2;         // A blocks of 32 rows per wavefront

// Per-thread constants of the main loop.
struct PackedLanes {
  int hslot;          // LDS slot of this thread's first B chunk (next: + 32 j)
  int bslot[4];       // LDS slot of the B fragment of K slice s, block 0 (block tb: + 32 tb)
  int brow, bchunk;   // B row and 16-byte chunk this thread loads (rows brow + 32 j)
  uint32_t aoff;      // byte offset of this lane's 16 bytes in an A block
};

__device__ __forceinline__ PackedLanes packed_lanes(int tid) {
  PackedLanes p;
  const int lane = tid & 63, q = lane & 31, hl = lane >> 5;
  p.bchunk = tid & 7;
  p.brow = tid >> 3;
  // chunk i = tid + 256 j of the 128 x 64 slice is row i / 8 = tid / 8 + 32 j,
  // chunk i % 8; slot 128 c + (t ^ 2c) = hslot + 32 j (2c < 32 leaves bit 5 alone)
  p.hslot = p.bchunk * kPkBRows + (p.brow ^ (2 * p.bchunk));
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int c = 2 * s + hl;
    p.bslot[s] = c * kPkBRows + (q ^ (2 * c));
  }
  p.aoff = static_cast<uint32_t>(lane) * 16u;
  return p;
}

// acc = A(this wavefront's two row blocks) x B(the workgroup's 128 rows)^T
// over K = 64 * nsteps.
//   A0, A1: byte bases of the wavefront's two packed A row blocks
//   Bb:     byte base of the tile's B row 0
//   boff:   byte offsets from Bb of this thread's four B chunks (per K step
//           the base advances by 128 bytes)
//   hs:     the workgroup's two LDS stages
// Every wavefront of the workgroup calls this together (it contains barriers).
template <int NTB, int NAB>
__device__ __forceinline__ void packed_tile_gemm(f32x16 (&acc)[NTB][NAB],
                                                 u32x4 (&hs)[2][8 * kPkBRows],
                                                 const char* __restrict__ A0,
                                                 const char* __restrict__ A1,
                                                 const char* __restrict__ Bb,
                                                 const uint32_t (&boff)[4], const PackedLanes& pl,
                                                 int nsteps) {
  static_assert(NAB == 2, "two A row blocks per wavefront");
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][ab][r] = 0.f;

  u32x4 R0[NAB][4], R1[NAB][4], hr[4];
  // A operands of step g: blocks kp = 4g + s of the two row blocks
  auto load_a = [&](u32x4 (&dst)[NAB][4], int g) {
    const char* a0 = A0 + static_cast<int64_t>(g) * 4096;
    const char* a1 = A1 + static_cast<int64_t>(g) * 4096;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      dst[0][s] = *reinterpret_cast<const u32x4*>(a0 + pl.aoff + s * 1024);
      dst[1][s] = *reinterpret_cast<const u32x4*>(a1 + pl.aoff + s * 1024);
    }
  };
  auto load_b = [&](int g) {
    const char* a = Bb + static_cast<int64_t>(g) * (kPkBK * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) hr[j] = *reinterpret_cast<const u32x4*>(a + boff[j]);
  };
  auto store_b = [&](int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hs[st][pl.hslot + 32 * j] = hr[j];
  };
  auto mfma = [&](const u32x4 (&cur)[NAB][4], int st) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 b[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) b[tb] = __builtin_bit_cast(bf16x8, hs[st][pl.bslot[s] + 32 * tb]);
#pragma unroll
      for (int ab = 0; ab < NAB; ++ab) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, cur[ab][s]);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[tb][ab] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[tb], acc[tb][ab], 0, 0, 0);
      }
    }
  };
  // Step g: prefetch step g + 1 (the last step re-reads itself), compute
  // step g from LDS stage st, publish the prefetched B slice in stage st ^ 1.
  auto step = [&](const u32x4 (&cur)[NAB][4], u32x4 (&nxt)[NAB][4], int g, int st) {
    const int gn = g + 1 < nsteps ? g + 1 : g;
    load_b(gn);
    load_a(nxt, gn);
    mfma(cur, st);
    store_b(st ^ 1);
    __syncthreads();
  };
  load_b(0);
  store_b(0);
  load_a(R0, 0);
  __syncthreads();
  int g = 0;
  for (; g + 2 <= nsteps; g += 2) {
    step(R0, R1, g, 0);
    step(R1, R0, g + 1, 1);
  }
  if (g < nsteps) step(R0, R1, g, 0);
}

// Variant whose B operand is stored K-major: B(b, k) is the element at
// (k * ldb + b) of a row-major [K x ldb] matrix, e.g. the logit gradients
// G [tokens x vocabulary] when the product runs over tokens (dW = G^T h).
// The 128 product rows of the tile are 128 consecutive columns of that
// matrix.  Each 64 x 128 slice (64 K rows of 128 columns, 16 KB) is copied
// into LDS as loaded: K row k at byte 256 k, its four 64-byte quarters
// permuted by XOR with k mod 4 so that the fragment reads below touch all 64
// banks.  The MFMA fragments come out of LDS through the gfx950 transposing
// load ds_read_b64_tr_b16.  Within each group of 16 lanes that load hands
// lane 4a + b the b-th 16-bit element of the 8-byte words addressed by lanes
// a, a + 4, a + 8, a + 12 of the group.  Lane (q, h) of the MFMA needs K rows
// 16 s + 8 h .. +7 of column q, so source lane S = 16 g + 4 j + a (g = S / 16)
// addresses K row 16 s + 8 (g / 2) + j (+ 4 for the second load) at column
// 32 tb + 16 (g mod 2) + 4 a.
//   Bb:         byte address of element (k = 0, column b0) of the tile
//   ldb:        row stride of the K-major matrix, in elements (< 2^24)
//   k_valid:    K rows that exist (rows k_valid .. 64 nsteps - 1 read as 0)
//   cols_valid: columns of this tile that exist (a multiple of 8, <= 128)
template <int NTB, int NAB>
__device__ __forceinline__ void packed_tile_gemm_kmajor(f32x16 (&acc)[NTB][NAB],
                                                        u32x4 (&hs)[2][8 * kPkBRows],
                                                        const char* __restrict__ A0,
                                                        const char* __restrict__ A1,
                                                        const char* __restrict__ Bb, int64_t ldb,
                                                        int64_t k_valid, int cols_valid,
                                                        int nsteps) {
  static_assert(NAB == 2 && NTB * 32 == kPkBRows, "128 columns, two A row blocks per wavefront");
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tb][ab][r] = 0.f;

  const int tid = threadIdx.x, lane = tid & 63;
  // loads: K row tid / 16 + 16 j of the slice, 16-byte chunk tid % 16
  const int lrow = tid >> 4, lchunk = tid & 15;
  const bool col_ok = 8 * lchunk < cols_valid;
  uint32_t boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    boff[j] = static_cast<uint32_t>(((lrow + 16 * j) * ldb + 8 * lchunk) * 2);
  const int wslot = lrow * 16 + (lchunk ^ ((lrow & 3) << 2));   // + 256 j per row group
  // fragment reads: byte offset in a stage of (s = 0, load 0) for block tb
  const int g = lane >> 4, ja = (lane >> 2) & 3, aa = lane & 3;
  uint32_t roff[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
    roff[tb] = static_cast<uint32_t>((8 * (g >> 1) + ja) * 256 + 64 * (tb ^ ja) + 32 * (g & 1) + 8 * aa);
  const uint32_t aoff = static_cast<uint32_t>(lane) * 16u;
  const int64_t step_bytes = int64_t{kPkBK} * ldb * 2;

  u32x4 R0[NAB][4], R1[NAB][4], hr[4];
  auto load_a = [&](u32x4 (&dst)[NAB][4], int gs) {
    const char* a0 = A0 + static_cast<int64_t>(gs) * 4096;
    const char* a1 = A1 + static_cast<int64_t>(gs) * 4096;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      dst[0][s] = *reinterpret_cast<const u32x4*>(a0 + aoff + s * 1024);
      dst[1][s] = *reinterpret_cast<const u32x4*>(a1 + aoff + s * 1024);
    }
  };
  auto load_b = [&](int gs) {
    const char* base = Bb + gs * step_bytes;
    const int64_t k0 = static_cast<int64_t>(gs) * kPkBK + lrow;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hr[j] = u32x4{0u, 0u, 0u, 0u};
      if (col_ok && k0 + 16 * j < k_valid) hr[j] = *reinterpret_cast<const u32x4*>(base + boff[j]);
    }
  };
  auto store_b = [&](int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hs[st][wslot + 256 * j] = hr[j];
  };
  auto mfma = [&](const u32x4 (&cur)[NAB][4], int st) {
    const char* stage = reinterpret_cast<const char*>(&hs[st][0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 b[NTB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const char* p = stage + roff[tb] + 16 * s * 256;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 256));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        b[tb] = __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
      }
#pragma unroll
      for (int ab = 0; ab < NAB; ++ab) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, cur[ab][s]);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[tb][ab] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[tb], acc[tb][ab], 0, 0, 0);
      }
    }
  };
  auto step = [&](const u32x4 (&cur)[NAB][4], u32x4 (&nxt)[NAB][4], int gs, int st) {
    const int gn = gs + 1 < nsteps ? gs + 1 : gs;
    load_b(gn);
    load_a(nxt, gn);
    mfma(cur, st);
    store_b(st ^ 1);
    __syncthreads();
  };
  load_b(0);
  store_b(0);
  load_a(R0, 0);
  __syncthreads();
  int gs = 0;
  for (; gs + 2 <= nsteps; gs += 2) {
    step(R0, R1, gs, 0);
    step(R1, R0, gs + 1, 1);
  }
  if (gs < nsteps) step(R0, R1, gs, 0);
}

}  // namespace nel
