// Shared pieces of the bf16 GEMMs whose A operand is in an MFMA-tiled layout
// (device side): the tile geometry, the thread-to-chunk maps and plain B
// sources, and the 32x32x16 main loop with a K-major B operand (the fused
// head backward's dW GEMM).  The 16x16x32 main loops of the head GEMM, the dh
// GEMM and the stored-gradient dW GEMM are in packed16_core.h.
//
// The K-major loop: a workgroup of 4 wavefronts computes a 128 x 256 tile of
// C = B A^T:
//  * A: 256 rows (64 per wavefront, two 32-row blocks), packed so that every
//    MFMA A operand is one contiguous 1 KB block: row block rb, K block kp
//    (16 columns) at byte (rb * K / 16 + kp) * 1024, lane l's 16 bytes at
//    l * 16 holding row 32 rb + vperm(l % 32), columns 16 kp + 8 (l / 32) ...+7.
//    Each wavefront loads its blocks straight into registers, one K step
//    (64 columns, 4 blocks per row block) ahead of the MFMAs.
//  * B: 128 columns of a K-major matrix (below).
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

// Row-major B: which 16-byte chunks of each 128 x 64 slice a thread copies,
// and where they go in the LDS stage (row t, chunk c in slot 128 c + (t ^ 2c)).
struct PackedLanes {
  int hslot;          // LDS slot of this thread's first B chunk (next: + 32 j)
  int brow, bchunk;   // B row and 16-byte chunk this thread loads (rows brow + 32 j)
};

__device__ __forceinline__ PackedLanes packed_lanes(int tid) {
  PackedLanes p;
  p.bchunk = tid & 7;
  p.brow = tid >> 3;
  // chunk i = tid + 256 j of the 128 x 64 slice is row i / 8 = tid / 8 + 32 j,
  // chunk i % 8; slot 128 c + (t ^ 2c) = hslot + 32 j (2c < 32 leaves bit 5 alone)
  p.hslot = p.bchunk * kPkBRows + (p.brow ^ (2 * p.bchunk));
  return p;
}

// B sources of the main loops.  Per K step a thread copies four 16-byte
// chunks of B into LDS: issue(g) starts the loads of step g before the
// step's matrix instructions, finish(hr) hands over the chunks after them.
//
// Row-major 16-bit B as stored; NCH chunks per thread.
template <int NCH = 4>
struct BRowsPlain {
  static constexpr int kChunks = NCH;
  const char* Bb;       // byte base of the tile's B row 0
  uint32_t boff[NCH];   // byte offsets from Bb of the thread's chunks (+128 per K step)
  u32x4 r[NCH];
  __device__ __forceinline__ void issue(int g) {
    const char* a = Bb + static_cast<int64_t>(g) * (kPkBK * 2);
#pragma unroll
    for (int j = 0; j < NCH; ++j) r[j] = *reinterpret_cast<const u32x4*>(a + boff[j]);
  }
  __device__ __forceinline__ void finish(u32x4 (&hr)[NCH]) const {
#pragma unroll
    for (int j = 0; j < NCH; ++j) hr[j] = r[j];
  }
};

// The B source's thread copies, per K step gs, 16-byte chunk tid % 16 of
// the slice's K rows tid / 16 + 16 j (KMajorLanes).
struct KMajorLanes {
  int lrow, lchunk;
};
__device__ __forceinline__ KMajorLanes kmajor_lanes(int tid) { return {tid >> 4, tid & 15}; }

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
//   src: the B source (threads as kmajor_lanes assigns them)
template <int NTB, int NAB, typename Src>
__device__ __forceinline__ void packed_tile_gemm_kmajor(f32x16 (&acc)[NTB][NAB],
                                                        u32x4 (&hs)[2][8 * kPkBRows],
                                                        const char* __restrict__ A0,
                                                        const char* __restrict__ A1, Src& src,
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
  const KMajorLanes kl = kmajor_lanes(tid);
  const int wslot = kl.lrow * 16 + (kl.lchunk ^ ((kl.lrow & 3) << 2));   // + 256 j per row group
  // fragment reads: byte offset in a stage of (s = 0, load 0) for block tb
  const int g = lane >> 4, ja = (lane >> 2) & 3, aa = lane & 3;
  uint32_t roff[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
    roff[tb] = static_cast<uint32_t>((8 * (g >> 1) + ja) * 256 + 64 * (tb ^ ja) + 32 * (g & 1) + 8 * aa);
  const uint32_t aoff = static_cast<uint32_t>(lane) * 16u;

  // One set of A fragments R[ab][s]: the half s = 2h, 2h + 1 is reloaded for
  // the next step right after the step's last matrix instruction that reads
  // it, and the B source's loads for the next step start with the step, so
  // every load has half a step of this wavefront's matrix instructions ahead
  // of its first use (the scheduling barriers keep that order).
  u32x4 R[NAB][4], hr[4];
  auto load_a = [&](int h, int gs) {
    const char* a0 = A0 + static_cast<int64_t>(gs) * 4096;
    const char* a1 = A1 + static_cast<int64_t>(gs) * 4096;
#pragma unroll
    for (int s = 2 * h; s < 2 * h + 2; ++s) {
      R[0][s] = *reinterpret_cast<const u32x4*>(a0 + aoff + s * 1024);
      R[1][s] = *reinterpret_cast<const u32x4*>(a1 + aoff + s * 1024);
    }
  };
  auto store_b = [&](int st) {
    src.finish(hr);
#pragma unroll
    for (int j = 0; j < 4; ++j) hs[st][wslot + 256 * j] = hr[j];
  };
  auto mfma = [&](int h, int st) {
    const char* stage = reinterpret_cast<const char*>(&hs[st][0]);
#pragma unroll
    for (int s = 2 * h; s < 2 * h + 2; ++s) {
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
        const bf16x8 a = __builtin_bit_cast(bf16x8, R[ab][s]);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[tb][ab] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[tb], acc[tb][ab], 0, 0, 0);
      }
    }
  };
  auto step = [&](int gs, int st) {
    const int gn = gs + 1 < nsteps ? gs + 1 : gs;
    src.issue(gn);
    __builtin_amdgcn_sched_barrier(0);
    mfma(0, st);
    __builtin_amdgcn_sched_barrier(0);
    load_a(0, gn);
    __builtin_amdgcn_sched_barrier(0);
    mfma(1, st);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, gn);
    store_b(st ^ 1);
    __syncthreads();
  };
  src.issue(0);
  store_b(0);
  load_a(0, 0);
  load_a(1, 0);
  __syncthreads();
  for (int gs = 0; gs < nsteps; ++gs) step(gs, gs & 1);
}

}  // namespace nel
