// Main loop of the bf16 GEMMs on 16x16x32 matrix instructions whose A operand
// is in the 16-row tiled layout (device side; shared by the head GEMM and the
// head backward's dh GEMM).
//
// A workgroup of 4 wavefronts computes a 128 x 256 tile of C = B A^T:
//  * A: 256 rows (64 per wavefront, four 16-row blocks), packed so that every
//    matrix-instruction A operand is one contiguous 1 KB block: row block rb,
//    K block kb (32 columns) at byte (rb * K / 32 + kb) * 1024, lane l's 16
//    bytes at l * 16 holding row 16 rb + (l mod 16), columns
//    32 kb + 8 (l / 16) ... + 7.  Each wavefront loads its blocks straight into
//    registers.
//  * B: 128 rows with K contiguous, from a B source (packed_core.h: issue(g)
//    starts the loads of K step g, finish(hr) hands over the thread's four
//    16-byte chunks, rows tid / 8 + 32 j, chunk tid mod 8).  The workgroup
//    publishes each 128 x 64 slice in LDS chunk-major: row t, chunk c in slot
//    128 c + (t ^ 2 c), so the fragment reads of 16 consecutive rows and the
//    writes of 2 rows x 8 chunks each cover all 64 banks.
//  * C: acc[tb][ab] is the 16 x 16 block (B rows 16 tb.., A rows 16 ab..) of
//    the wavefront; lane l holds B row 16 tb + (l mod 16) and the 4
//    consecutive A rows 16 ab + 4 (l / 16) + i, i = accumulator register.
#pragma once
#include "common.h"
#include "packed_core.h"

namespace nel {

typedef __attribute__((ext_vector_type(4))) float f32x4;
constexpr int k16NTB = 8;   // B blocks of 16 rows per wavefront (128 rows)
constexpr int k16NAB = 4;   // A blocks of 16 rows per wavefront (64 rows)

// acc = A(this wavefront's 64 rows) x B(the workgroup's 128 rows)^T over
// K = 64 nsteps.
//   Ab[ab]: byte base of the wavefront's packed A row block ab
//   src:    the B source
//   hs:     the workgroup's two LDS stages of two K steps each
//   hslot:  packed_lanes(tid).hslot
// Every wavefront of the workgroup calls this together (it has barriers), and
// it ends with a barrier, after which the stages are free.
template <typename Src>
__device__ __forceinline__ void packed16_tile_gemm(f32x4 (&acc)[k16NTB][k16NAB],
                                                   u32x4 (&hs)[2][16 * kPkBRows],
                                                   const char* const (&Ab)[k16NAB], Src& src,
                                                   int hslot, int nsteps) {
  constexpr int NTB = k16NTB, NAB = k16NAB;
  constexpr int NCH = 8 * kPkBRows / kPkThreads;   // B chunks per thread per K step
  static_assert(NCH == Src::kChunks, "the source's chunks per thread");
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) acc[tb][ab] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  // LDS slot of B row x, chunk 4 kh + g (block tb: + 16 tb)
  int fsl[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int c = 4 * kh + g;
    fsl[kh] = 128 * c + (x ^ (2 * c));
  }
  const uint32_t aoff = static_cast<uint32_t>(lane) * 16u;
  // One set of A fragments: R[ab][kh] is reloaded for the next step as soon
  // as the current step's last matrix instruction that reads it has issued
  // (kh = 0 after the first half of the step, kh = 1 after the second), and
  // the B slice of two steps later is loaded at the start of the step, so
  // every load has at least half a step of this wavefront's matrix
  // instructions ahead of its first use without a second register set.  The
  // scheduling barriers keep that order.
  u32x4 R[NAB][2], hr[NCH];
  auto load_a = [&](int kh, int gs) {
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab)
      R[ab][kh] = *reinterpret_cast<const u32x4*>(Ab[ab] + static_cast<int64_t>(2 * gs + kh) * 1024 + aoff);
  };
  // chunk j of the thread: B row tid / 8 + 32 j, slot hslot + 32 j
  auto store_b = [&](int st, int q) {
    src.finish(hr);
#pragma unroll
    for (int j = 0; j < NCH; ++j) hs[st][1024 * q + hslot + 32 * j] = hr[j];
  };
  auto mfma = [&](int kh, int st, int q) {
    bf16x8 b[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
      b[tb] = __builtin_bit_cast(bf16x8, hs[st][1024 * q + fsl[kh] + 16 * tb]);
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, R[ab][kh]);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        acc[tb][ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[tb], acc[tb][ab], 0, 0, 0);
    }
  };
  // Steps go in pairs: stage st holds the B slices of steps 2p and 2p + 1
  // (sub-stages q = 0, 1), so the workgroup meets at a barrier once per two
  // steps.  Step g = 2p + q computes from sub-stage q while it loads the B
  // slice of step g + 2 (into the other stage's sub-stage q) and the A
  // fragments of step g + 1; loads past the last step re-read it.
  const int last = nsteps - 1;
  auto step = [&](int gi, int st, int q) {
    src.issue(min(gi + 2, last));
    __builtin_amdgcn_sched_barrier(0);
    mfma(0, st, q);
    __builtin_amdgcn_sched_barrier(0);
    load_a(0, min(gi + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    mfma(1, st, q);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, min(gi + 1, last));
    store_b(st ^ 1, q);
  };
  src.issue(0);
  store_b(0, 0);
  src.issue(min(1, last));
  store_b(0, 1);
  load_a(0, 0);
  load_a(1, 0);
  __syncthreads();
  int gs = 0, st = 0;
  for (; gs + 2 <= nsteps; gs += 2, st ^= 1) {
    step(gs, st, 0);
    step(gs + 1, st, 1);
    __syncthreads();
  }
  if (gs < nsteps) {   // an odd last step; the barrier frees LDS for the epilogue
    step(gs, st, 0);
    __syncthreads();
  }
}

// The same main loop with a K-major B operand: B(b, k) is element
// (k * ldb + b) of a row-major [K x ldb] matrix (the logit gradients G when
// the product runs over tokens, dW = G^T h).  Thread tid copies, per K step,
// 16-byte chunk tid % 16 of K rows tid / 16 + 16 j (kmajor_lanes).  Each
// 64 x 128 slice (16 KB) sits in LDS as loaded: K row k at byte 256 k, its
// 16-byte chunk c at position c ^ 4 (k mod 4) ^ 2 ((k / 8) mod 2) (the four
// 64-byte quarters permuted by k mod 4, the two 32-byte halves of each by
// bit 3 of k).  The fragments come out through the gfx950 transposing load
// ds_read_b64_tr_b16: within each 16 lanes it hands lane 4 a + b the b-th
// 16-bit element of the 8-byte words addressed by lanes a, a + 4, a + 8,
// a + 12.  Lane (x, g) of the instruction needs K rows 8 g .. + 7 of column x
// of a 16-column block tb, so source lane 4 j + a of group g addresses K row
// 8 g + j (+ 4 for the second load) at columns 16 tb + 4 a .. + 3; the two
// permutations put the four rows of a group in four quarters and the groups
// g, g + 1 that one LDS cycle serves in different halves.
//
//   a, ablock: a buffer resource over the wavefront's 4 packed A row blocks
//              and the bytes of one block (K / 32 KB); A loads are buffer
//              loads with the block offset as the scalar operand
//   src:       the B source (threads as kmajor_lanes assigns them): issue(g)
//              starts the loads of K step g, finish(hr) hands over the
//              thread's 4 chunks (K rows lrow + 16 j)
//
// K-major B as stored, through buffer loads: a resource per K step whose byte
// range ends at the last valid K row (rows beyond it read as zero), and a lane
// offset at or above 2^31 for a chunk beyond the tile's valid columns (zero
// as well), so no load sits under a condition.
struct BKMajorBuf {
  const char* Bb;          // byte address of element (k = 0, first column of the tile)
  int64_t ldb;             // row stride of B in elements (below 2^22)
  int64_t k_valid;         // K rows that exist
  uint32_t voff;           // the thread's chunk of K row lrow in K step 0; row lrow + 16 j: + 16 j ldb 2
  u32x4 r[4];
  __device__ __forceinline__ void issue(int gs) {
    const int64_t step_bytes = int64_t{kPkBK} * ldb * 2;
    const int64_t rows =
        min(max(k_valid - static_cast<int64_t>(gs) * kPkBK, int64_t{0}), int64_t{kPkBK});
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(Bb + gs * step_bytes), 0, static_cast<int>(rows * ldb * 2), 0x00020000);
    const uint32_t row16 = static_cast<uint32_t>(16 * ldb * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, j * row16, 0);
  }
  __device__ __forceinline__ void finish(u32x4 (&hr)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) hr[j] = r[j];
  }
};

template <typename Src>
__device__ __forceinline__ void packed16_tile_gemm_kmajor(f32x4 (&acc)[k16NTB][k16NAB],
                                                          u32x4 (&hs)[2][16 * kPkBRows],
                                                          const __amdgpu_buffer_rsrc_t& a,
                                                          uint32_t ablock, Src& src, int nsteps) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  constexpr int NTB = k16NTB, NAB = k16NAB;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) acc[tb][ab] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tid = threadIdx.x, lane = tid & 63;
  const KMajorLanes kl = kmajor_lanes(tid);
  // slot of the thread's chunk j = 0 (K row lrow); + 256 j for row lrow + 16 j
  const int wslot = kl.lrow * 16 + (kl.lchunk ^ ((kl.lrow & 3) << 2) ^ (((kl.lrow >> 3) & 1) << 1));
  // byte offset in a sub-stage of block tb's first load for K sub-step 0:
  // rbase ^ 32 tb (tb only flips the quarter and half bits)
  const int g = lane >> 4, ja = (lane >> 2) & 3, aa = lane & 3;
  const uint32_t rbase =
      static_cast<uint32_t>((8 * g + ja) * 256 + ((ja << 6) | ((g & 1) << 5) | (8 * aa)));
  u32x4 R[NAB][2], hr[4];
  const uint32_t aoff = static_cast<uint32_t>(lane) * 16u;
  auto load_a = [&](int kh, int gs) {
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab)
      R[ab][kh] = __builtin_amdgcn_raw_buffer_load_b128(a, aoff + kh * 1024, ab * ablock + gs * 2048, 0);
  };
  auto issue_b = [&](int gs) { src.issue(gs); };
  auto store_b = [&](int st, int q) {
    src.finish(hr);
#pragma unroll
    for (int j = 0; j < 4; ++j) hs[st][1024 * q + wslot + 256 * j] = hr[j];
  };
  auto mfma = [&](int kh, int st, int q) {
    const char* stage = reinterpret_cast<const char*>(&hs[st][1024 * q]) + kh * 8192;
    // one register for the 8 read offsets: the XOR is applied per read
    // rather than keeping 8 offsets live across the loop
    uint32_t rb = rbase;
    asm volatile("" : "+v"(rb));
    bf16x8 b[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const char* p = stage + (rb ^ (32u * tb));
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 256));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      b[tb] = __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
    }
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, R[ab][kh]);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        acc[tb][ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[tb], acc[tb][ab], 0, 0, 0);
    }
  };
  // The same schedule as packed16_tile_gemm: steps in pairs per LDS stage,
  // B of step g + 2 loaded at the start of step g, A of step g + 1 reloaded
  // half by half after the instructions that read it.
  const int last = nsteps - 1;
  auto step = [&](int gi, int st, int q) {
    issue_b(min(gi + 2, last));
    __builtin_amdgcn_sched_barrier(0);
    mfma(0, st, q);
    __builtin_amdgcn_sched_barrier(0);
    load_a(0, min(gi + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    mfma(1, st, q);
    __builtin_amdgcn_sched_barrier(0);
    load_a(1, min(gi + 1, last));
    store_b(st ^ 1, q);
  };
  issue_b(0);
  store_b(0, 0);
  issue_b(min(1, last));
  store_b(0, 1);
  load_a(0, 0);
  load_a(1, 0);
  __syncthreads();
  int gs = 0, st = 0;
  for (; gs + 2 <= nsteps; gs += 2, st ^= 1) {
    step(gs, st, 0);
    step(gs + 1, st, 1);
    __syncthreads();
  }
  if (gs < nsteps) {   // an odd last step; the barrier frees LDS for the epilogue
    step(gs, st, 0);
    __syncthreads();
  }
}

}  // namespace nel
