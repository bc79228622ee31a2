// Main loop of the head GEMM at one wavefront per SIMD (device side).
//
// A workgroup of 4 wavefronts computes a 128 x 512 tile of C = B A^T, B the
// 128 token rows of h_m and A 512 rows of the packed head W^m.  Each
// wavefront owns a 128 x 128 block: 8 x 8 blocks of 16 x 16 on
// v_mfma_f32_16x16x32_bf16, 256 fp32 accumulators per lane (the whole AGPR
// file, hence one wavefront per SIMD).  A 128 x 128 block per wavefront moves
// 0.25 KB of operands into registers per matrix instruction, against 0.375 KB
// for a 128 x 64 block.
//
//  * A (W^m in the 16-row tiled layout): each wavefront streams its 8 row
//    blocks straight into registers.  One register set: the 1 KB block
//    (ab, kh) of a K step is reloaded with the next step's block right after
//    the 8 matrix instructions that read it, so every load has a whole step
//    of matrix work ahead of its use.
//  * B (h_m, row-major): each K step's 128 x 64 slice is staged in a ring of
//    three 16 KB LDS stages, chunk-major (row t, 16-byte chunk c in slot
//    128 c + (t ^ 2 c): 16 consecutive rows of a fragment read, and 2 rows x
//    8 chunks of a write, each cover all 64 banks).  A thread's 4 chunks of a
//    slice are loaded two register sets deep: the loads for step g + 3 go out
//    in the second half of step g and are stored into the ring in the middle
//    of step g + 1.  The fragments are double buffered: the next half step's
//    8 are read from LDS while this half step's instructions run.
//  * Loads are buffer loads: the wave-uniform K offset is a scalar operand and
//    the lane offsets are computed once, so no vector instruction computes an
//    address in the loop; a load outside the resource's byte range returns
//    zero, which covers token rows beyond n and vocabulary rows beyond V.
//  * One barrier per K step.  Stage (g + 2) mod 3 is written in step g after
//    the barrier of step g - 1 (every read of step g - 1 is done) and is first
//    read in step g + 1's second half, after the barrier of step g.  That
//    barrier waits only for the LDS writes, which were issued half a step
//    earlier, not for the 8 fragment reads issued after them.
//  * Between the groups of 8 matrix instructions the scheduling barriers pin
//    the loads: per group at most one W block, one fragment read and one h
//    chunk, spread evenly over the step.
//
// Layout of the accumulators: acc[tb][ab] is the 16 x 16 block of token rows
// 16 tb .. and A rows 16 ab .. of the wavefront; lane l holds token row
// 16 tb + (l mod 16) and the 4 consecutive A rows 16 ab + 4 (l / 16) + i,
// i = accumulator register.
#pragma once
#include "common.h"

namespace nel {

constexpr int kW128Threads = 256;   // 4 wavefronts
constexpr int kW128Tok = 128;       // token rows (B) per workgroup
constexpr int kW128Voc = 512;       // A rows per workgroup (128 per wavefront)
constexpr int kW128Slots = 8 * kW128Tok;   // 16-byte LDS slots per stage
constexpr int kW128Stages = 3;

typedef __amdgpu_buffer_rsrc_t buf_rsrc;

// Cache-policy operand of a nontemporal buffer access (the "nt" bit).
constexpr int kBufNontemporal = 2;

// Raw buffer resource over `bytes` bytes from `base` (clamped to 32 bits).
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(static_cast<uint32_t>(b)), 0x00020000);
}

// Operands of one workgroup tile.
struct W128Operands {
  buf_rsrc h;          // the tile's token rows of h_m (row t0 at byte 0), rows beyond n excluded
  buf_rsrc w;          // the wavefront's first packed row block of W^m, blocks beyond V excluded
  uint32_t hoff[4];    // the thread's h chunks in K step 0: rows brow + 32 j, chunk bchunk
  uint32_t woff[8];    // the lane's 16 bytes of row block ab in K block 0
};

// Thread -> h chunk map: chunk i = tid + 256 j of a 128 x 64 slice is row
// i / 8 = tid / 8 + 32 j, chunk i % 8, at slot 128 c + (t ^ 2c) = hslot + 32 j.
__device__ __forceinline__ void w128_lanes(int tid, int d, W128Operands& op, int& hslot) {
  const int bchunk = tid & 7, brow = tid >> 3;
  hslot = bchunk * kW128Tok + (brow ^ (2 * bchunk));
#pragma unroll
  for (int j = 0; j < 4; ++j)   // unsigned: 128 rows of d < 2^24 entries stay below 2^32 bytes
    op.hoff[j] = static_cast<uint32_t>(brow + 32 * j) * static_cast<uint32_t>(d) * 2u +
                 static_cast<uint32_t>(bchunk) * 16u;
  const uint32_t lane = tid & 63;
#pragma unroll
  for (int ab = 0; ab < 8; ++ab) op.woff[ab] = static_cast<uint32_t>(ab) * d * 32u + lane * 16u;
}

// acc = W(the wavefront's 128 rows) x h(the tile's 128 rows)^T over K = 64 nsteps.
// stage: the workgroup's kW128Stages * kW128Slots LDS slots.  Every wavefront
// of the workgroup calls this together; it ends with a full barrier, after
// which the stages are free.
__device__ __forceinline__ void w128_tile_gemm(f32x4 (&acc)[8][8], u32x4* stage,
                                               const W128Operands& op, int hslot, int nsteps) {
  constexpr int NB = 8;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb)
#pragma unroll
    for (int ab = 0; ab < NB; ++ab) acc[tb][ab] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  int fsl[2];   // slot of fragment row x, chunk 4 kh + g (token block tb: + 16 tb)
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int c = 4 * kh + g;
    fsl[kh] = kW128Tok * c + (x ^ (2 * c));
  }
  u32x4 R[NB][2], hr[2][4];
  bf16x8 b[2][NB];
  auto ld_w = [&](int ab, int kh, int gs) {
    R[ab][kh] = __builtin_amdgcn_raw_buffer_load_b128(op.w, op.woff[ab] + kh * 1024, gs * 2048, 0);
  };
  auto ld_h = [&](int set, int j, int gs) {
    hr[set][j] = __builtin_amdgcn_raw_buffer_load_b128(op.h, op.hoff[j], gs * 128, 0);
  };
  auto st_h = [&](int set, int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) stage[st * kW128Slots + hslot + 32 * j] = hr[set][j];
  };
  const int last = nsteps - 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) ld_h(0, j, 0);
  st_h(0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) ld_h(1, j, min(1, last));
  st_h(1, 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) ld_h(0, j, min(2, last));
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int ab = 0; ab < NB; ++ab) ld_w(ab, kh, 0);
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) b[0][tb] = __builtin_bit_cast(bf16x8, stage[fsl[0] + 16 * tb]);
  // Step gi reads stage st and h register set hs holds step gi + 2's slice.
  auto step = [&](int gi, int st, int hs) {
    const int gw = min(gi + 1, last), gh = min(gi + 3, last);
    const int nst = st == 2 ? 0 : st + 1;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int ab = 0; ab < NB; ++ab) {
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
          acc[tb][ab] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, R[ab][kh]), b[kh][tb], acc[tb][ab], 0, 0, 0);
        ld_w(ab, kh, gw);
        // next half step's fragment ab (fragments are indexed by token block)
        const int idx = kh == 0 ? st * kW128Slots + fsl[1] + 16 * ab
                                : nst * kW128Slots + fsl[0] + 16 * ab;
        b[kh ^ 1][ab] = __builtin_bit_cast(bf16x8, stage[idx]);
        if (kh == 1 && ab < 4) ld_h(hs ^ 1, ab, gh);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kh == 0) {
        st_h(hs, st == 0 ? 2 : st - 1);   // (st + 2) mod 3
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the LDS writes above are done once at most the 8 fragment reads issued
    // after them are outstanding (LDS operations complete in order)
    asm volatile("s_waitcnt lgkmcnt(8)\n\ts_barrier" ::: "memory");
  };
  // unrolled by 6 so that the stage (mod 3) and h set (mod 2) are constants
  for (int gs = 0; gs < nsteps; gs += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u)
      if (gs + u < nsteps) step(gs + u, u % 3, u & 1);
  }
  __syncthreads();
}

}  // namespace nel
