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
//  * B (h_m, row-major): each K step's 128 x 64 slice goes straight from
//    memory into a ring of four 16 KB LDS stages (buffer loads that write
//    LDS, no registers), two steps ahead of its first use.  Stage layout:
//    row t, 16-byte chunk c at slot 8 t + (c ^ ((t / 2) mod 8)).  A load
//    instruction fills 64 consecutive slots (8 rows, every chunk of each, so
//    8 lanes read one row's 128 bytes), and the 16 rows of a fragment read
//    fall in 16 different bank groups.  The fragments are double buffered:
//    the next half step's 8 are read from LDS while this half step's
//    instructions run.
//  * Loads are buffer loads: the wave-uniform K offset is a scalar operand and
//    the lane offsets are computed once, so no vector instruction computes an
//    address in the loop; a load outside the resource's byte range returns
//    zero, which covers token rows beyond n and vocabulary rows beyond V.
//  * One barrier per K step.  Step g's slice is loaded at the start of step
//    g - 3 (the prologue loads steps 0 to 2) into stage g mod 4, last read in
//    step g - 4's first half, so every wavefront is past those reads (the
//    barrier of step g - 4).  It is first read in step g - 1's second half;
//    the barrier of step g - 2 waits for it (a fixed count of later loads may
//    still be outstanding: every step issues the same loads, past the last
//    step they re-read it).
//  * Scheduling barriers pin the order: a step's 4 stage loads at its start,
//    then after every group of 8 matrix instructions one W block and one
//    fragment read.
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
constexpr int kW128Stages = 4;

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
  uint32_t hoff[4];    // the lane's h chunk of stage load j in K step 0
  uint32_t woff[8];    // the lane's 16 bytes of row block ab in K block 0
};

// Stage load j of wavefront w fills slots 64 (4 w + j) + lane: row
// t = 32 w + 8 j + lane / 8 at position lane mod 8, i.e. chunk
// (lane mod 8) ^ ((t / 2) mod 8).
__device__ __forceinline__ void w128_lanes(int tid, int d, W128Operands& op) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {   // unsigned: 128 rows of d < 2^24 entries stay below 2^32 bytes
    const int t = 32 * w + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((t >> 1) & 7);
    op.hoff[j] = static_cast<uint32_t>(t) * static_cast<uint32_t>(d) * 2u + static_cast<uint32_t>(c) * 16u;
  }
#pragma unroll
  for (int ab = 0; ab < 8; ++ab) op.woff[ab] = static_cast<uint32_t>(ab) * d * 32u + lane * 16u;
}

// acc = W(the wavefront's 128 rows) x h(the tile's 128 rows)^T over K = 64 nsteps.
// stage: the workgroup's kW128Stages * kW128Slots LDS slots.  Every wavefront
// of the workgroup calls this together; it ends with a full barrier, after
// which the stages are free.
__device__ __forceinline__ void w128_tile_gemm(f32x4 (&acc)[8][8], u32x4* stage,
                                               const W128Operands& op, int nsteps) {
  constexpr int NB = 8;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb)
#pragma unroll
    for (int ab = 0; ab < NB; ++ab) acc[tb][ab] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  int fsl[2];   // slot of fragment row x, chunk 4 kh + g (token block tb: + 128 tb)
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) fsl[kh] = 8 * x + ((4 * kh + g) ^ ((x >> 1) & 7));
  u32x4 R[NB][2];
  bf16x8 b[2][NB];
  auto ld_w = [&](int ab, int kh, int gs) {
    R[ab][kh] = __builtin_amdgcn_raw_buffer_load_b128(op.w, op.woff[ab] + kh * 1024, gs * 2048, 0);
  };
  // Step gs's slice into stage st: 4 loads per wavefront, 1 KB of slots each
  // (lane l's 16 bytes go to the LDS address in m0 plus 16 l).  Written as
  // assembly so that the compiler, which cannot tell the stages apart, adds
  // no wait for these loads before every fragment read; the barrier of each
  // step waits for them instead.  The loads have no register destination,
  // and the compiler's own waits for the W registers stay correct (loads
  // complete in order; loads it does not know of only make them wait
  // longer).  m0 is saved and restored around the load, with the one wait
  // state a write of m0 needs before a load that reads it.
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                            (__attribute__((address_space(3))) u32x4*)(stage))) +
                        1024u * static_cast<uint32_t>(4 * wave);
  auto ld_stage = [&](int st, int gs) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
          "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(lds0 + static_cast<uint32_t>(st * kW128Slots * 16 + 1024 * j)), "v"(op.hoff[j]),
            "s"(op.h), "s"(gs * 128)
          : "memory");
    }
  };
  const int last = nsteps - 1;
  ld_stage(0, 0);
  ld_stage(1, min(1, last));
  ld_stage(2, min(2, last));
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int ab = 0; ab < NB; ++ab) ld_w(ab, kh, 0);
  // steps 0 and 1 have landed once at most step 2's 4 and the 16 W loads are outstanding
  asm volatile("s_waitcnt vmcnt(20)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) b[0][tb] = __builtin_bit_cast(bf16x8, stage[fsl[0] + 128 * tb]);
  // Step gi reads stage st = gi mod 4.
  auto step = [&](int gi, int st) {
    const int gw = min(gi + 1, last), gh = min(gi + 3, last);
    const int nst = (st + 1) & 3;
    ld_stage((st + 3) & 3, gh);
    __builtin_amdgcn_sched_barrier(0);
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
        const u32x4 v = kh == 0 ? stage[st * kW128Slots + fsl[1] + 128 * ab]
                            : stage[nst * kW128Slots + fsl[0] + 128 * ab];
        b[kh ^ 1][ab] = __builtin_bit_cast(bf16x8, v);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // step gi + 2's slice (loaded at the start of step gi - 1, or in the
    // prologue) has landed once at most the 16 W loads before this step, this
    // step's stage load and its 16 W loads are outstanding
    asm volatile("s_waitcnt vmcnt(36)\n\ts_barrier" ::: "memory");
  };
  // unrolled by 4 so that the stage is a constant
  for (int gs = 0; gs < nsteps; gs += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (gs + u < nsteps) step(gs + u, u);
  }
  __syncthreads();
}

}  // namespace nel
