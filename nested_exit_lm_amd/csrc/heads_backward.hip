// Backward of one exit head (bf16, gfx950): with G = dL/dl (the logit
// gradients) and l = h W^T (copyedit of Sec. 2 "Modeling": sub-model m ends
// in its own head W^m in R^{V x D}), the chain rule gives
//     dH = G W      [N x D] = sum over the vocabulary
//     dW = G^T h    [V x D] = sum over the tokens.
//     dH:  16x16x32 main loop of packed16_core.h (the head GEMM's): A = W^T
//          in the 16-row tiled layout (rows d, K = vocabulary), B = G
//          row-major (rows tokens, K = vocabulary contiguous)
//     dW:  32x32x16 K-major main loop of packed_core.h: A = h^T tiled (rows d,
//          K = tokens), B = G read K-major (rows vocabulary, K = tokens):
//          staged in LDS as stored and transposed by the LDS fragment loads,
//          so G is never copied
// Both outputs are row-major.  W^T and h^T are written tiled by one
// transposing pass each (HBM-bound, into the workspace; K zero-padded to a
// multiple of 64).
// The fused form reads no G: each thread forms its B chunks from the fp16
// scratch of the packed loss GEMM and 16-byte row constants per (vocabulary
// tile, token), with the arithmetic of the in-place gradient pass
// (grad_chunk.h), so G only ever exists in registers and LDS and the
// products equal those of the stored G bit for bit.
#include <cstdint>

#include "common.h"
#include "grad_chunk.h"
#include "internal.h"
#include "packed16_core.h"
#include "packed_core.h"
#include "tiles.h"

namespace nel {

namespace {

constexpr int kBwdGroup = 8;   // B tiles per tile group (see tile_coords)

// ---------------------------------------------------------------- packing
// Tiled A operand of S^T for S [k_rows, R] row-major (R % 64 == 0): element
// (r, k) = S[k][r] for k < k_rows, 0 up to k_pad.  One workgroup per 64 x 64
// tile: rows k0..k0+63 of S are read whole (128-byte pieces) into LDS, then
// every thread writes two 16-byte lane slots of the tile's eight 1 KB blocks,
// reading its 8 elements down an LDS column.
__global__ __launch_bounds__(256) void pack_t_kernel(const bf16_t* __restrict__ S,
                                                     bf16_t* __restrict__ P, int64_t k_rows,
                                                     int R, int64_t k_pad, int r_tiles) {
  __shared__ bf16_t tile[64][64 + 2];   // +2: row pitch 132 bytes spreads the column reads
  const int tid = threadIdx.x;
  const int rt = static_cast<int>(blockIdx.x % r_tiles);
  const int64_t kt = blockIdx.x / r_tiles;
  const int r0 = rt * 64;
  const int64_t k0 = kt * 64;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + 256 * j, row = i >> 3, ch = i & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + row < k_rows)
      v = *reinterpret_cast<const u32x4*>(S + (k0 + row) * R + r0 + ch * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[row][ch * 8]);
#pragma unroll
    for (int w = 0; w < 4; ++w) dst[w] = v[w];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + 256 * j;          // 512 lane slots: block (rbl, kpl), lane l
    const int l = i & 63, blk = i >> 6;   // blk 0..7
    const int rbl = blk & 1, kpl = blk >> 1;
    const int r = 32 * rbl + vperm(l & 31);
    const int kk = 16 * kpl + 8 * (l >> 5);
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      v[w] = static_cast<uint32_t>(tile[kk + 2 * w][r]) |
             (static_cast<uint32_t>(tile[kk + 2 * w + 1][r]) << 16);
    const int64_t rb = r0 / 32 + rbl, kp = k0 / 16 + kpl;
    *reinterpret_cast<u32x4*>(P + ((rb * (k_pad / 16) + kp) * 64 + l) * 8) = v;
  }
}

// 16-row tiled A operand of S^T (packed16_core.h) for S [k_rows, R]
// row-major (R % 64 == 0): element (r, k) = S[k][r] for k < k_rows, 0 up to
// k_pad, at P[((rb * (k_pad / 32) + kb) * 64 + l) * 8 + j] for r = 16 rb +
// (l mod 16), k = 32 kb + 8 (l / 16) + j.  One workgroup per 64 x 64 tile:
// rows k0..k0+63 of S are read whole into LDS, then every thread writes two
// 16-byte lane slots of the tile's eight 1 KB blocks, reading its 8 elements
// down an LDS column (16 lanes take 16 adjacent columns, the four lane groups
// rows 8 apart: 32 distinct banks).
__global__ __launch_bounds__(256) void pack16_t_kernel(const bf16_t* __restrict__ S,
                                                       bf16_t* __restrict__ P, int64_t k_rows,
                                                       int R, int64_t k_pad, int r_tiles) {
  __shared__ bf16_t tile[64][64 + 2];
  const int tid = threadIdx.x;
  const int rt = static_cast<int>(blockIdx.x % r_tiles);
  const int64_t kt = blockIdx.x / r_tiles;
  const int r0 = rt * 64;
  const int64_t k0 = kt * 64;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + 256 * j, row = i >> 3, ch = i & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + row < k_rows)
      v = *reinterpret_cast<const u32x4*>(S + (k0 + row) * R + r0 + ch * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[row][ch * 8]);
#pragma unroll
    for (int w = 0; w < 4; ++w) dst[w] = v[w];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = tid + 256 * j;          // 512 lane slots: block (rbl, kbl), lane l
    const int l = i & 63, blk = i >> 6;   // blk 0..7
    const int rbl = blk & 3, kbl = blk >> 2;
    const int r = 16 * rbl + (l & 15);
    const int kk = 32 * kbl + 8 * (l >> 4);
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      v[w] = static_cast<uint32_t>(tile[kk + 2 * w][r]) |
             (static_cast<uint32_t>(tile[kk + 2 * w + 1][r]) << 16);
    const int64_t rb = r0 / 16 + rbl, kb = k0 / 32 + kbl;
    *reinterpret_cast<u32x4*>(P + ((rb * (k_pad / 32) + kb) * 64 + l) * 8) = v;
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t count) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.f;
}

// ---------------------------------------------------------------- fused B
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// {c, k} of a row constant record (the label's entry and term are read once
// per row where the row does not change).
__device__ __forceinline__ u32x2 load_c_k(const GradRowConst* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// B = G of one exit, rows = tokens, K = vocabulary (dh = G W), NCH chunks
// per thread.  A K step (64 entries) lies inside one statistics tile (at
// least 128 wide).
template <int NCH>
struct BRowsGrad {
  static constexpr int kChunks = NCH;
  const char* S;              // exit's scratch at the tile's token row 0 (bytes)
  const char* W;              // the teacher's weights, same place
  const GradRowConst* tab;    // the exit's constants, [tile][n]
  int64_t n;
  int32_t row[NCH];           // tokens of the thread's chunks
  int32_t y[NCH];             // their labels
  float lab[NCH];             // and the label's terms
  uint32_t boff[NCH];         // byte offsets of the chunks at K step 0
  int vlane, vshift;          // first entry of the thread's chunk in a K step; log2 tile width
  uint32_t neg;               // grad_chunk's sign mask of the exit
  int gcur;
  u32x4 rs[NCH], rw[NCH];
  u32x2 k[NCH];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      y[j] = tab[row[j]].y;
      lab[j] = tab[row[j]].lab;
    }
  }
  __device__ __forceinline__ void issue(int g) {
    gcur = g;
    const int64_t off = static_cast<int64_t>(g) * (kPkBK * 2);
    const GradRowConst* t = tab + ((static_cast<int64_t>(g) * kPkBK) >> vshift) * n;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      rw[j] = *reinterpret_cast<const u32x4*>(W + off + boff[j]);
      rs[j] = *reinterpret_cast<const u32x4*>(S + off + boff[j]);
      k[j] = load_c_k(t + row[j]);
    }
  }
  __device__ __forceinline__ void finish(u32x4 (&hr)[NCH]) const {
    const int v0 = gcur * kPkBK + vlane;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      hr[j] = grad_chunk(rs[j], rw[j], __uint_as_float(k[j][0]), __uint_as_float(k[j][1]), lab[j],
                         label_offset(y[j], v0), neg);
  }
};

// B = G of one exit read K-major: K = tokens, the tile's 128 product rows =
// 128 vocabulary entries inside one statistics tile (dW = G^T h).  Tokens
// from n on read as 0.
struct BKMajorGrad {
  const char* S;              // exit's scratch at (token lrow, entry v0) (bytes)
  const char* W;              // the teacher's weights, same place
  const GradRowConst* tab;    // the exit's constants of the tile's statistics tile, [n]
  int64_t n, step_bytes;
  uint32_t rstride;           // bytes between the thread's K rows (16 rows)
  int lrow, v0;               // the thread's first K row; its chunk's first vocabulary entry
  bool col_ok;
  uint32_t neg;               // grad_chunk's sign mask of the exit
  unsigned valid;             // bit j: chunk j of the current step exists
  u32x4 rs[4], rw[4];
  u32x4 k[4];
  __device__ __forceinline__ void issue(int gs) {
    const int64_t base = gs * step_bytes;
    const int64_t k0 = static_cast<int64_t>(gs) * kPkBK + lrow;
    valid = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = k0 + 16 * j;
      if (col_ok && t < n) {
        valid |= 1u << j;
        rw[j] = *reinterpret_cast<const u32x4*>(W + base + j * rstride);
        rs[j] = *reinterpret_cast<const u32x4*>(S + base + j * rstride);
        k[j] = *reinterpret_cast<const u32x4*>(tab + t);
      } else {
        rw[j] = rs[j] = u32x4{0u, 0u, 0u, 0u};
        k[j] = u32x4{0u, 0u, 0u, ~0u};   // finite constants, no label
      }
    }
  }
  __device__ __forceinline__ void finish(u32x4 (&hr)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // every lane forms the chunk (grad_chunk's wavefront vote); a missing
      // one has finite inputs (issue zeroes them)
      const u32x4 v = grad_chunk(rs[j], rw[j], __uint_as_float(k[j][0]), __uint_as_float(k[j][1]),
                                 __uint_as_float(k[j][2]), label_offset(k[j][3], v0), neg);
      hr[j] = (valid & (1u << j)) ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
};

// ---------------------------------------------------------------- dh GEMM
// dh[t][d] = sum_v G[t][v] W[v][d] for t < b_rows (tokens), d < a_rows, on
// the head GEMM's main loop: A = W^T in the 16-row tiled layout (K = V),
// B = the token rows of G (row stride ldb), or with FUSED the gradients formed
// from the scratch.  Tile 128 tokens x 256 columns of d.  FUSED runs one
// workgroup per CU: forming the gradients beside the accumulators takes more
// than the 256 registers per lane of two (measured: spills inside the main
// loop at two, and a slower eight-wavefront variant).  One launch covers a
// group of exits: workgroup ids are split by the prefix sums `first` of the
// exits' tile counts, so one exit's workgroups fill another's last partial
// round.  The bf16 outputs leave through a wave-local LDS transpose: a lane
// holds four consecutive d of one token per 16 x 16 block and the
// wavefront's 64 d of a token are one 128-byte line, so after the transpose
// eight lanes store each whole line (nontemporal).  Row r, 16-byte chunk c
// of a wavefront's 32-token stage sits at slot 8 r + (c ^ ((r / 2) mod 8)).
template <bool FUSED>
__global__ __launch_bounds__(kPkThreads, FUSED ? 1 : 2) void dh16_kernel(
    BwdGroup /*read through the kernarg pointer*/) {
  constexpr int NCH = 8 * kPkBRows / kPkThreads;   // B chunks per thread
  const BwdGroup& g = *(const BwdGroup*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ u32x4 hs[2][16 * kPkBRows];
  int e = 0;
  while (e + 1 < g.count && static_cast<int>(blockIdx.x) >= g.first[e + 1]) ++e;
  const char* __restrict__ A = reinterpret_cast<const char*>(g.A[e]);
  const bf16_t* __restrict__ B = g.B[e];
  char* __restrict__ out = static_cast<char*>(g.out[e]);
  const int a_rows = g.a_rows[e];
  const int64_t b_rows = g.b_rows[e], ldb = g.ldb[e], K = g.K[e], ldo = g.ldo[e];
  const int tid = threadIdx.x, lane = tid & 63, x = lane & 15, gq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bt, at;
  tile_coords(static_cast<int>(blockIdx.x) - g.first[e], g.n_bt[e], g.n_at[e], kBwdGroup, bt, at);
  const int64_t b0 = static_cast<int64_t>(bt) * kPkBRows;
  const int aw = at * kPkARows + wave * 64;   // this wavefront's first column of d
  const char* Ab[k16NAB];
#pragma unroll
  for (int ab = 0; ab < k16NAB; ++ab)
    Ab[ab] = A + static_cast<int64_t>(min((aw >> 4) + ab, a_rows / 16 - 1)) * (K / 32) * 1024;
  const PackedLanes pl = packed_lanes(tid);
  uint32_t boff[NCH];
  int64_t rows[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    rows[j] = min(b0 + pl.brow + 32 * j, b_rows - 1);
    boff[j] = static_cast<uint32_t>(((rows[j] - b0) * ldb + pl.bchunk * 8) * 2);
  }
  const int64_t tile_off = b0 * ldb * 2;
  const int nsteps = static_cast<int>(K / kPkBK);
  f32x4 acc[k16NTB][k16NAB];
  if constexpr (FUSED) {
    BRowsGrad<NCH> src;
    src.S = reinterpret_cast<const char*>(B) + tile_off;
    src.W = reinterpret_cast<const char*>(g.tw) + tile_off;
    src.tab = static_cast<const GradRowConst*>(g.tab[e]);
    src.n = g.n_tok;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      src.row[j] = static_cast<int32_t>(rows[j]);
      src.boff[j] = boff[j];
    }
    src.vlane = 8 * pl.bchunk;
    src.vshift = g.vshift;
    src.neg = g.neg[e];
    src.init();
    packed16_tile_gemm(acc, hs, Ab, src, pl.hslot, nsteps);
  } else {
    BRowsPlain<NCH> src;
    src.Bb = reinterpret_cast<const char*>(B) + tile_off;
#pragma unroll
    for (int j = 0; j < NCH; ++j) src.boff[j] = boff[j];
    packed16_tile_gemm(acc, hs, Ab, src, pl.hslot, nsteps);
  }
  char* const stage = reinterpret_cast<char*>(&hs[0][0]) + wave * 4096;
  const bool col_ok = aw < a_rows;   // a_rows % 64 == 0: all 64 columns or none
  const int ch = lane & 7;
  // 32-bit lane offsets from a wave-uniform row base (ldo is below 2^22)
  const uint32_t loff = (static_cast<uint32_t>(lane >> 3) * static_cast<uint32_t>(ldo) +
                         static_cast<uint32_t>(aw + 8 * ch)) * 2u;
#pragma unroll
  for (int tp = 0; tp < k16NTB / 2; ++tp) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tb = 2 * tp + u, row = 16 * u + x;
#pragma unroll
      for (int ab = 0; ab < k16NAB; ++ab) {
        // d = 16 ab + 4 gq .. + 3 of the row: chunk 2 ab + gq / 2, half gq % 2
        const int c = 2 * ab + (gq >> 1);
        *reinterpret_cast<uint2*>(stage + (8 * row + (c ^ ((row >> 1) & 7))) * 16 + 8 * (gq & 1)) =
            make_uint2(pack_bf16x2(acc[tb][ab][0], acc[tb][ab][1]),
                       pack_bf16x2(acc[tb][ab][2], acc[tb][ab][3]));
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * j + (lane >> 3);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (8 * row + (ch ^ ((row >> 1) & 7))) * 16);
      const int64_t r0 = b0 + 32 * tp + 8 * j;   // this store's first token
      if (col_ok && r0 + (lane >> 3) < b_rows)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + r0 * ldo * 2 + loff));
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------- dW GEMM
// dW[v][d] = sum_t G[t][v] h[t][d]: out[b][a] = sum_k A[a][k] B(b, k) with
// A = h^T tiled for the 32x32x16 loop (a_rows = d, K = padded tokens,
// launch_pack_t) and B the exit's G, read K-major (b = vocabulary entry,
// k = token; K rows from k_valid read as 0) and formed from its scratch
// (g.B[e]) and the teacher's (g.tw); fp32 output.  Grouped over the exits
// like dh16_kernel.  The gradients it forms are those the loss pass stores,
// so its dW differs from the stored-gradient one only by the fp32 summation
// order of the same products.
__global__ __launch_bounds__(kPkThreads, 2) void dw_fused_kernel(
    BwdGroup /*read through the kernarg pointer*/) {
  // Per-product fields are read through the kernarg segment pointer, which
  // keeps the lookups by a run-time product index scalar.
  const BwdGroup& g = *(const BwdGroup*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int NTB = kPkNTB, NAB = kPkNAB;
  __shared__ u32x4 hs[2][8 * kPkBRows];
  int e = 0;
  while (e + 1 < g.count && static_cast<int>(blockIdx.x) >= g.first[e + 1]) ++e;
  const bf16_t* __restrict__ A = g.A[e];
  const bf16_t* __restrict__ B = g.B[e];
  float* __restrict__ out = static_cast<float*>(g.out[e]);
  const int a_rows = g.a_rows[e];
  const int64_t b_rows = g.b_rows[e], ldb = g.ldb[e], K = g.K[e], ldo = g.ldo[e];
  const int tid = threadIdx.x, lane = tid & 63, q = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bt, at;
  tile_coords(static_cast<int>(blockIdx.x) - g.first[e], g.n_bt[e], g.n_at[e], kBwdGroup, bt, at);
  const int64_t b0 = static_cast<int64_t>(bt) * kPkBRows;
  const int aw = at * kPkARows + wave * (NAB * 32);   // this wavefront's first A row
  const int rb0 = min(aw >> 5, a_rows / 32 - 1), rb1 = min((aw >> 5) + 1, a_rows / 32 - 1);
  const char* Ab = reinterpret_cast<const char*>(A);
  f32x16 acc[NTB][NAB];
  const char* A0 = Ab + static_cast<int64_t>(rb0) * 64 * K;
  const char* A1 = Ab + static_cast<int64_t>(rb1) * 64 * K;
  const int nsteps = static_cast<int>(K / kPkBK);
  const int cols = static_cast<int>(min(b_rows - b0, static_cast<int64_t>(kPkBRows)));
  const KMajorLanes kl = kmajor_lanes(tid);
  BKMajorGrad src;
  const int64_t off = (static_cast<int64_t>(kl.lrow) * ldb + b0 + 8 * kl.lchunk) * 2;
  src.S = reinterpret_cast<const char*>(B) + off;
  src.W = reinterpret_cast<const char*>(g.tw) + off;
  src.tab = static_cast<const GradRowConst*>(g.tab[e]) + (b0 >> g.vshift) * g.n_tok;
  src.n = g.k_valid[e];
  src.step_bytes = int64_t{kPkBK} * ldb * 2;
  src.rstride = static_cast<uint32_t>(16 * ldb * 2);
  src.lrow = kl.lrow;
  src.v0 = static_cast<int>(b0) + 8 * kl.lchunk;
  src.col_ok = 8 * kl.lchunk < cols;
  src.neg = g.neg[e];
  packed_tile_gemm_kmajor<NTB, NAB>(acc, hs, A0, A1, src, nsteps);
  // Stores leave through a wave-local LDS transpose, one 32-row block at a
  // time: a lane holds 16 consecutive outputs of one row, but the
  // wavefront's 64 fp32 outputs of a row are two whole 128-byte lines, so
  // after the transpose each store instruction writes whole lines,
  // nontemporal (nothing reads them back here).  The wavefront uses its own
  // 8 KB of the B stage, free since the main loop's last barrier.  Row r,
  // 16-byte chunk c sits at slot 16 r + (c ^ (r mod 16)); writes and reads
  // then cover all 64 banks.  Addresses: a wave-uniform 64-bit row base and
  // 32-bit lane offsets (the outputs' row length ldo is below 2^22).
  char* const stage = reinterpret_cast<char*>(&hs[0][0]) + wave * 8192;
  const bool col_ok = aw < a_rows;               // a_rows % 64 == 0: all 64 columns or none
  const int ch = lane & 15;
  const uint32_t loff = (static_cast<uint32_t>(lane >> 4) * static_cast<uint32_t>(ldo) +
                         static_cast<uint32_t>(aw + ch * 4)) * 4;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) {
      // (+ 0.0f: storing the accumulators unchanged made the register
      // allocator spill accumulator blocks inside the main loop)
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) {
        u32x4 pk;
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = __float_as_uint(acc[tb][ab][4 * h4 + j] + 0.0f);
        const int c = 8 * ab + 4 * hl + h4;
        *reinterpret_cast<u32x4*>(stage + (16 * q + (c ^ (q & 15))) * 16) = pk;
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + (lane >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (16 * row + (ch ^ (row & 15))) * 16);
      const int64_t r0 = b0 + 32 * tb + 4 * j;   // this store's first row
      char* rb = reinterpret_cast<char*>(out) + r0 * ldo * 4;
      if (col_ok && r0 + (lane >> 4) < b_rows)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(rb + loff));
    }
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------- dW GEMM
// The stored-gradient dW on the 16x16x32 K-major main loop (packed16_core.h):
// the product of dw_fused_kernel with B the stored G and A = h^T in the
// 16-row tiled layout (launch_pack16_t).  A wavefront owns 128 vocabulary rows x 64 columns of d.
// (The fused dW stays on dw_fused_kernel: forming the gradients beside
// this loop's operands needs more than the 256 registers of two workgroups
// per CU, and at one workgroup per CU it measured slower than the 32x32x16
// loop at two.)
// The fp32 outputs leave through a wave-local LDS transpose of one 16-row
// block at a time: a lane holds four consecutive d of one row per 16 x 16
// block, the wavefront's 64 d of a row are 256 contiguous bytes, and after
// the transpose 16 lanes store each row's 256 bytes (nontemporal).  Row r,
// 16-byte chunk c of the wavefront's 4 KB sits at slot 16 r + (c ^ r).
__global__ __launch_bounds__(kPkThreads, 2) void dw16_kernel(
    BwdGroup /*read through the kernarg pointer*/) {
  const BwdGroup& g = *(const BwdGroup*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ u32x4 hs[2][16 * kPkBRows];
  int e = 0;
  while (e + 1 < g.count && static_cast<int>(blockIdx.x) >= g.first[e + 1]) ++e;
  const char* __restrict__ A = reinterpret_cast<const char*>(g.A[e]);
  const bf16_t* __restrict__ B = g.B[e];
  char* __restrict__ out = static_cast<char*>(g.out[e]);
  const int a_rows = g.a_rows[e];
  const int64_t b_rows = g.b_rows[e], ldb = g.ldb[e], K = g.K[e], ldo = g.ldo[e];
  const int tid = threadIdx.x, lane = tid & 63, x = lane & 15, gq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bt, at;
  tile_coords(static_cast<int>(blockIdx.x) - g.first[e], g.n_bt[e], g.n_at[e], kBwdGroup, bt, at);
  const int64_t b0 = static_cast<int64_t>(bt) * kPkBRows;
  const int aw = at * kPkARows + wave * 64;   // this wavefront's first column of d
  const int cols = static_cast<int>(min(b_rows - b0, static_cast<int64_t>(kPkBRows)));
  const KMajorLanes kl = kmajor_lanes(tid);
  // the wavefront's 4 packed A row blocks (a wavefront beyond a_rows reads
  // the last 4 and stores nothing)
  const int rb0 = min(aw >> 4, a_rows / 16 - k16NAB);
  const uint32_t ablock = static_cast<uint32_t>((K / 32) * 1024);
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(A) + static_cast<int64_t>(rb0) * ablock, 0,
      static_cast<int>(k16NAB * ablock), 0x00020000);
  const int nsteps = static_cast<int>(K / kPkBK);
  f32x4 acc[k16NTB][k16NAB];
  BKMajorBuf src;
  src.Bb = reinterpret_cast<const char*>(B + b0);
  src.ldb = ldb;
  src.k_valid = g.k_valid[e];
  src.voff = 8 * kl.lchunk < cols ? static_cast<uint32_t>((kl.lrow * ldb + 8 * kl.lchunk) * 2)
                                   : 0x80000000u;   // beyond the step's byte range: reads as zero
  packed16_tile_gemm_kmajor(acc, hs, ar, ablock, src, nsteps);
  char* const stage = reinterpret_cast<char*>(&hs[0][0]) + wave * 4096;
  const bool col_ok = aw < a_rows;   // a_rows % 64 == 0: all 64 columns or none
  const int ch = lane & 15;
  // 32-bit lane offsets from a wave-uniform row base (ldo is below 2^22)
  const uint32_t loff = (static_cast<uint32_t>(lane >> 4) * static_cast<uint32_t>(ldo) +
                         static_cast<uint32_t>(aw + 4 * ch)) * 4u;
#pragma unroll
  for (int tb = 0; tb < k16NTB; ++tb) {
#pragma unroll
    for (int ab = 0; ab < k16NAB; ++ab) {
      // d = 16 ab + 4 gq .. + 3 of row x: chunk 4 ab + gq
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = __float_as_uint(acc[tb][ab][i] + 0.0f);
      *reinterpret_cast<u32x4*>(stage + (16 * x + ((4 * ab + gq) ^ x)) * 16) = pk;
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 4 * j + (lane >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (16 * row + (ch ^ row)) * 16);
      const int64_t r0 = b0 + 16 * tb + 4 * j;   // this store's first row
      if (col_ok && r0 + (lane >> 4) < b_rows)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + r0 * ldo * 4 + loff));
    }
    wave_lds_sync();
  }
}

}  // namespace

HeadBwdWs head_bwd_ws_layout(int64_t n, int vocab, int d) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  HeadBwdWs L;
  L.n_pad = (n + kPkBK - 1) / kPkBK * kPkBK;
  L.wt = 0;
  L.ht = L.wt + up(sizeof(bf16_t) * static_cast<size_t>(vocab) * d);
  L.total = L.ht + up(sizeof(bf16_t) * static_cast<size_t>(L.n_pad) * d);
  return L;
}

hipError_t launch_pack_t(const void* S, int64_t k_rows, int R, int64_t k_pad, void* P,
                         hipStream_t s) {
  const int r_tiles = R / 64;
  const int64_t tiles = static_cast<int64_t>(r_tiles) * (k_pad / 64);
  hipLaunchKernelGGL(pack_t_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(S), static_cast<bf16_t*>(P), k_rows, R, k_pad,
                     r_tiles);
  return hipGetLastError();
}

hipError_t launch_pack16_t(const void* S, int64_t k_rows, int R, int64_t k_pad, void* P,
                           hipStream_t s) {
  const int r_tiles = R / 64;
  const int64_t tiles = static_cast<int64_t>(r_tiles) * (k_pad / 64);
  hipLaunchKernelGGL(pack16_t_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(S), static_cast<bf16_t*>(P), k_rows, R, k_pad,
                     r_tiles);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t s) {
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, s, p, count);
  return hipGetLastError();
}

// Adds product (A, B) -> out to a group; false if the group is full.
bool bwd_group_add(BwdGroup& g, const void* A, int a_rows, const void* B, int64_t b_rows,
                   int64_t ldb, int64_t K, void* out, int64_t ldo, int64_t k_valid) {
  if (b_rows == 0) return true;   // nothing to compute
  if (g.count >= kMaxExits) return false;
  const int64_t n_bt = (b_rows + kPkBRows - 1) / kPkBRows;
  const int64_t n_at = (int64_t{a_rows} + kPkARows - 1) / kPkARows;
  if (g.first[g.count] + n_bt * n_at > INT32_MAX) return false;   // grid size is an int
  const int e = g.count++;
  g.A[e] = static_cast<const bf16_t*>(A);
  g.B[e] = static_cast<const bf16_t*>(B);
  g.out[e] = out;
  g.a_rows[e] = a_rows;
  g.b_rows[e] = b_rows;
  g.ldb[e] = ldb;
  g.K[e] = K;
  g.ldo[e] = ldo;
  g.k_valid[e] = k_valid < 0 ? K : k_valid;
  g.n_bt[e] = static_cast<int>(n_bt);
  g.n_at[e] = static_cast<int>(n_at);
  g.first[e + 1] = g.first[e] + g.n_bt[e] * g.n_at[e];
  return true;
}

template <bool FUSED>
hipError_t launch_dh_group(const BwdGroup& g, hipStream_t s) {
  if (g.count == 0 || g.first[g.count] == 0) return hipSuccess;
  hipLaunchKernelGGL((dh16_kernel<FUSED>), dim3(static_cast<unsigned>(g.first[g.count])),
                     dim3(kPkThreads), 0, s, g);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_dw_group(const BwdGroup& g, hipStream_t s) {
  if (g.count == 0 || g.first[g.count] == 0) return hipSuccess;
  if constexpr (FUSED)
    hipLaunchKernelGGL(dw_fused_kernel, dim3(static_cast<unsigned>(g.first[g.count])),
                       dim3(kPkThreads), 0, s, g);
  else
    hipLaunchKernelGGL(dw16_kernel, dim3(static_cast<unsigned>(g.first[g.count])),
                       dim3(kPkThreads), 0, s, g);
  return hipGetLastError();
}

template hipError_t launch_dh_group<false>(const BwdGroup&, hipStream_t);
template hipError_t launch_dh_group<true>(const BwdGroup&, hipStream_t);
template hipError_t launch_dw_group<false>(const BwdGroup&, hipStream_t);
template hipError_t launch_dw_group<true>(const BwdGroup&, hipStream_t);

}  // namespace nel
