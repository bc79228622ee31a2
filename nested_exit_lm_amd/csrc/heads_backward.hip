// Backward of one exit head (bf16, gfx950): with G = dL/dl (the logit
// gradients) and l = h W^T (copyedit of Sec. 2 "Modeling": sub-model m ends
// in its own head W^m in R^{V x D}), the chain rule gives
//     dH = G W      [N x D] = sum over the vocabulary
//     dW = G^T h    [V x D] = sum over the tokens.
// Both run on the MFMA main loops of packed_core.h, whose A operand is
// MFMA-tiled:
//     dH:  A = W^T tiled (rows d, K = vocabulary),  B = G row-major (rows tokens,
//          K = vocabulary contiguous)
//     dW:  A = h^T tiled (rows d, K = tokens),      B = G read K-major (rows
//          vocabulary, K = tokens): staged in LDS as stored and transposed by
//          the LDS fragment loads, so G is never copied
// so each lane's accumulators are 16 consecutive d of one output row and the
// stores are row-major.  W^T and h^T are written tiled by one transposing
// pass each (HBM-bound, into the workspace; K zero-padded to a multiple of 64).
#include <cstdint>

#include "common.h"
#include "internal.h"
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

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t count) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.f;
}

// ---------------------------------------------------------------- GEMM
// out[b][a] = sum_k A[a][k] B[b][k] for a < a_rows, b < b_rows; A tiled
// (a_rows % 32 == 0, K % 64 == 0), B row-major with row stride ldb.  One
// launch covers a group of such products (the exits of a suite): workgroup
// ids are split by the prefix sums `first` of the products' tile counts, so
// one product's workgroups fill another's last partial round.
template <typename OutT, bool KMAJOR>
__global__ __launch_bounds__(kPkThreads, 2) void bwd_gemm_kernel(
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
  OutT* __restrict__ out = static_cast<OutT*>(g.out[e]);
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
  if constexpr (KMAJOR) {
    const int cols = static_cast<int>(min(b_rows - b0, static_cast<int64_t>(kPkBRows)));
    packed_tile_gemm_kmajor<NTB, NAB>(acc, hs, Ab + static_cast<int64_t>(rb0) * 64 * K,
                                      Ab + static_cast<int64_t>(rb1) * 64 * K,
                                      reinterpret_cast<const char*>(B + b0), ldb, g.k_valid[e],
                                      cols, static_cast<int>(K / kPkBK));
  } else {
    const PackedLanes pl = packed_lanes(tid);
    uint32_t boff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = min(b0 + pl.brow + 32 * j, b_rows - 1) - b0;
      boff[j] = static_cast<uint32_t>((row * ldb + pl.bchunk * 8) * 2);
    }
    const char* Bb = reinterpret_cast<const char*>(B) + b0 * ldb * 2;
    packed_tile_gemm<NTB, NAB>(acc, hs, Ab + static_cast<int64_t>(rb0) * 64 * K,
                               Ab + static_cast<int64_t>(rb1) * 64 * K, Bb, boff, pl,
                               static_cast<int>(K / kPkBK));
  }
  // Stores leave through a wave-local LDS transpose, one 32-row block at a
  // time: a lane holds 16 consecutive outputs of one row, but the
  // wavefront's 64 outputs of a row are whole 128-byte lines (bf16: one,
  // fp32: two), so after the transpose each store instruction writes whole
  // lines, nontemporal (nothing reads them back here).  The wavefront uses
  // its own 8 KB of the B stage, free since the main loop's last barrier.
  // Row r, 16-byte chunk c sits at slot CPR r + (c ^ swizzle(r)), CPR chunks
  // per row; writes and reads then cover all 64 banks.  Addresses: a
  // wave-uniform 64-bit row base and 32-bit lane offsets (the outputs' row
  // length ldo is below 2^22).
  constexpr int ES = sizeof(OutT);
  constexpr int CPR = 64 * ES / 16;              // 16-byte chunks per row: 8 or 16
  constexpr int RPS = 64 / CPR;                  // rows per wavefront store: 8 or 4
  auto swz = [](int r) { return CPR == 8 ? (r >> 1) & 7 : r & 15; };
  char* const stage = reinterpret_cast<char*>(&hs[0][0]) + wave * 8192;
  const bool col_ok = aw < a_rows;               // a_rows % 64 == 0: all 64 columns or none
  const int ch = lane % CPR;
  const uint32_t loff = (static_cast<uint32_t>(lane / CPR) * static_cast<uint32_t>(ldo) +
                         static_cast<uint32_t>(aw + ch * (16 / ES))) * ES;
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
    for (int ab = 0; ab < NAB; ++ab) {
      if constexpr (ES == 2) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            pk[j] = pack_bf16x2(acc[tb][ab][8 * h2 + 2 * j], acc[tb][ab][8 * h2 + 2 * j + 1]);
          const int c = 4 * ab + 2 * hl + h2;
          *reinterpret_cast<u32x4*>(stage + (CPR * q + (c ^ swz(q))) * 16) = pk;
        }
      } else {
        // (+ 0.0f: storing the accumulators unchanged made the register
        // allocator spill accumulator blocks inside the main loop)
#pragma unroll
        for (int h4 = 0; h4 < 4; ++h4) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) pk[j] = __float_as_uint(acc[tb][ab][4 * h4 + j] + 0.0f);
          const int c = 8 * ab + 4 * hl + h4;
          *reinterpret_cast<u32x4*>(stage + (CPR * q + (c ^ swz(q))) * 16) = pk;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 32 / RPS; ++j) {
      const int row = RPS * j + lane / CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + (CPR * row + (ch ^ swz(row))) * 16);
      const int64_t r0 = b0 + 32 * tb + RPS * j;   // this store's first row
      char* rb = static_cast<char*>(static_cast<void*>(out)) + r0 * ldo * ES;
      if (col_ok && r0 + lane / CPR < b_rows)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(rb + loff));
    }
    __builtin_amdgcn_wave_barrier();
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

template <typename OutT, bool KMAJOR>
hipError_t launch_bwd_group(const BwdGroup& g, hipStream_t s) {
  if (g.count == 0 || g.first[g.count] == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_gemm_kernel<OutT, KMAJOR>), dim3(static_cast<unsigned>(g.first[g.count])),
                     dim3(kPkThreads), 0, s, g);
  return hipGetLastError();
}

template <typename OutT>
hipError_t launch_bwd_gemm(const void* A, int a_rows, const void* B, int64_t b_rows, int64_t ldb,
                           int64_t K, OutT* out, int64_t ldo, hipStream_t s) {
  BwdGroup g{};
  if (!bwd_group_add(g, A, a_rows, B, b_rows, ldb, K, out, ldo)) return hipErrorInvalidValue;
  return launch_bwd_group<OutT, false>(g, s);
}

template hipError_t launch_bwd_gemm<bf16_t>(const void*, int, const void*, int64_t, int64_t,
                                            int64_t, bf16_t*, int64_t, hipStream_t);
template hipError_t launch_bwd_gemm<float>(const void*, int, const void*, int64_t, int64_t,
                                           int64_t, float*, int64_t, hipStream_t);
template hipError_t launch_bwd_group<bf16_t, false>(const BwdGroup&, hipStream_t);
template hipError_t launch_bwd_group<float, false>(const BwdGroup&, hipStream_t);
template hipError_t launch_bwd_group<float, true>(const BwdGroup&, hipStream_t);

}  // namespace nel
