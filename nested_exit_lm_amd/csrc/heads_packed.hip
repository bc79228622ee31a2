// Multi-exit LM-head GEMM on MFMA-tiled head weights (bf16, gfx950).
//
// Same contraction and epilogues as the row-major head GEMM: every exit m's
// logits l_m = h_m W^m^T (copyedit of Sec. 2 "Modeling") in fp32 registers,
// turned into per-tile loss statistics for the distillation loss
// ("Matryoshka Language Model Suites", distillation paragraph) or into a
// per-tile greedy argmax; no fp32 logit tensor is written for the loss.
//
// Instruction: v_mfma_f32_16x16x32_bf16.  With W as the row operand and h as
// the column operand, lane l of a 16 x 16 block holds vocabulary rows
// 4 (l / 16) + i, i < 4, of token column l % 16 (checked on the device), so
// a lane's accumulator is four consecutive vocabulary entries of one token.
// On this chip the 16x16x32 shape sustains about 9 % more than 32x32x16 with
// the same operand traffic (main loop measured alone at the widest exit).
//
// Why a second weight layout.  A wavefront that keeps its vocabulary slice of
// W in registers needs no LDS for W at all; but the matrix-core operand puts
// 16 different W rows in consecutive lanes, and such strided row loads run at
// a third of the rate of contiguous ones.  So W is first rewritten
// (nel_pack_weights, one HBM-bound pass) into 1 KB blocks that are exactly one
// A operand each:
//     block (rb, kb), rb < V/16, kb < D/32, at element offset (rb * D/32 + kb) * 512;
//     lane l's 8 elements at l * 8 are W[16 rb + l % 16][32 kb + 8 (l / 16) + j],
// so every operand load is one contiguous 1 KB read.
//
// Loss and greedy-verify GEMMs: workgroups of 4 wavefronts, tile 128 tokens x
// 512 vocabulary entries, one workgroup per CU, on the main loop of
// wave128_core.h (W as the A operand straight into registers, h as the B
// operand staged through LDS, 128 x 128 per wavefront).  Exits of mean width
// below 512 (loss) and grids of fewer than two workgroups per CU (verify) run
// a 128 x 256 tile at two workgroups per CU on the main loop of
// packed16_core.h instead.
//
// Loss epilogue, per wavefront and token: the maximum m of its 128 logits,
// sum exp(l - m) and the label's logit (one statistics tile per wavefront),
// and one 16-bit copy of those 128 logits in the exit's gradient buffer, in
// fp16 (relative rounding 2^-11).  kModeLossF16 (the cross-entropy to the
// teacher): the teacher (the last exit) stores its weights
// w = exp(l_M - m), the smaller exits l - m; the row-wise gradient pass forms
// the teacher-weighted sums sum_v p_v l_m,v from them.  kModeLossPlain (the
// other divergences, whose pass reads every exit's l - m) stores l - m for
// every exit.  No epilogue reads another exit's tile back.
#include <limits.h>

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "packed16_core.h"
#include "packed_core.h"
#include "tiles.h"
#include "wave128_core.h"

namespace nel {

namespace {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kPkTok = kPkBRows;   // tokens per workgroup (the h rows)
constexpr int kPkVoc = kPkARows;   // vocabulary entries per workgroup
constexpr int kPkGroup = 8;        // token tiles per tile group (see tile_coords)
constexpr int kNTB = k16NTB;       // token blocks of 16 per wavefront
constexpr int kNVB = k16NAB;       // vocabulary blocks of 16 per wavefront

// ---------------------------------------------------------------- packing
// One workgroup per (16-row block rb, four 32-column blocks kb0 .. kb0 + 3):
// thread i reads row i / 16, 16-byte chunk i % 16 of the 256-byte row piece
// (whole rows per 16 lanes) and writes it to lane 16 (chunk % 4) + row of
// block kb0 + chunk / 4 (the four 1 KB blocks are filled together).
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ w,
                                                   bf16_t* __restrict__ p, int vocab, int d) {
  const int nkb = d / 32;
  const int units_per_rb = (nkb + 3) / 4;
  const int64_t units = static_cast<int64_t>(vocab / 16) * units_per_rb;
  const int x = threadIdx.x >> 4, c16 = threadIdx.x & 15;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t rb = u / units_per_rb;
    const int kb = static_cast<int>(u - rb * units_per_rb) * 4 + (c16 >> 2);
    if (kb >= nkb) continue;
    const int g = c16 & 3;
    const u32x4 v =
        *reinterpret_cast<const u32x4*>(w + (rb * 16 + x) * d + kb * 32 + g * 8);
    *reinterpret_cast<u32x4*>(p + ((rb * nkb + kb) * 64 + 16 * g + x) * 8) = v;
  }
}

// ---------------------------------------------------------------- loss GEMM
// One workgroup per (128-token tile, 512-entry vocabulary tile) runs every
// exit in turn, the teacher first, on the main loop of wave128_core.h (one
// wavefront per SIMD).  Wavefront w owns vocabulary entries [128 w, 128 w + 128)
// of the tile for all 128 tokens; lane (x, g) of block (tb, vb) holds token
// 16 tb + x and vocabulary entries 16 vb + 4 g .. + 3.
//
// The epilogue is local to the wavefront: its 128 entries of a row are one
// statistics tile (kW128StatTile), so no value crosses wavefronts and the
// epilogue has no workgroup barrier.  With one wavefront per SIMD nothing else
// runs beside it, so its cost counts in full.
constexpr int kW128StatTile = 128;

template <int MODE>
__global__ __launch_bounds__(kW128Threads, 1) void heads_loss_kernel(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    const int32_t* __restrict__ labels, float* __restrict__ stats, float* __restrict__ lab,
    int n_tt, int n_vt_wg, int n_st) {
  // The exit table is the first kernel argument; indexing it through the
  // kernarg segment pointer keeps per-exit lookups scalar.
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ u32x4 stage[kW128Stages * kW128Slots];
  // per wavefront: 32 token rows x 256 bytes of 16-bit values in transit
  __shared__ u32x4 outbuf[4][32 * 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tt, vt;
  tile_coords(blockIdx.x, n_tt, n_vt_wg, kPkGroup, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kW128Tok;
  const int vw = vt * kW128Voc + wave * 128;   // this wavefront's first vocabulary entry
  const int64_t plane = static_cast<int64_t>(n_st) * n;
  constexpr int NB = 8;

  f32x4 acc[NB][NB];
  for (int ei = 0; ei < n_exits; ++ei) {
    const int e = ei == 0 ? n_exits - 1 : ei - 1;
    const int D = ex.d[e];
    W128Operands op;
    w128_lanes(tid, D, op);
    op.h = make_rsrc(static_cast<const char*>(ex.h[e]) + t0 * D * 2, (n - t0) * D * 2);
    op.w = make_rsrc(static_cast<const char*>(ex.w[e]) + static_cast<int64_t>(vw >> 4) * D * 32,
                     static_cast<int64_t>(vocab / 16 - (vw >> 4)) * D * 32);
    w128_tile_gemm(acc, stage, op, D / 64);

    // Opaque copies of values that are the same for every exit keep the
    // compiler from hoisting the epilogue's per-lane offsets and predicates
    // out of the exit loop, where they would be live (and spilled) across
    // the main loop.
    int vwe = vw;
    int64_t t0e = t0;
    int lane = tid & 63;
    asm volatile("" : "+s"(vwe), "+s"(t0e), "+v"(lane));
    const int x = lane & 15, g = lane >> 4;
    // Per-token values go through buffer resources that cover the tile's
    // tokens below n (accesses beyond: loads read 0, stores are dropped),
    // with 32-bit lane offsets; a lane offset at or above 2^31 drops a store
    // (every resource here spans less than 2^31 bytes).  The labels of this
    // lane's 8 tokens are loaded ahead of their use.
    const int64_t n_left = n - t0e;
    const int tok_left = static_cast<int>(min(n_left, static_cast<int64_t>(kW128Tok)));
    const uint32_t toff = static_cast<uint32_t>(x) * 4u;   // token x of block 0, bytes
    const buf_rsrc lab_in = make_rsrc(labels + t0e, tok_left * 4);
    int ylab[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const int yy = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lab_in, toff, 64 * tb, 0));
      ylab[tb] = x + 16 * tb < tok_left ? yy : -1;
    }
    // vocabulary entries beyond V vanish under exp; V is a multiple of 32, so
    // a 16-block is wholly in or beyond V
    if (vwe + 128 > vocab) {
#pragma unroll
      for (int vb = 0; vb < NB; ++vb)
        if (vwe + 16 * vb >= vocab)
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) acc[tb][vb] = f32x4{kMasked, kMasked, kMasked, kMasked};
    }
    // this wavefront's statistics tile: the maxima, then (a plane further) the sums
    float* const st = stats + (static_cast<int64_t>(e) * 3 * n_st + (vwe >> 7)) * n + t0e;
    const buf_rsrc st_m = make_rsrc(st, tok_left * 4), st_s = make_rsrc(st + plane, tok_left * 4);
    const buf_rsrc lab_out = make_rsrc(lab + static_cast<int64_t>(e) * n + t0e, tok_left * 4);
    // (a wavefront wholly beyond V, in the last tile only, writes no statistics)
    const uint32_t st_off = g == 0 && vwe < vocab ? toff : 0x80000000u;
    bf16_t* __restrict__ O = static_cast<bf16_t*>(ex.out[e]);
    char* const ob = reinterpret_cast<char*>(&outbuf[wave][0]);
    // one instance per kind of exit, so that no branch sits inside the loops
    auto epilogue = [&](auto teacher_tag) {
      constexpr bool teacher = decltype(teacher_tag)::value;
#pragma unroll
      for (int tp = 0; tp < NB / 2; ++tp) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int tb = 2 * tp + u;
          // row maximum over the wavefront's 128 entries: a lane's 32, then
          // the four lane groups of its token (lanes 16 apart)
          float m = acc[tb][0][0];
#pragma unroll
          for (int vb = 0; vb < NB; ++vb)
#pragma unroll
            for (int i = (vb == 0 ? 1 : 0); i < 4; ++i) m = fmaxf(m, acc[tb][vb][i]);
          m = max_xor32(max_xor16(m));
          const float ml = m * kLog2e;
          const int row = 16 * u + x;
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int vb = 0; vb < NB; ++vb) {
            uint32_t pk0, pk1;
            if constexpr (teacher) {
              float wv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) wv[i] = __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][i], kLog2e, -ml));
              s0 += wv[0] + wv[2];
              s1 += wv[1] + wv[3];
              pk0 = pack_f16x2(wv[0], wv[1]);
              pk1 = pack_f16x2(wv[2], wv[3]);
            } else {
#pragma unroll
              for (int i = 0; i < 4; i += 2) {
                s0 += __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][i], kLog2e, -ml));
                s1 += __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][i + 1], kLog2e, -ml));
              }
              pk0 = pack_f16x2(acc[tb][vb][0] - m, acc[tb][vb][1] - m);
              pk1 = pack_f16x2(acc[tb][vb][2] - m, acc[tb][vb][3] - m);
            }
            // The 16-bit copies leave through LDS: a lane holds 8-byte pieces
            // of one token row, but the wavefront's 128 entries of a row are
            // 256 contiguous bytes.  Row r, 16-byte chunk c sits at slot
            // 16 r + (c ^ (r mod 16)), so the 8-byte writes of a half
            // wavefront and the 16-byte reads of 16 lanes each cover all 64
            // banks.  Entries 16 vb + 4 g .. + 3: chunk 2 vb + g / 2, half g % 2.
            const int c = 2 * vb + (g >> 1);
            *reinterpret_cast<u32x2*>(ob + (16 * row + (c ^ x)) * 16 + 8 * (g & 1)) = u32x2{pk0, pk1};
          }
          const float s = sum_xor32(sum_xor16(s0 + s1));
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), st_m, st_off, 64 * tb, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), st_s, st_off, 64 * tb, 0);
        }
        wave_lds_sync();
        {
          // chunk lane % 16 of rows lane / 16 + 4 j, whole row segments, not
          // read again before the gradient pass: nontemporal buffer stores
          // from a resource over the pair's 32 rows that ends at token n
          // (rows beyond it are dropped; below 2^31 bytes since V < 2^24)
          // and a lane offset of 2^31 for entries beyond V, so no store sits
          // under a condition and no 64-bit address is formed per lane
          const int ch = lane & 15;
          const int64_t r0 = t0e + 32 * tp;
          const int64_t rows = min(max(n - r0, int64_t{0}), int64_t{32});
          const buf_rsrc orr = make_rsrc(reinterpret_cast<const char*>(O) + (r0 * vocab + vwe) * 2,
                                         rows * vocab * 2 - static_cast<int64_t>(vwe) * 2);
          const uint32_t loff = vwe + 8 * ch < vocab
                                    ? (static_cast<uint32_t>(lane >> 4) * static_cast<uint32_t>(vocab) +
                                       8u * static_cast<uint32_t>(ch)) * 2u
                                    : 0x80000000u;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int row = 4 * j + (lane >> 4);
            const u32x4 v = *reinterpret_cast<const u32x4*>(ob + (16 * row + (ch ^ (row & 15))) * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, orr, loff, j * 8 * vocab, kBufNontemporal);
          }
        }
        wave_lds_sync();
      }
        // The label's logit, from the one lane that holds it: entry
        // 16 vb + 4 g + i of this wavefront.  The 16 tokens of a block rarely
        // have a label among the wavefront's 128 entries, so the selection
        // runs only in a wavefront where one does.  It follows the pair's
        // statistics (a branch between the two token blocks would keep the
        // compiler from interleaving their arithmetic), and the pair's
        // accumulators are dead after it.
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          const int y = ylab[tb];
          const int rel = y - (vwe + 4 * g);
          const bool hit = rel >= 0 && rel < 128 && (rel & 12) == 0 && y < vocab;
          if (__any(hit)) {
            const int vsel = rel >> 4, isel = rel & 3;
            float yv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              yv[i] = acc[tb][0][i];
#pragma unroll
              for (int vb = 1; vb < NB; ++vb) yv[i] = vsel == vb ? acc[tb][vb][i] : yv[i];
            }
            float lv = yv[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) lv = isel == i ? yv[i] : lv;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lab_out, hit ? toff : 0x80000000u,
                                                  64 * tb, 0);
          }
        }
    };
    if (MODE == kModeLossF16 && ei == 0)
      epilogue(std::true_type{});
    else
      epilogue(std::false_type{});
  }
}

// ------------------------------------------------- loss GEMM, narrow exits
// Two workgroups per CU, 128 tokens x 256 vocabulary entries each, on the main
// loop of packed16_core.h (128 x 64 per wavefront, 128 accumulators): the
// statistics tiles are the workgroup's 256 entries.  Its main loop is slower
// than the one-wavefront-per-SIMD kernel's, but each workgroup's epilogue
// runs beside the other workgroup's matrix instructions, which pays off when
// the exits are narrow and the epilogue (the same per logit at any width) is
// a large share of the work.
template <int MODE>
__global__ __launch_bounds__(kPkThreads, 2) void heads_loss_kernel_2wg(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    const int32_t* __restrict__ labels, float* __restrict__ stats, float* __restrict__ lab,
    int n_tt, int n_vt) {
  // The exit table is the first kernel argument; indexing it through the
  // kernarg segment pointer keeps per-exit lookups scalar.
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ u32x4 hs[2][16 * kPkTok];
  __shared__ float xmax[4][kPkTok];
  __shared__ float xsum[4][kPkTok][2];

  const int tid = threadIdx.x, lane = tid & 63, x = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tt, vt;
  tile_coords(blockIdx.x, n_tt, n_vt, kPkGroup, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kPkTok;
  const int vw = vt * kPkVoc + wave * 64;   // this wavefront's first vocabulary entry
  const int vlane = vw + 4 * g;             // first of this lane's 4 entries in block 0
  const int64_t tx = t0 + x;                // token of this lane in token block 0

  int ylab[kNTB];
#pragma unroll
  for (int tb = 0; tb < kNTB; ++tb)
    ylab[tb] = tx + 16 * tb < n ? labels[tx + 16 * tb] : -1;
  const PackedLanes pl = packed_lanes(tid);
  uint32_t hoff[4];   // byte offsets of this thread's h chunks from row t0 (rows beyond n clamped)
  // packed row blocks of the wavefront's 4 vocabulary blocks, clamped: rows beyond V are never stored
  int rbk[kNVB];
#pragma unroll
  for (int vb = 0; vb < kNVB; ++vb) rbk[vb] = min((vw >> 4) + vb, vocab / 16 - 1);

  f32x4 acc[kNTB][kNVB];
  for (int ei = 0; ei < n_exits; ++ei) {
    const int e = ei == 0 ? n_exits - 1 : ei - 1;
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
    const char* Wb[kNVB];
#pragma unroll
    for (int vb = 0; vb < kNVB; ++vb) Wb[vb] = P + static_cast<int64_t>(rbk[vb]) * D * 32;
    BRowsPlain<4> hsrc;
    hsrc.Bb = Hb;
#pragma unroll
    for (int j = 0; j < 4; ++j) hsrc.boff[j] = hoff[j];
    packed16_tile_gemm(acc, hs, Wb, hsrc, pl.hslot, D / kPkBK);

    // vocabulary entries beyond V (last tile only) vanish under exp and never
    // win a max; V is a multiple of 32, so a 16-block is wholly in or beyond V
    if (vt * kPkVoc + kPkVoc > vocab) {
#pragma unroll
      for (int vb = 0; vb < kNVB; ++vb)
        if (vw + 16 * vb >= vocab)
#pragma unroll
          for (int tb = 0; tb < kNTB; ++tb) acc[tb][vb] = f32x4{kMasked, kMasked, kMasked, kMasked};
    }

    const int64_t plane = static_cast<int64_t>(n_vt) * n;
    // (1) row maximum over the tile's 256 entries: a lane's 16, the four
    // lane groups of its token (lanes 16 apart), then the 4 wavefronts
#pragma unroll
    for (int tb = 0; tb < kNTB; ++tb) {
      float m = acc[tb][0][0];
#pragma unroll
      for (int vb = 0; vb < kNVB; ++vb)
#pragma unroll
        for (int i = (vb == 0 ? 1 : 0); i < 4; ++i) m = fmaxf(m, acc[tb][vb][i]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (g == 0) xmax[wave][16 * tb + x] = m;
    }
    __syncthreads();
    float M[kNTB];
#pragma unroll
    for (int tb = 0; tb < kNTB; ++tb) {
      const int j = 16 * tb + x;
      M[tb] = fmaxf(fmaxf(xmax[0][j], xmax[1][j]), fmaxf(xmax[2][j], xmax[3][j]));
    }
    // (2) sums, teacher weights / shifted logits, label logit
    bf16_t* __restrict__ O = static_cast<bf16_t*>(ex.out[e]);
    // The 16-bit copies leave through LDS, 32 tokens at a time: a lane holds
    // four 8-byte pieces of one token row, but the wavefront's 64 entries of
    // a row are one aligned 128-byte line, so after a wave-local transpose
    // eight lanes store a whole line.  The wavefront uses its own 4 KB of the
    // h stage, which no wavefront reads again before the barrier that ends
    // this exit's epilogue.  Row r, 16-byte chunk c sits at slot
    // 8 r + (c ^ ((r / 2) mod 8)): the 8-byte writes of a half wavefront and
    // the 16-byte reads of 16 lanes each cover all 64 banks.
    char* const stage = reinterpret_cast<char*>(&hs[0][0]) + wave * 4096;
#pragma unroll
    for (int tp = 0; tp < kNTB / 2; ++tp) {
      float s[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tb = 2 * tp + u;
        const float ml = M[tb] * kLog2e;
        const int row = 16 * u + x;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int vb = 0; vb < kNVB; ++vb) {
          uint32_t pk0, pk1;
          if (teacher) {
            float wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][i], kLog2e, -ml));
            s0 += wv[0] + wv[2];
            s1 += wv[1] + wv[3];
            pk0 = pack_f16x2(wv[0], wv[1]);
            pk1 = pack_f16x2(wv[2], wv[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              s0 += __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][i], kLog2e, -ml));
              s1 += __builtin_amdgcn_exp2f(fmaf(acc[tb][vb][i + 1], kLog2e, -ml));
            }
            pk0 = pack_f16x2(acc[tb][vb][0] - M[tb], acc[tb][vb][1] - M[tb]);
            pk1 = pack_f16x2(acc[tb][vb][2] - M[tb], acc[tb][vb][3] - M[tb]);
          }
          // entries 16 vb + 4 g .. + 3 of the row: chunk 2 vb + g / 2, half g % 2
          const int c = 2 * vb + (g >> 1);
          *reinterpret_cast<u32x2*>(stage + (8 * row + (c ^ ((row >> 1) & 7))) * 16 + 8 * (g & 1)) =
              u32x2{pk0, pk1};
        }
        s[u] = s0 + s1;
      }
      wave_lds_sync();
      {
        // whole lines, not read again before the gradient pass: nontemporal
        // buffer stores from a resource over the pair's 32 rows that ends at
        // token n (rows beyond it are dropped; below 2^31 bytes since
        // V < 2^24) and a lane offset of 2^31 for entries beyond V, so no
        // store sits under a condition
        const int ch = lane & 7;
        const int64_t r0 = t0 + 32 * tp;
        const int64_t rows = min(max(n - r0, int64_t{0}), int64_t{32});
        const buf_rsrc orr = make_rsrc(reinterpret_cast<const char*>(O) + (r0 * vocab + vw) * 2,
                                       rows * vocab * 2 - static_cast<int64_t>(vw) * 2);
        const uint32_t loff = vw + 8 * ch < vocab
                                  ? (static_cast<uint32_t>(lane >> 3) * static_cast<uint32_t>(vocab) +
                                     8u * static_cast<uint32_t>(ch)) * 2u
                                  : 0x80000000u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 8 * j + (lane >> 3);
          const u32x4 v =
              *reinterpret_cast<const u32x4*>(stage + (8 * row + (ch ^ ((row >> 1) & 7))) * 16);
          __builtin_amdgcn_raw_buffer_store_b128(v, orr, loff, j * 16 * vocab, kBufNontemporal);
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float t = s[u];
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        if (g == 0) xsum[wave][32 * tp + 16 * u + x][0] = t;
      }
    }
    // the label's logit, from the one lane that holds it (entry
    // 16 vb + 4 g + i of the wavefront), in a wavefront where one does
#pragma unroll
    for (int tb = 0; tb < kNTB; ++tb) {
      const int rel = ylab[tb] - vlane;
      const bool hit = rel >= 0 && rel < 64 && (rel & 12) == 0 && ylab[tb] < vocab;
      if (__any(hit)) {
        const int vsel = rel >> 4, isel = rel & 3;
        float yv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          yv[i] = acc[tb][0][i];
#pragma unroll
          for (int vb = 1; vb < kNVB; ++vb) yv[i] = vsel == vb ? acc[tb][vb][i] : yv[i];
        }
        float lv = yv[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) lv = isel == i ? yv[i] : lv;
        if (hit) lab[static_cast<int64_t>(e) * n + tx + 16 * tb] = lv;
      }
    }
    __syncthreads();
    // (3) thread j < 128 writes the statistics of token j
    if (tid < kPkTok && t0 + tid < n) {
      const int j = tid;
      float* st = stats + (static_cast<int64_t>(e) * 3 * n_vt + vt) * n + t0 + j;
      st[0] = fmaxf(fmaxf(xmax[0][j], xmax[1][j]), fmaxf(xmax[2][j], xmax[3][j]));
      st[plane] = (xsum[0][j][0] + xsum[1][j][0]) + (xsum[2][j][0] + xsum[3][j][0]);
    }
    // xmax / xsum are next written after this exit's main loop, behind its
    // barriers, which also end every read of them above
  }
}

// ------------------------------------------- argmax GEMM, one wavefront per SIMD
// Greedy verify on the main loop of wave128_core.h: one exit per workgroup
// (the widest exit's tiles first), 128 tokens x 512 entries; per token and
// wavefront the maximum logit of its 128 entries and the lowest index that
// holds it (one tile of the argmax merge per wavefront); optional fp32 logits.
__global__ __launch_bounds__(kW128Threads, 1) void heads_argmax_kernel_w128(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    float* __restrict__ best, int n_tt, int n_vt_wg, int n_st) {
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ u32x4 stage[kW128Stages * kW128Slots];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = blockIdx.x / (n_tt * n_vt_wg);
  const int e = n_exits - 1 - k;
  int tt, vt;
  tile_coords(blockIdx.x - k * (n_tt * n_vt_wg), n_tt, n_vt_wg, kPkGroup, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kW128Tok;
  const int vw = vt * kW128Voc + wave * 128;   // this wavefront's first vocabulary entry
  const int D = ex.d[e];
  W128Operands op;
  w128_lanes(tid, D, op);
  op.h = make_rsrc(static_cast<const char*>(ex.h[e]) + t0 * D * 2, (n - t0) * D * 2);
  op.w = make_rsrc(static_cast<const char*>(ex.w[e]) + static_cast<int64_t>(vw >> 4) * D * 32,
                   static_cast<int64_t>(vocab / 16 - (vw >> 4)) * D * 32);
  constexpr int NB = 8;
  f32x4 acc[NB][NB];
  w128_tile_gemm(acc, stage, op, D / 64);
  // opaque copies: the epilogue's lane values are computed here, not kept
  // live (and spilled) across the main loop
  int vwe = vw;
  int64_t t0e = t0;
  int lane = tid & 63;
  asm volatile("" : "+s"(vwe), "+s"(t0e), "+v"(lane));
  const int x = lane & 15, g = lane >> 4;
  // entries beyond V never win a max; V is a multiple of 32, so a 16-block is
  // wholly in or beyond V
  if (vwe + 128 > vocab) {
#pragma unroll
    for (int vb = 0; vb < NB; ++vb)
      if (vw + 16 * vb >= vocab)
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) acc[tb][vb] = f32x4{kMasked, kMasked, kMasked, kMasked};
  }
  const int vlane = vwe + 4 * g;   // first of this lane's 4 entries in block 0
  const int64_t plane = static_cast<int64_t>(n_st) * n;
  float* __restrict__ O = static_cast<float*>(ex.out[e]);
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int vb = 0; vb < NB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (acc[tb][vb][i] > bv) {   // ascending vocabulary: strict > keeps the lowest index
          bv = acc[tb][vb][i];
          bi = vlane + 16 * vb + i;
        }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    const int64_t tok = t0e + x + 16 * tb;
    if (O != nullptr && tok < n) {
#pragma unroll
      for (int vb = 0; vb < NB; ++vb) {
        const int vbase = vlane + 16 * vb;
        if (vbase >= vocab) continue;
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = __float_as_uint(acc[tb][vb][i]);
        *reinterpret_cast<u32x4*>(O + tok * vocab + vbase) = pk;
      }
    }
    // (a wavefront wholly beyond V, in the last tile only, writes nothing)
    if (g == 0 && tok < n && vwe < vocab) {
      float* b = best + (static_cast<int64_t>(e) * 2 * n_st + (vwe >> 7)) * n + tok;
      b[0] = bv;
      b[plane] = __int_as_float(bi);
    }
  }
}

// ---------------------------------------------------------------- argmax GEMM
// Greedy verify: per (token, tile) the maximum logit and its lowest index, on
// the main loop of packed16_core.h (128 tokens x 256 entries per workgroup,
// two workgroups per CU).  One exit per workgroup, the widest exit's tiles
// first, so that at small token counts the narrow exits' short workgroups fill
// the last round; optional fp32 logits.
__global__ __launch_bounds__(kPkThreads, 2) void heads_argmax_kernel(
    ExitSet /*read through the kernarg pointer*/, int n_exits, int64_t n, int vocab,
    float* __restrict__ best, int n_tt, int n_vt) {
  const ExitSet& ex = *(const ExitSet*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ u32x4 hs[2][16 * kPkTok];
  __shared__ float xbest[4][kPkTok][2];

  const int tid = threadIdx.x, lane = tid & 63, x = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = blockIdx.x / (n_tt * n_vt);
  const int e = n_exits - 1 - k;
  int tt, vt;
  tile_coords(blockIdx.x - k * (n_tt * n_vt), n_tt, n_vt, kPkGroup, tt, vt);
  const int64_t t0 = static_cast<int64_t>(tt) * kPkTok;
  const int vw = vt * kPkVoc + wave * 64;   // this wavefront's first vocabulary entry
  const int vlane = vw + 4 * g;             // first of this lane's 4 entries in block 0
  const int64_t tx = t0 + x;                // token of this lane in token block 0

  const PackedLanes pl = packed_lanes(tid);
  const int D = ex.d[e];
  // wave-uniform bases; per-lane 32-bit byte offsets of this thread's h chunks
  // from row t0 (rows beyond n clamped) and of the wavefront's 4 packed row
  // blocks (clamped: rows beyond V are never stored)
  BRowsPlain<4> hsrc;
  hsrc.Bb = static_cast<const char*>(ex.h[e]) + t0 * D * 2;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t row = min(t0 + pl.brow + 32 * j, n - 1) - t0;
    hsrc.boff[j] = static_cast<uint32_t>((row * D + pl.bchunk * 8) * 2);
  }
  const char* Wb[kNVB];
#pragma unroll
  for (int vb = 0; vb < kNVB; ++vb)
    Wb[vb] = static_cast<const char*>(ex.w[e]) +
             static_cast<int64_t>(min((vw >> 4) + vb, vocab / 16 - 1)) * D * 32;
  f32x4 acc[kNTB][kNVB];
  packed16_tile_gemm(acc, hs, Wb, hsrc, pl.hslot, D / kPkBK);
  // vocabulary entries beyond V (last tile only) never win a max
  if (vt * kPkVoc + kPkVoc > vocab) {
#pragma unroll
    for (int vb = 0; vb < kNVB; ++vb)
      if (vw + 16 * vb >= vocab)
#pragma unroll
        for (int tb = 0; tb < kNTB; ++tb) acc[tb][vb] = f32x4{kMasked, kMasked, kMasked, kMasked};
  }
  float* __restrict__ O = static_cast<float*>(ex.out[e]);
#pragma unroll
  for (int tb = 0; tb < kNTB; ++tb) {
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int vb = 0; vb < kNVB; ++vb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (acc[tb][vb][i] > bv) {   // ascending vocabulary: strict > keeps the lowest index
          bv = acc[tb][vb][i];
          bi = vlane + 16 * vb + i;
        }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    const int64_t tok = tx + 16 * tb;
    if (O != nullptr && tok < n) {
#pragma unroll
      for (int vb = 0; vb < kNVB; ++vb) {
        const int vbase = vlane + 16 * vb;
        if (vbase >= vocab) continue;
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = __float_as_uint(acc[tb][vb][i]);
        *reinterpret_cast<u32x4*>(O + tok * vocab + vbase) = pk;
      }
    }
    if (g == 0) {
      xbest[wave][16 * tb + x][0] = bv;
      xbest[wave][16 * tb + x][1] = __int_as_float(bi);
    }
  }
  __syncthreads();
  if (tid < kPkTok && t0 + tid < n) {
    const int j = tid;
    float bv = xbest[0][j][0];
    int bi = __float_as_int(xbest[0][j][1]);
#pragma unroll
    for (int w = 1; w < 4; ++w)   // later wavefronts hold higher indices: ties keep the first
      if (xbest[w][j][0] > bv) {
        bv = xbest[w][j][0];
        bi = __float_as_int(xbest[w][j][1]);
      }
    const int64_t plane = static_cast<int64_t>(n_vt) * n;
    float* b = best + (static_cast<int64_t>(e) * 2 * n_vt + vt) * n + t0 + j;
    b[0] = bv;
    b[plane] = __int_as_float(bi);
  }
}

constexpr int64_t kCUs = 256;   // compute units of the MI355X

// Exits whose mean width is below this use the two-workgroups-per-CU kernel.
// Measured, one-wavefront-per-SIMD kernel against it (TF/s, V = 32,768):
// widths 512 / 768 / 1024 at 16,384 tokens 936 / 926; 512 / 1024 / 1536 /
// 2048 at 32,768 tokens 1123 / 1095; 1024 / 1536 / 2048 1149 / 1113;
// 1024 / 2304 / 4352 1254 / 1202.  Narrower exits are not measured.
constexpr int kWideMeanD = 512;

template <int MODE>
hipError_t launch_loss(int n_exits, int64_t n, int vocab, const ExitSet& ex, const int32_t* labels,
                       float* stats, float* lab, TileInfo* info, hipStream_t s) {
  info->teacher_w16 = MODE == kModeLossF16;
  int64_t dsum = 0;
  for (int e = 0; e < n_exits; ++e) dsum += ex.d[e];
  if (dsum < static_cast<int64_t>(kWideMeanD) * n_exits) {
    info->vtile = kPkVoc;
    if (n == 0) return hipSuccess;
    const int n_tt = static_cast<int>((n + kPkTok - 1) / kPkTok);
    const int n_vt = (vocab + kPkVoc - 1) / kPkVoc;
    hipLaunchKernelGGL((heads_loss_kernel_2wg<MODE>), dim3(n_tt * n_vt), dim3(kPkThreads), 0, s,
                       ex, n_exits, n, vocab, labels, stats, lab, n_tt, n_vt);
    return hipGetLastError();
  }
  info->vtile = kW128StatTile;
  if (n == 0) return hipSuccess;
  const int n_tt = static_cast<int>((n + kW128Tok - 1) / kW128Tok);
  const int n_vt = (vocab + kW128Voc - 1) / kW128Voc;
  const int n_st = (vocab + kW128StatTile - 1) / kW128StatTile;
  hipLaunchKernelGGL((heads_loss_kernel<MODE>), dim3(n_tt * n_vt), dim3(kW128Threads), 0, s, ex,
                     n_exits, n, vocab, labels, stats, lab, n_tt, n_vt, n_st);
  return hipGetLastError();
}

}  // namespace

// d below 2^24 keeps the 32-bit byte offsets of a 128-token slice of h in range.
bool packed_shape_ok(int vocab, int d) {
  return vocab >= 32 && vocab % 32 == 0 && vocab < (1 << 24) && d >= 64 && d % 64 == 0 &&
         d < (1 << 24);
}

hipError_t launch_pack_weights(int vocab, int d, const void* w, void* packed, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(vocab / 16) * ((d / 32 + 3) / 4);
  const int grid = static_cast<int>(units < 65536 ? units : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, static_cast<const bf16_t*>(w),
                     static_cast<bf16_t*>(packed), vocab, d);
  return hipGetLastError();
}

hipError_t launch_heads_loss_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                                    const int32_t* labels, float* stats, float* lab, bool plain,
                                    TileInfo* info, hipStream_t s) {
  if (plain) return launch_loss<kModeLossPlain>(n_exits, n, vocab, ex, labels, stats, lab, info, s);
  return launch_loss<kModeLossF16>(n_exits, n, vocab, ex, labels, stats, lab, info, s);
}

hipError_t launch_heads_argmax_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                                      float* best, TileInfo* info, hipStream_t s) {
  info->teacher_w16 = false;
  // The one-wavefront-per-SIMD kernel when its grid gives every CU at least
  // two workgroups (its tiles are twice as wide); below that, at small token
  // counts, the two-workgroups-per-CU kernel keeps more CUs busy.
  {
    const int64_t n_tt = (n + kW128Tok - 1) / kW128Tok;
    const int n_vt = (vocab + kW128Voc - 1) / kW128Voc;
    if (n_tt * n_vt * n_exits >= 2 * kCUs) {
      info->vtile = kW128StatTile;
      const int n_st = (vocab + kW128StatTile - 1) / kW128StatTile;
      hipLaunchKernelGGL(heads_argmax_kernel_w128, dim3(static_cast<unsigned>(n_tt * n_vt * n_exits)),
                         dim3(kW128Threads), 0, s, ex, n_exits, n, vocab, best,
                         static_cast<int>(n_tt), n_vt, n_st);
      return hipGetLastError();
    }
  }
  info->vtile = kPkVoc;
  if (n == 0) return hipSuccess;
  const int n_tt = static_cast<int>((n + kPkTok - 1) / kPkTok);
  const int n_vt = (vocab + kPkVoc - 1) / kPkVoc;
  hipLaunchKernelGGL(heads_argmax_kernel, dim3(n_tt * n_vt * n_exits), dim3(kPkThreads), 0, s, ex,
                     n_exits, n, vocab, best, n_tt, n_vt);
  return hipGetLastError();
}

}  // namespace nel
