// Launchers of the gfx950 kernels (host side), shared by the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nel {

// Junction modes (values of nel_junction_mode).
constexpr int kJunctionRescale = 0, kJunctionNoRescale = 1, kJunctionZeroFill = 2;

constexpr int kMaxExits = 8;

// Distillation divergences (values of nel_divergence).
constexpr int kDivForward = 0, kDivReverseKL = 1, kDivJS = 2, kDivTV = 3;

// Per-exit loss weights, passed to kernels by value.
struct ExitW {
  float w[kMaxExits];
};
// Smallest token and vocabulary extent of a head-GEMM workgroup tile.  Loss
// statistics are kept per (exit, vocabulary tile, token); the GEMM reports
// the vocabulary tile it used and the workspace is sized for the smallest.
constexpr int kTokTile = 128;
constexpr int kVocTile = 128;

struct ExitSet {
  const void* h[kMaxExits];   // [n, d[e]]
  const void* w[kMaxExits];   // [V, d[e]]
  void* out[kMaxExits];       // loss: dlogits[e] [n, V] (dt) or null; argmax: fp32 logits or null
  int d[kMaxExits];
};

// What the head GEMM that ran tells the passes after it: the vocabulary
// width of its statistics tiles, and whether the teacher's gradient buffer
// holds its weights exp(l_M - m) (packed GEMM, cross-entropy to the teacher)
// rather than its tile-shifted logits l - m.  Either way the scratch is in
// the codec Scratch<T> of the element type (fp16 for bf16 inputs).
struct TileInfo {
  int vtile = kVocTile;
  bool teacher_w16 = false;
};

inline int64_t n_vocab_tiles(int vocab) { return (vocab + kVocTile - 1) / kVocTile; }

// Tokens per workgroup of the loss merge; each workgroup leaves fp64 partial
// sums of the 3M + 1 reported means.
constexpr int kMergeTok = 64;
inline int64_t n_merge_blocks(int64_t n) { return (n + kMergeTok - 1) / kMergeTok; }

// Workspace layout of the loss op (byte offsets from the base); dv and kv
// hold a divergence's value and gradient row constant per (exit, token).
struct LossWs {
  size_t flags, stats, lab, lse, tokloss, partials, dv, kv, total;
};
inline LossWs loss_ws_layout(int n_exits, int64_t n, int vocab) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  LossWs L;
  const size_t nvt = static_cast<size_t>(n_vocab_tiles(vocab));
  L.flags = 0;
  L.stats = 256;
  L.lab = L.stats + up(sizeof(float) * n_exits * 3 * nvt * n);
  L.lse = L.lab + up(sizeof(float) * n_exits * n);
  L.tokloss = L.lse + up(sizeof(float) * n_exits * n);
  L.partials = L.tokloss + up(sizeof(float) * n_exits * 3 * n);
  L.dv = L.partials + up(sizeof(double) * (3 * n_exits + 1) * n_merge_blocks(n));
  L.kv = L.dv + up(sizeof(float) * n_exits * n);
  L.total = L.kv + up(sizeof(float) * n_exits * n);
  return L;
}
struct HeadsWs {
  size_t flags, best, total;
};
inline HeadsWs heads_ws_layout(int n_exits, int64_t n, int vocab) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  HeadsWs L;
  const size_t nvt = static_cast<size_t>(n_vocab_tiles(vocab));
  L.flags = 0;
  L.best = 256;
  L.total = L.best + up(sizeof(float) * 2 * n_exits * nvt * n);
  return L;
}

// Sampled speculative verification (fp32 logits of the two exits).
size_t speculative_ws_bytes(int batch, int draft_len);
hipError_t launch_speculative_verify(int batch, int positions, int draft_len, int vocab,
                                     const float* draft, const float* verify,
                                     const int32_t* tokens, const float* u_accept,
                                     const float* u_next, float temperature, float top_p,
                                     float* beta, int32_t* accepted, int32_t* next_token,
                                     int32_t* flags, void* workspace, hipStream_t s);

// Workspace of the junction backward (byte offsets): c_t, rank in block and
// the id-sorted token list per token; per-block counts per id; per id: count,
// list start, first partial slot; the totals of segments and partial slots;
// per-workgroup totals of the id scan; per segment {id, list begin, list end,
// partial slot}; the partial slot -> id table; partial sums.
struct JunctionBwdWs {
  size_t ct, rank, list, hist, cnt, rowoff, poff, counts, wgtot, seginfo, prow, pcs, partial, total;
};
JunctionBwdWs junction_bwd_ws_layout(int64_t n, int d_in, int d_out, int vocab);
// Token indices, list offsets and segment numbers are int32.
constexpr int64_t kJunctionBwdMaxTokens = int64_t{1} << 30;
template <typename T>
hipError_t launch_junction_backward(int64_t n, int d_in, int d_out, int vocab, const void* h,
                                    const int32_t* ids, const void* emb, const void* dout,
                                    int stop_grad, int mode, void* dh, float* demb,
                                    void* workspace, int32_t* flags, hipStream_t s);

// Workspace of the head backward (byte offsets): W^T and h^T in the tiled
// layout; K of the token dimension padded to n_pad.
struct HeadBwdWs {
  int64_t n_pad;
  size_t wt, ht, total;
};
HeadBwdWs head_bwd_ws_layout(int64_t n, int vocab, int d);
// A group of backward products out[b][a] = sum_k A[a][k] B[b][k] (one per
// exit) for one launch; first[e] is the first workgroup id of product e.
struct BwdGroup {
  const uint16_t* A[kMaxExits];
  const uint16_t* B[kMaxExits];
  void* out[kMaxExits];
  int64_t b_rows[kMaxExits], ldb[kMaxExits], K[kMaxExits], ldo[kMaxExits];
  int64_t k_valid[kMaxExits];   // K-major B: K rows that exist (the rest read as 0)
  int a_rows[kMaxExits], n_bt[kMaxExits], n_at[kMaxExits];
  int first[kMaxExits + 1];
  int count;
  // Fused launches (B = G formed from the packed loss GEMM's fp16 scratch):
  // B[e] is exit e's scratch, tw the teacher's, tab[e] exit e's row
  // constants [vocabulary tile][n_tok] (launch_grad_consts), which scale by
  // |grad_scale * lambda_e|; neg[e] is 0x80008000 where that product is
  // negative (grad_chunk flips the bf16 gradients, as the stored pass does).
  const uint16_t* tw;
  const void* tab[kMaxExits];
  uint32_t neg[kMaxExits];
  int64_t n_tok;
  int vshift;   // log2 of the statistics tile width
};
bool bwd_group_add(BwdGroup& g, const void* A, int a_rows, const void* B, int64_t b_rows,
                   int64_t ldb, int64_t K, void* out, int64_t ldo, int64_t k_valid = -1);
// dh: out[b][a] = sum_k A[a][k] B[b][k], A tiled for the 16x16x32 loop
// (launch_pack16_t), B row-major [b_rows x ldb] with K contiguous; bf16 out.
// dW: the same with B(b, k) the element k * ldb + b of a row-major [K x ldb]
// matrix (b_rows columns of it; K rows k_valid.. read as 0); fp32 out.
// FUSED: B is formed from the scratch (the fused fields of the group).
template <bool FUSED>
hipError_t launch_dh_group(const BwdGroup& g, hipStream_t s);
template <bool FUSED>
hipError_t launch_dw_group(const BwdGroup& g, hipStream_t s);
// Tiled A operand of S^T for S [k_rows, R] row-major, K zero-padded to k_pad:
// for the 32x32x16 loop (pack_t) or the 16x16x32 loop (pack16_t).
hipError_t launch_pack_t(const void* S, int64_t k_rows, int R, int64_t k_pad, void* P,
                         hipStream_t s);
hipError_t launch_pack16_t(const void* S, int64_t k_rows, int R, int64_t k_pad, void* P,
                           hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t s);
template <typename T>
hipError_t launch_junction(int64_t n, int d_in, int d_out, int vocab, const void* h,
                           const int32_t* ids, const void* emb, void* out, int32_t* flags,
                           int mode, hipStream_t s);

// Head GEMM + per-tile loss statistics (teacher = exit n_exits-1 first),
// row-major weights.
template <typename T>
hipError_t launch_heads_loss(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                             const int32_t* labels, float* stats, float* lab, TileInfo* info,
                             hipStream_t s);
// Head GEMM + per-tile (max, lowest index); optional fp32 logits in ex.out.
template <typename T>
hipError_t launch_heads_argmax(int n_exits, int64_t n, int vocab, const ExitSet& ex, float* best,
                               TileInfo* info, hipStream_t s);

// MFMA-tiled (packed) bf16 weights: shape rule, packing, and the two GEMMs.
// The loss GEMM needs every ex.out[e] (the teacher's holds its weights).
bool packed_shape_ok(int vocab, int d);
hipError_t launch_pack_weights(int vocab, int d, const void* w, void* packed, hipStream_t s);
// What the packed loss GEMM leaves for the passes after it: the teacher's
// weights and the smaller exits' l - m in fp16 (for finalize_rows), or with
// `plain` l - m in bf16 for every exit (for the other divergences).
hipError_t launch_heads_loss_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                                    const int32_t* labels, float* stats, float* lab, bool plain,
                                    TileInfo* info, hipStream_t s);
hipError_t launch_heads_argmax_packed(int n_exits, int64_t n, int vocab, const ExitSet& ex,
                                      float* best, TileInfo* info, hipStream_t s);

hipError_t launch_loss_merge(int n_exits, int64_t n, int vocab, int vtile, const int32_t* labels,
                             float alpha, const float* stats, const float* lab, float* lse,
                             float* tokloss, double* partials, int32_t* flags, const ExitW& lam,
                             bool skip_dist, hipStream_t s);
// After the fp16 scratch: every exit's gradient in place (unless !write_g,
// which leaves the scratch as it is), one token row per workgroup, and
// dv[e][t] = Dist_e from the teacher-weighted logit sums.
hipError_t launch_finalize_rows(int n_exits, int64_t n, int vocab, const TileInfo& info,
                                const int32_t* labels, float alpha, float grad_scale,
                                const float* stats, const float* lse, void* const* dlogits,
                                float* dv, const ExitW& lam, bool write_g, hipStream_t s);
// Row constants of the gradients formed from the fp16 scratch: 16 bytes per
// (exit, vocabulary tile, token) at out + 16 ((e n_vt + tile) n + t): c1 (-inf
// for the teacher), the teacher's scale, the label (grad_chunk.h).
hipError_t launch_grad_consts(int n_exits, int64_t n, int vocab, const TileInfo& info,
                              const int32_t* labels, float alpha, float grad_scale,
                              const ExitW& lam, const float* stats, const float* lse, void* out,
                              hipStream_t s);
// The losses and mean partials with Dist from dv (after launch_loss_merge with skip_dist).
hipError_t launch_loss_finish(int n_exits, int64_t n, float alpha, const float* dv,
                              float* tokloss, double* partials, const ExitW& lam, hipStream_t s);
// Divergence D (not the forward cross-entropy) per student and token, then
// the losses and mean partials with it (after launch_loss_merge with skip_dist).
template <typename T>
hipError_t launch_divergence(int n_exits, int64_t n, int vocab, const TileInfo& info, int div,
                             float alpha, const float* stats, const float* lse,
                             void* const* dlogits, float* dv, float* kv, float* tokloss,
                             double* partials, const ExitW& lam, hipStream_t s);
hipError_t launch_loss_means(int n_exits, int64_t n, const double* partials, float* means,
                             hipStream_t s);
template <typename T>
hipError_t launch_finalize(int n_exits, int64_t n, int vocab, const TileInfo& info,
                           const int32_t* labels, float alpha, float grad_scale,
                           const float* stats, const float* lse, void* const* dlogits, int div,
                           const float* kv, const ExitW& lam, hipStream_t s);
hipError_t launch_argmax_merge(int n_exits, int64_t n, int vocab, int vtile, const float* best,
                               int32_t* argmax, hipStream_t s);
hipError_t launch_accept(int batch, int positions, int draft_len, const int32_t* draft,
                         const int32_t* verify, int32_t* accepted, hipStream_t s);
hipError_t launch_clear_flags(int32_t* flags, hipStream_t s);

}  // namespace nel
