// C ABI (include/nel.h): argument validation, workspace carving and kernel
// sequencing.  Every entry point validates everything it can on the host
// before enqueuing any work, so an error return means nothing was launched.
#include <limits.h>
#include <math.h>
#include <atomic>
#include <mutex>
#include <vector>

#include "nel.h"
#include "common.h"
#include "internal.h"
#include "packed_core.h"

using namespace nel;

namespace {

// Tensors read or written in 16-byte chunks (h, w, emb, junction output,
// dlogits, fp32 logits, workspace) need 16-byte alignment; int32 arrays and
// per-element fp32 outputs need 4.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

// ---------------------------------------------------------------- timing hooks
struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};   // read without the lock on every launch
  struct Pending {
    int k;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  double total_ms[NEL_K_COUNT] = {};
  int64_t launches[NEL_K_COUNT] = {};
};
Timing& timing() {
  static Timing t;
  return t;
}

// Brackets one launch with events on its stream when timing is enabled.
// Every launch goes through here.  hipGetLastError reports the last error of
// any runtime call on this thread, including calls other libraries made and
// ignored; it is cleared first so that a launch reports only its own error.
template <typename F>
hipError_t timed(int k, hipStream_t s, F&& launch) {
  (void)hipGetLastError();
  Timing& T = timing();
  if (!T.on.load(std::memory_order_relaxed)) return launch();
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return hipErrorUnknown;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return hipErrorUnknown;
  }
  if (hipEventRecord(a, s) != hipSuccess) {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return hipErrorUnknown;
  }
  hipError_t err = launch();
  if (hipEventRecord(b, s) != hipSuccess && err == hipSuccess) err = hipErrorUnknown;
  std::lock_guard<std::mutex> g(T.mu);
  T.pending.push_back({k, a, b});
  return err;
}

// The HIP error behind this thread's most recent NEL_EHIP.
thread_local hipError_t g_last_hip = hipSuccess;

nel_status from_hip(hipError_t e) {
  if (e == hipSuccess) return NEL_OK;
  g_last_hip = e;
  return NEL_EHIP;
}

nel_status check_exits(int32_t n_exits, int64_t n, const int32_t* d, const void* const* h,
                       const void* const* w, bool strict) {
  if (n_exits < 1 || n_exits > NEL_MAX_EXITS) return NEL_EINVAL;
  if (!d || !h || !w) return NEL_EINVAL;
  for (int e = 0; e < n_exits; ++e) {
    if (d[e] < 1) return NEL_ESHAPE;
    if (strict && e > 0 && d[e] <= d[e - 1]) return NEL_ESHAPE;
    if (n > 0 && (!h[e] || !w[e])) return NEL_EINVAL;
    if (misaligned(h[e]) || misaligned(w[e])) return NEL_EALIGN;
  }
  return NEL_OK;
}

bool grid_fits(int64_t n, int32_t vocab) {
  const int64_t n_tt = (n + kTokTile - 1) / kTokTile;
  return n_tt * n_vocab_tiles(vocab) <= INT_MAX && n <= (int64_t{1} << 40);
}

}  // namespace

extern "C" {

const char* nel_last_hip_error(void) {
  return g_last_hip == hipSuccess ? "none" : hipGetErrorName(g_last_hip);
}

const char* nel_status_string(nel_status s) {
  switch (s) {
    case NEL_OK: return "ok";
    case NEL_EINVAL: return "invalid argument";
    case NEL_ESHAPE: return "invalid shape";
    case NEL_EDTYPE: return "invalid element type";
    case NEL_EALIGN: return "pointer misaligned";
    case NEL_EWORKSPACE: return "workspace missing or too small";
    case NEL_EHIP: return "HIP runtime error";
    case NEL_ETOOLARGE: return "request exceeds the fixed scratch of the allocation-free entry point";
  }
  return "unknown status";
}

size_t nel_workspace_size(int32_t op, int32_t n_exits, int64_t n_tokens, int32_t vocab) {
  if (n_exits < 1 || n_exits > NEL_MAX_EXITS || n_tokens < 0 || vocab < 1) return 0;
  if (op == NEL_OP_LOSS) return loss_ws_layout(n_exits, n_tokens, vocab).total;
  if (op == NEL_OP_HEADS) return heads_ws_layout(n_exits, n_tokens, vocab).total;
  return 0;
}

nel_status nel_junction(nel_dtype dt, int64_t n_tokens, int32_t d_in, int32_t d_out,
                        int32_t vocab, const void* h, const int32_t* ids, const void* emb,
                        void* out, int32_t mode, int32_t* flags, void* stream) {
  if (dt != NEL_F32 && dt != NEL_BF16) return NEL_EDTYPE;
  if (n_tokens < 0 || d_in < 0 || d_out <= d_in || vocab < 1) return NEL_ESHAPE;
  if (mode < NEL_JUNCTION_RESCALE || mode > NEL_JUNCTION_ZERO_FILL) return NEL_EINVAL;
  if (n_tokens > 0 && (!ids || !emb || !out || (d_in > 0 && !h))) return NEL_EINVAL;
  if (misaligned(h) || misaligned4(ids) || misaligned(emb) || misaligned(out) || misaligned4(flags))
    return NEL_EALIGN;
  if (n_tokens == 0) return NEL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(timed(NEL_K_JUNCTION, s, [&] {
    return dt == NEL_BF16
               ? launch_junction<bf16_t>(n_tokens, d_in, d_out, vocab, h, ids, emb, out, flags,
                                         mode, s)
               : launch_junction<float>(n_tokens, d_in, d_out, vocab, h, ids, emb, out, flags,
                                        mode, s);
  }));
}

nel_status nel_accept_prefix(int32_t batch, int32_t positions, int32_t draft_len,
                             const int32_t* draft_argmax, const int32_t* verify_argmax,
                             int32_t* accepted, void* stream) {
  if (batch < 0 || positions < 1 || draft_len < 0 || draft_len > positions) return NEL_ESHAPE;
  if (batch > 0 && (!draft_argmax || !verify_argmax || !accepted)) return NEL_EINVAL;
  if (misaligned4(draft_argmax) || misaligned4(verify_argmax) || misaligned4(accepted))
    return NEL_EALIGN;
  if (batch == 0) return NEL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(timed(NEL_K_ACCEPT, s, [&] {
    return launch_accept(batch, positions, draft_len, draft_argmax, verify_argmax, accepted, s);
  }));
}

}  // extern "C"

namespace {

// Host validation of an exit-heads call (everything but the workspace); on
// success *L is the workspace layout the call needs.
nel_status exit_heads_check(bool packed, nel_dtype dt, int32_t n_exits, int64_t n_tokens,
                            int32_t vocab, const int32_t* d, const void* const* h,
                            const void* const* w, float* const* logits, const int32_t* argmax,
                            HeadsWs* L) {
  if (dt != NEL_F32 && dt != NEL_BF16) return NEL_EDTYPE;
  if (packed && dt != NEL_BF16) return NEL_EDTYPE;
  if (n_tokens < 0 || vocab < 1) return NEL_ESHAPE;
  nel_status st = check_exits(n_exits, n_tokens, d, h, w, /*strict=*/false);
  if (st != NEL_OK) return st;
  if (packed)
    for (int e = 0; e < n_exits; ++e)
      if (!packed_shape_ok(vocab, d[e])) return NEL_ESHAPE;
  if (!grid_fits(n_tokens, vocab)) return NEL_ESHAPE;
  // the packed argmax grid has a workgroup per (token tile, 256-entry tile, exit)
  if (packed && (n_tokens + 127) / 128 * ((vocab + 255) / 256) * n_exits > INT_MAX)
    return NEL_ESHAPE;
  if (logits)
    for (int e = 0; e < n_exits; ++e) {
      if (n_tokens > 0 && !logits[e]) return NEL_EINVAL;
      if (misaligned(logits[e])) return NEL_EALIGN;
    }
  if (misaligned4(argmax)) return NEL_EALIGN;
  *L = heads_ws_layout(n_exits, n_tokens, vocab);
  return NEL_OK;
}

// The exit-heads kernels on a validated call, with `ws` (>= L.total bytes) as
// the per-tile partial results.  hooks = false bypasses the timing hooks
// (which create events).
nel_status exit_heads_run(bool packed, bool hooks, nel_dtype dt, int32_t n_exits,
                          int64_t n_tokens, int32_t vocab, const int32_t* d, const void* const* h,
                          const void* const* w, float* const* logits, int32_t* argmax, char* ws,
                          const HeadsWs& L, hipStream_t s) {
  if (n_tokens == 0 || (!logits && !argmax)) return NEL_OK;
  ExitSet ex{};
  for (int e = 0; e < n_exits; ++e) {
    ex.h[e] = h[e];
    ex.w[e] = w[e];
    ex.out[e] = logits ? logits[e] : nullptr;
    ex.d[e] = d[e];
  }
  float* best = reinterpret_cast<float*>(ws + L.best);
  TileInfo info;
  auto run = [&](int k, auto&& launch) -> hipError_t {
    if (hooks) return timed(k, s, launch);
    (void)hipGetLastError();
    return launch();
  };
  hipError_t err = run(NEL_K_HEADS_ARGMAX, [&] {
    if (packed) return launch_heads_argmax_packed(n_exits, n_tokens, vocab, ex, best, &info, s);
    return dt == NEL_BF16
               ? launch_heads_argmax<bf16_t>(n_exits, n_tokens, vocab, ex, best, &info, s)
               : launch_heads_argmax<float>(n_exits, n_tokens, vocab, ex, best, &info, s);
  });
  if (err != hipSuccess) return from_hip(err);
  if (argmax) {
    err = run(NEL_K_ARGMAX_MERGE, [&] {
      return launch_argmax_merge(n_exits, n_tokens, vocab, info.vtile, best, argmax, s);
    });
  }
  return from_hip(err);
}

nel_status exit_heads_impl(bool packed, nel_dtype dt, int32_t n_exits, int64_t n_tokens,
                           int32_t vocab, const int32_t* d, const void* const* h,
                           const void* const* w, float* const* logits, int32_t* argmax,
                           void* workspace, size_t ws_bytes, void* stream) {
  HeadsWs L;
  const nel_status st =
      exit_heads_check(packed, dt, n_exits, n_tokens, vocab, d, h, w, logits, argmax, &L);
  if (st != NEL_OK) return st;
  if (misaligned(workspace)) return NEL_EALIGN;
  if (!workspace || ws_bytes < L.total) return NEL_EWORKSPACE;
  return exit_heads_run(packed, true, dt, n_exits, n_tokens, vocab, d, h, w, logits, argmax,
                        static_cast<char*>(workspace), L, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------ no-allocation
// Scratch of nel_exit_heads_packed_noalloc: the per-tile partial results of
// the argmax GEMM, in a fixed array that every device holds from module load
// to process end.  Host code never uses `scratch` itself (in host code the
// name is a stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = NEL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kNoAllocMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// This device's address of `scratch` (looked up on the device's first call).
hipError_t noalloc_scratch(int device, void** ptr) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

nel_status loss_impl(bool packed, nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                     const int32_t* d, const void* const* h, const void* const* w,
                     const int32_t* labels, float alpha_d, float grad_scale,
                     const float* exit_weights, int32_t div, float* token_loss,
                     float* mean_loss, void* const* dlogits, void* workspace, size_t ws_bytes,
                     void* stream, bool write_g = true, TileInfo* info_out = nullptr) {
  if (dt != NEL_F32 && dt != NEL_BF16) return NEL_EDTYPE;
  if (packed && dt != NEL_BF16) return NEL_EDTYPE;
  if (n_tokens < 0 || vocab < 1) return NEL_ESHAPE;
  nel_status st = check_exits(n_exits, n_tokens, d, h, w, /*strict=*/true);
  if (st != NEL_OK) return st;
  if (packed) {
    for (int e = 0; e < n_exits; ++e)
      if (!packed_shape_ok(vocab, d[e])) return NEL_ESHAPE;
    if (!dlogits) return NEL_EINVAL;   // the teacher's buffer carries its weights
  }
  if (!(alpha_d >= 0.f && alpha_d <= 1.f) || !isfinite(grad_scale)) return NEL_EINVAL;
  if (div < NEL_DIV_FORWARD || div > NEL_DIV_TV) return NEL_EINVAL;
  if (div != NEL_DIV_FORWARD && !dlogits) return NEL_EINVAL;   // its pass reads the stored logits
  ExitW lam;
  for (int e = 0; e < kMaxExits; ++e) lam.w[e] = 1.f;
  if (exit_weights)
    for (int e = 0; e < n_exits; ++e) {
      if (!(exit_weights[e] >= 0.f) || !isfinite(exit_weights[e])) return NEL_EINVAL;
      lam.w[e] = exit_weights[e];
    }
  if (!grid_fits(n_tokens, vocab)) return NEL_ESHAPE;
  if (!mean_loss || (n_tokens > 0 && !labels)) return NEL_EINVAL;
  if (dlogits)
    for (int e = 0; e < n_exits; ++e) {
      if (n_tokens > 0 && !dlogits[e]) return NEL_EINVAL;
      if (misaligned(dlogits[e])) return NEL_EALIGN;
    }
  if (misaligned4(labels) || misaligned4(token_loss) || misaligned4(mean_loss) ||
      misaligned(workspace))
    return NEL_EALIGN;
  const LossWs L = loss_ws_layout(n_exits, n_tokens, vocab);
  if (!workspace || ws_bytes < L.total) return NEL_EWORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + L.flags);
  float* stats = reinterpret_cast<float*>(ws + L.stats);
  float* lab = reinterpret_cast<float*>(ws + L.lab);
  float* lse = reinterpret_cast<float*>(ws + L.lse);
  float* tl = token_loss ? token_loss : reinterpret_cast<float*>(ws + L.tokloss);
  double* partials = reinterpret_cast<double*>(ws + L.partials);
  ExitSet ex{};
  for (int e = 0; e < n_exits; ++e) {
    ex.h[e] = h[e];
    ex.w[e] = w[e];
    ex.out[e] = dlogits ? dlogits[e] : nullptr;
    ex.d[e] = d[e];
  }
  TileInfo info;
  const bool fwd = div == NEL_DIV_FORWARD;
  // packed heads with the method's divergence: fp16 scratch, and the
  // teacher-weighted sums formed by the row-wise gradient pass
  const bool rows = packed && fwd;
  hipError_t err = timed(NEL_K_HEADS_LOSS, s, [&] {
    if (packed)
      return launch_heads_loss_packed(n_exits, n_tokens, vocab, ex, labels, stats, lab, !fwd,
                                      &info, s);
    return dt == NEL_BF16 ? launch_heads_loss<bf16_t>(n_exits, n_tokens, vocab, ex, labels, stats,
                                                      lab, &info, s)
                          : launch_heads_loss<float>(n_exits, n_tokens, vocab, ex, labels, stats,
                                                     lab, &info, s);
  });
  if (err != hipSuccess) return from_hip(err);
  err = timed(NEL_K_MERGE, s, [&] {
    return launch_loss_merge(n_exits, n_tokens, vocab, info.vtile, labels, alpha_d, stats, lab, lse, tl,
                             partials, flags, lam, !fwd || rows, s);
  });
  if (err != hipSuccess) return from_hip(err);
  float* dv = reinterpret_cast<float*>(ws + L.dv);
  float* kv = reinterpret_cast<float*>(ws + L.kv);
  if (!fwd) {
    err = timed(NEL_K_DIVERGENCE, s, [&] {
      return dt == NEL_BF16
                 ? launch_divergence<bf16_t>(n_exits, n_tokens, vocab, info, div, alpha_d, stats,
                                             lse, dlogits, dv, kv, tl, partials, lam, s)
                 : launch_divergence<float>(n_exits, n_tokens, vocab, info, div, alpha_d, stats,
                                            lse, dlogits, dv, kv, tl, partials, lam, s);
    });
    if (err != hipSuccess) return from_hip(err);
  }
  if (rows && n_tokens > 0) {
    err = timed(NEL_K_FINALIZE, s, [&] {
      return launch_finalize_rows(n_exits, n_tokens, vocab, info, labels, alpha_d, grad_scale,
                                  stats, lse, dlogits, dv, lam, write_g, s);
    });
    if (err != hipSuccess) return from_hip(err);
  }
  err = timed(NEL_K_MEANS, s, [&] {
    if (rows) {
      const hipError_t e = launch_loss_finish(n_exits, n_tokens, alpha_d, dv, tl, partials, lam, s);
      if (e != hipSuccess) return e;
    }
    return launch_loss_means(n_exits, n_tokens, partials, mean_loss, s);
  });
  if (err != hipSuccess) return from_hip(err);
  if (info_out) *info_out = info;
  if (dlogits && n_tokens > 0 && !rows) {
    err = timed(NEL_K_FINALIZE, s, [&] {
      return dt == NEL_BF16 ? launch_finalize<bf16_t>(n_exits, n_tokens, vocab, info, labels,
                                                      alpha_d, grad_scale, stats, lse, dlogits,
                                                      div, kv, lam, s)
                            : launch_finalize<float>(n_exits, n_tokens, vocab, info, labels,
                                                     alpha_d, grad_scale, stats, lse, dlogits,
                                                     div, kv, lam, s);
    });
  }
  return from_hip(err);
}

}  // namespace

extern "C" {

nel_status nel_exit_heads(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                          const int32_t* d, const void* const* h, const void* const* w,
                          float* const* logits, int32_t* argmax, void* workspace,
                          size_t ws_bytes, void* stream) {
  return exit_heads_impl(false, dt, n_exits, n_tokens, vocab, d, h, w, logits, argmax, workspace,
                         ws_bytes, stream);
}

nel_status nel_exit_heads_packed_noalloc(nel_dtype dt, int32_t n_exits, int64_t n_tokens,
                                         int32_t vocab, const int32_t* d, const void* const* h,
                                         const void* const* w_packed, float* const* logits,
                                         int32_t* argmax, void* stream) {
  HeadsWs L;
  const nel_status st =
      exit_heads_check(true, dt, n_exits, n_tokens, vocab, d, h, w_packed, logits, argmax, &L);
  if (st != NEL_OK) return st;
  if (L.total > kNoAllocScratchBytes) return NEL_ETOOLARGE;
  if (n_tokens == 0 || (!logits && !argmax)) return NEL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e);
  if (dev < 0 || dev >= kNoAllocMaxDevices) return NEL_EINVAL;
  if (s) {   // the scratch address below is the current device's
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return from_hip(e);
    if (sdev != dev) return NEL_EINVAL;
  }
  void* ptr = nullptr;
  e = noalloc_scratch(dev, &ptr);
  if (e != hipSuccess) return from_hip(e);
  return exit_heads_run(true, false, dt, n_exits, n_tokens, vocab, d, h, w_packed, logits, argmax,
                        static_cast<char*>(ptr), L, s);
}

nel_status nel_exit_heads_packed(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                                 const int32_t* d, const void* const* h,
                                 const void* const* w_packed, float* const* logits,
                                 int32_t* argmax, void* workspace, size_t ws_bytes, void* stream) {
  return exit_heads_impl(true, dt, n_exits, n_tokens, vocab, d, h, w_packed, logits, argmax,
                         workspace, ws_bytes, stream);
}

nel_status nel_matryoshka_loss(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                               const int32_t* d, const void* const* h, const void* const* w,
                               const int32_t* labels, float alpha_d, float grad_scale,
                               const float* exit_weights, int32_t divergence,
                               float* token_loss, float* mean_loss, void* const* dlogits,
                               void* workspace, size_t ws_bytes, void* stream) {
  return loss_impl(false, dt, n_exits, n_tokens, vocab, d, h, w, labels, alpha_d, grad_scale,
                   exit_weights, divergence, token_loss, mean_loss, dlogits, workspace, ws_bytes,
                   stream);
}

nel_status nel_matryoshka_loss_packed(nel_dtype dt, int32_t n_exits, int64_t n_tokens,
                                      int32_t vocab, const int32_t* d, const void* const* h,
                                      const void* const* w_packed, const int32_t* labels,
                                      float alpha_d, float grad_scale, const float* exit_weights,
                                      int32_t divergence, float* token_loss, float* mean_loss,
                                      void* const* dlogits, void* workspace, size_t ws_bytes,
                                      void* stream) {
  return loss_impl(true, dt, n_exits, n_tokens, vocab, d, h, w_packed, labels, alpha_d,
                   grad_scale, exit_weights, divergence, token_loss, mean_loss, dlogits,
                   workspace, ws_bytes, stream);
}

nel_status nel_pack_weights(nel_dtype dt, int32_t vocab, int32_t d, const void* w, void* w_packed,
                            void* stream) {
  if (dt != NEL_BF16) return NEL_EDTYPE;
  if (!packed_shape_ok(vocab, d)) return NEL_ESHAPE;
  if (!w || !w_packed) return NEL_EINVAL;
  if (misaligned(w) || misaligned(w_packed)) return NEL_EALIGN;
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(w_packed);
  const size_t bytes = static_cast<size_t>(vocab) * d * 2;
  if (a < b + bytes && b < a + bytes) return NEL_EINVAL;   // overlapping buffers
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(timed(NEL_K_PACK, s, [&] { return launch_pack_weights(vocab, d, w, w_packed, s); }));
}

size_t nel_speculative_workspace(int32_t batch, int32_t draft_len) {
  if (batch < 0 || draft_len < 0) return 0;
  return speculative_ws_bytes(batch, draft_len) + 256;
}

nel_status nel_speculative_verify(int32_t batch, int32_t positions, int32_t draft_len,
                                  int32_t vocab, const float* draft_logits,
                                  const float* verify_logits, const int32_t* draft_tokens,
                                  const float* u_accept, const float* u_next, float temperature,
                                  float top_p, float* beta, int32_t* accepted,
                                  int32_t* next_token, int32_t* flags, void* workspace,
                                  size_t ws_bytes, void* stream) {
  if (batch < 0 || draft_len < 0 || positions < draft_len + 1 || vocab < 1 || vocab > 32768)
    return NEL_ESHAPE;
  if (static_cast<int64_t>(batch) * (draft_len + 1) * 2 > INT_MAX) return NEL_ESHAPE;
  if (!(temperature > 0.f) || !isfinite(temperature) || !(top_p > 0.f && top_p <= 1.f))
    return NEL_EINVAL;
  if (batch > 0 && (!draft_logits || !verify_logits || !u_next || !accepted || !next_token ||
                    (draft_len > 0 && (!draft_tokens || !u_accept))))
    return NEL_EINVAL;
  if (misaligned4(draft_logits) || misaligned4(verify_logits) || misaligned4(draft_tokens) ||
      misaligned4(u_accept) || misaligned4(u_next) || misaligned4(beta) ||
      misaligned4(accepted) || misaligned4(next_token) || misaligned4(flags) ||
      misaligned(workspace))
    return NEL_EALIGN;
  if (!workspace || ws_bytes < speculative_ws_bytes(batch, draft_len)) return NEL_EWORKSPACE;
  if (batch == 0) return NEL_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(timed(NEL_K_SPECULATIVE, s, [&] {
    return launch_speculative_verify(batch, positions, draft_len, vocab, draft_logits,
                                     verify_logits, draft_tokens, u_accept, u_next, temperature,
                                     top_p, beta, accepted, next_token, flags, workspace, s);
  }));
}

size_t nel_junction_backward_workspace(int64_t n_tokens, int32_t d_in, int32_t d_out,
                                       int32_t vocab) {
  if (n_tokens < 0 || n_tokens > kJunctionBwdMaxTokens || d_in < 0 || d_out <= d_in || vocab < 1)
    return 0;
  return junction_bwd_ws_layout(n_tokens, d_in, d_out, vocab).total;
}

nel_status nel_junction_backward(nel_dtype dt, int64_t n_tokens, int32_t d_in, int32_t d_out,
                                 int32_t vocab, const void* h, const int32_t* ids,
                                 const void* emb, const void* dout, int32_t stop_grad,
                                 int32_t mode, void* dh, float* demb, int32_t* flags,
                                 void* workspace, size_t ws_bytes, void* stream) {
  if (dt != NEL_F32 && dt != NEL_BF16) return NEL_EDTYPE;
  if (n_tokens < 0 || d_in < 0 || d_out <= d_in || vocab < 1) return NEL_ESHAPE;
  if (mode < NEL_JUNCTION_RESCALE || mode > NEL_JUNCTION_ZERO_FILL) return NEL_EINVAL;
  if (n_tokens > kJunctionBwdMaxTokens) return NEL_ESHAPE;
  if (!dh && !demb) return NEL_EINVAL;
  if (d_in == 0 && dh) return NEL_EINVAL;   // block 1 has no h to differentiate
  if (n_tokens > 0 && (!ids || !emb || !dout || (d_in > 0 && !h))) return NEL_EINVAL;
  if (demb && !emb) return NEL_EINVAL;
  if (misaligned(h) || misaligned4(ids) || misaligned(emb) || misaligned(dout) ||
      misaligned(dh) || misaligned(demb) || misaligned4(flags) || misaligned(workspace))
    return NEL_EALIGN;
  const JunctionBwdWs L = junction_bwd_ws_layout(n_tokens, d_in, d_out, vocab);
  if (!workspace || ws_bytes < L.total) return NEL_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(timed(NEL_K_JUNCTION_BWD, s, [&] {
    return dt == NEL_BF16
               ? launch_junction_backward<bf16_t>(n_tokens, d_in, d_out, vocab, h, ids, emb, dout,
                                                  stop_grad != 0, mode, dh, demb, workspace, flags, s)
               : launch_junction_backward<float>(n_tokens, d_in, d_out, vocab, h, ids, emb, dout,
                                                 stop_grad != 0, mode, dh, demb, workspace, flags, s);
  }));
}

// Shape rule of the head backward: bf16, V and d multiples of 64, and every
// grid and 32-bit in-tile byte offset within range.
static bool head_bwd_shape_ok(int64_t n, int32_t vocab, int32_t d) {
  if (n < 0 || vocab < 64 || vocab % 64 != 0 || d < 64 || d % 64 != 0 || d >= (1 << 22))
    return false;
  const int64_t n_pad = (n + 63) / 64 * 64;
  if (n_pad >= (int64_t{1} << 24) || vocab >= (1 << 24)) return false;
  return (n_pad / 64) * (vocab / 64) < (int64_t{1} << 31) &&
         (int64_t{vocab} / 64) * (d / 64) < (int64_t{1} << 31);
}

size_t nel_head_backward_workspace(int64_t n_tokens, int32_t vocab, int32_t d) {
  if (!head_bwd_shape_ok(n_tokens, vocab, d)) return 0;
  return head_bwd_ws_layout(n_tokens, vocab, d).total;
}

nel_status nel_head_backward(nel_dtype dt, int64_t n_tokens, int32_t vocab, int32_t d,
                             const void* dlogits, const void* h, const void* w, void* dh,
                             float* dw, void* workspace, size_t ws_bytes, void* stream) {
  if (dt != NEL_BF16) return NEL_EDTYPE;
  if (!head_bwd_shape_ok(n_tokens, vocab, d)) return NEL_ESHAPE;
  if (!dh && !dw) return NEL_EINVAL;
  if (n_tokens > 0 && (!dlogits || !h || !w)) return NEL_EINVAL;
  if (misaligned(dlogits) || misaligned(h) || misaligned(w) || misaligned(dh) || misaligned(dw) ||
      misaligned(workspace))
    return NEL_EALIGN;
  const HeadBwdWs L = head_bwd_ws_layout(n_tokens, vocab, d);
  if (!workspace || ws_bytes < L.total) return NEL_EWORKSPACE;
  if (n_tokens == 0) {   // no tokens: dH is empty, dW = 0
    if (!dw) return NEL_OK;
    hipStream_t s0 = static_cast<hipStream_t>(stream);
    return from_hip(timed(NEL_K_BWD_DW, s0, [&] {
      return launch_zero_f32(dw, static_cast<int64_t>(vocab) * d, s0);
    }));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* wt = ws + L.wt;
  void* ht = ws + L.ht;
  hipError_t err;
  if (dh) {
    err = timed(NEL_K_BWD_PACK, s, [&] { return launch_pack16_t(w, vocab, d, vocab, wt, s); });
    if (err != hipSuccess) return from_hip(err);
    BwdGroup gh{};
    if (!bwd_group_add(gh, wt, d, dlogits, n_tokens, vocab, vocab, dh, d)) return NEL_ESHAPE;
    err = timed(NEL_K_BWD_DH, s, [&] { return launch_dh_group<false>(gh, s); });
    if (err != hipSuccess) return from_hip(err);
  }
  if (dw) {
    err = timed(NEL_K_BWD_PACK, s, [&] { return launch_pack16_t(h, n_tokens, d, L.n_pad, ht, s); });
    if (err != hipSuccess) return from_hip(err);
    // G itself is the K-major B operand: no transposed copy
    BwdGroup gw{};
    if (!bwd_group_add(gw, ht, d, dlogits, vocab, vocab, L.n_pad, dw, d, n_tokens))
      return NEL_ESHAPE;
    err = timed(NEL_K_BWD_DW, s, [&] { return launch_dw_group<false>(gw, s); });
    if (err != hipSuccess) return from_hip(err);
  }
  return NEL_OK;
}

// Workspace of nel_heads_backward: the per-exit layouts one after another.
static size_t heads_bwd_offset(int32_t e, int64_t n, int32_t vocab, const int32_t* d) {
  size_t o = 0;
  for (int32_t k = 0; k < e; ++k) o += head_bwd_ws_layout(n, vocab, d[k]).total;
  return o;
}

size_t nel_heads_backward_workspace(int32_t n_exits, int64_t n_tokens, int32_t vocab,
                                    const int32_t* d) {
  if (n_exits < 1 || n_exits > NEL_MAX_EXITS || !d) return 0;
  for (int32_t e = 0; e < n_exits; ++e)
    if (!head_bwd_shape_ok(n_tokens, vocab, d[e])) return 0;
  return heads_bwd_offset(n_exits, n_tokens, vocab, d);
}

nel_status nel_heads_backward(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                              const int32_t* d, const void* const* dlogits,
                              const void* const* h, const void* const* w, void* const* dh,
                              float* const* dw, void* workspace, size_t ws_bytes, void* stream) {
  if (dt != NEL_BF16) return NEL_EDTYPE;
  if (n_exits < 1 || n_exits > NEL_MAX_EXITS || !d) return NEL_EINVAL;
  for (int32_t e = 0; e < n_exits; ++e)
    if (!head_bwd_shape_ok(n_tokens, vocab, d[e])) return NEL_ESHAPE;
  if (!dh && !dw) return NEL_EINVAL;
  if (n_tokens > 0 && (!dlogits || !h || !w)) return NEL_EINVAL;
  for (int32_t e = 0; e < n_exits; ++e) {
    if (n_tokens > 0 && (!dlogits[e] || !h[e] || !w[e])) return NEL_EINVAL;
    if ((dh && !dh[e]) || (dw && !dw[e])) return NEL_EINVAL;
    if ((n_tokens > 0 && (misaligned(dlogits[e]) || misaligned(h[e]) || misaligned(w[e]))) ||
        (dh && misaligned(dh[e])) || (dw && misaligned(dw[e])))
      return NEL_EALIGN;
  }
  if (misaligned(workspace)) return NEL_EALIGN;
  if (!workspace || ws_bytes < heads_bwd_offset(n_exits, n_tokens, vocab, d))
    return NEL_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (n_tokens == 0) {   // no tokens: dH is empty, dW = 0
    if (!dw) return NEL_OK;
    for (int32_t e = 0; e < n_exits && err == hipSuccess; ++e)
      err = timed(NEL_K_BWD_DW, s, [&] {
        return launch_zero_f32(dw[e], static_cast<int64_t>(vocab) * d[e], s);
      });
    return from_hip(err);
  }
  char* ws = static_cast<char*>(workspace);
  BwdGroup gh{}, gw{};
  for (int32_t e = 0; e < n_exits; ++e) {
    const HeadBwdWs L = head_bwd_ws_layout(n_tokens, vocab, d[e]);
    char* base = ws + heads_bwd_offset(e, n_tokens, vocab, d);
    if (dh) {
      err = timed(NEL_K_BWD_PACK, s, [&] { return launch_pack16_t(w[e], vocab, d[e], vocab, base + L.wt, s); });
      if (err != hipSuccess) return from_hip(err);
      if (!bwd_group_add(gh, base + L.wt, d[e], dlogits[e], n_tokens, vocab, vocab, dh[e], d[e]))
        return NEL_ESHAPE;
    }
    if (dw) {
      err = timed(NEL_K_BWD_PACK, s, [&] {
        return launch_pack16_t(h[e], n_tokens, d[e], L.n_pad, base + L.ht, s);
      });
      if (err != hipSuccess) return from_hip(err);
      if (!bwd_group_add(gw, base + L.ht, d[e], dlogits[e], vocab, vocab, L.n_pad, dw[e], d[e],
                         n_tokens))
        return NEL_ESHAPE;
    }
  }
  if (dh) {
    err = timed(NEL_K_BWD_DH, s, [&] { return launch_dh_group<false>(gh, s); });
    if (err != hipSuccess) return from_hip(err);
  }
  if (dw) err = timed(NEL_K_BWD_DW, s, [&] { return launch_dw_group<false>(gw, s); });
  return from_hip(err);
}

// Workspace of nel_matryoshka_loss_backward_packed: the loss op's, then the
// gradient row constants (16 bytes per exit, statistics tile and token,
// sized for the narrowest tile), then nel_heads_backward's.
struct LossBwdWs {
  size_t loss, consts, bwd, total;
};
static LossBwdWs loss_bwd_ws_layout(int32_t n_exits, int64_t n, int32_t vocab, const int32_t* d) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  LossBwdWs L;
  L.loss = 0;
  L.consts = up(loss_ws_layout(n_exits, n, vocab).total);
  L.bwd = L.consts + up(size_t{16} * n_exits * static_cast<size_t>(n_vocab_tiles(vocab)) *
                        static_cast<size_t>(n));
  L.total = L.bwd + heads_bwd_offset(n_exits, n, vocab, d);
  return L;
}

size_t nel_loss_backward_workspace(int32_t n_exits, int64_t n_tokens, int32_t vocab,
                                   const int32_t* d) {
  if (nel_heads_backward_workspace(n_exits, n_tokens, vocab, d) == 0) return 0;
  for (int32_t e = 0; e < n_exits; ++e)
    if (!packed_shape_ok(vocab, d[e])) return 0;
  if (!grid_fits(n_tokens, vocab)) return 0;
  return loss_bwd_ws_layout(n_exits, n_tokens, vocab, d).total;
}

nel_status nel_matryoshka_loss_backward_packed(
    nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab, const int32_t* d,
    const void* const* h, const void* const* w, const void* const* w_packed,
    const int32_t* labels, float alpha_d, float grad_scale, const float* exit_weights,
    float* token_loss, float* mean_loss, void* const* scratch, void* const* dh,
    float* const* dw, void* workspace, size_t ws_bytes, void* stream) {
  // everything the backward needs is checked before the loss launches anything
  if (dt != NEL_BF16) return NEL_EDTYPE;
  if (n_exits < 1 || n_exits > NEL_MAX_EXITS || !d) return NEL_EINVAL;
  for (int32_t e = 0; e < n_exits; ++e)
    if (!head_bwd_shape_ok(n_tokens, vocab, d[e]) || !packed_shape_ok(vocab, d[e]))
      return NEL_ESHAPE;
  if (!dh && !dw) return NEL_EINVAL;
  if (!scratch || (n_tokens > 0 && (!h || !w || !w_packed))) return NEL_EINVAL;
  for (int32_t e = 0; e < n_exits; ++e) {
    if (n_tokens > 0 && (!scratch[e] || !h[e] || !w[e] || !w_packed[e])) return NEL_EINVAL;
    if ((dh && n_tokens > 0 && !dh[e]) || (dw && !dw[e])) return NEL_EINVAL;   // dh may be empty
    if ((n_tokens > 0 && (misaligned(scratch[e]) || misaligned(h[e]) || misaligned(w[e]))) ||
        (dh && misaligned(dh[e])) || (dw && misaligned(dw[e])))
      return NEL_EALIGN;
  }
  if (misaligned(workspace)) return NEL_EALIGN;
  if (!grid_fits(n_tokens, vocab)) return NEL_ESHAPE;
  const LossBwdWs L = loss_bwd_ws_layout(n_exits, n_tokens, vocab, d);
  if (!workspace || ws_bytes < L.total) return NEL_EWORKSPACE;
  ExitW lam;
  for (int e = 0; e < kMaxExits; ++e) lam.w[e] = 1.f;
  if (exit_weights)
    for (int e = 0; e < n_exits; ++e) lam.w[e] = exit_weights[e];   // checked by the loss
  char* ws = static_cast<char*>(workspace);
  TileInfo info;
  nel_status st = loss_impl(true, dt, n_exits, n_tokens, vocab, d, h, w_packed, labels, alpha_d,
                            grad_scale, exit_weights, NEL_DIV_FORWARD, token_loss, mean_loss,
                            scratch, ws + L.loss, L.consts - L.loss, stream, /*write_g=*/false,
                            &info);
  if (st != NEL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (n_tokens == 0) {   // no tokens: dH is empty, dW = 0
    if (!dw) return NEL_OK;
    for (int32_t e = 0; e < n_exits && err == hipSuccess; ++e)
      err = timed(NEL_K_BWD_DW, s, [&] {
        return launch_zero_f32(dw[e], static_cast<int64_t>(vocab) * d[e], s);
      });
    return from_hip(err);
  }
  if ((info.vtile & (info.vtile - 1)) != 0 || info.vtile < kPkBRows) return NEL_EINVAL;
  const LossWs LL = loss_ws_layout(n_exits, n_tokens, vocab);
  const float* stats = reinterpret_cast<const float*>(ws + L.loss + LL.stats);
  const float* lse = reinterpret_cast<const float*>(ws + L.loss + LL.lse);
  char* consts = ws + L.consts;
  err = timed(NEL_K_GRAD_CONSTS, s, [&] {
    return launch_grad_consts(n_exits, n_tokens, vocab, info, labels, alpha_d, grad_scale, lam,
                              stats, lse, consts, s);
  });
  if (err != hipSuccess) return from_hip(err);
  const int64_t plane = ((vocab + info.vtile - 1) / info.vtile) * n_tokens;
  BwdGroup gh{}, gw{};
  for (BwdGroup* g : {&gh, &gw}) {
    g->tw = static_cast<const uint16_t*>(scratch[n_exits - 1]);
    g->n_tok = n_tokens;
    g->vshift = __builtin_ctz(static_cast<unsigned>(info.vtile));
  }
  for (int32_t e = 0; e < n_exits; ++e) {
    const HeadBwdWs HL = head_bwd_ws_layout(n_tokens, vocab, d[e]);
    char* base = ws + L.bwd + heads_bwd_offset(e, n_tokens, vocab, d);
    auto fill = [&](BwdGroup& g) {
      const int k = g.count - 1;
      g.tab[k] = consts + size_t{16} * static_cast<size_t>(e) * plane;
      g.neg[k] = grad_scale * lam.w[e] < 0.f ? 0x80008000u : 0u;
    };
    if (dh) {
      err = timed(NEL_K_BWD_PACK, s, [&] { return launch_pack16_t(w[e], vocab, d[e], vocab, base + HL.wt, s); });
      if (err != hipSuccess) return from_hip(err);
      if (!bwd_group_add(gh, base + HL.wt, d[e], scratch[e], n_tokens, vocab, vocab, dh[e], d[e]))
        return NEL_ESHAPE;
      fill(gh);
    }
    if (dw) {
      err = timed(NEL_K_BWD_PACK, s, [&] {
        return launch_pack_t(h[e], n_tokens, d[e], HL.n_pad, base + HL.ht, s);
      });
      if (err != hipSuccess) return from_hip(err);
      if (!bwd_group_add(gw, base + HL.ht, d[e], scratch[e], vocab, vocab, HL.n_pad, dw[e], d[e],
                         n_tokens))
        return NEL_ESHAPE;
      fill(gw);
    }
  }
  if (dh) {
    err = timed(NEL_K_BWD_DH, s, [&] { return launch_dh_group<true>(gh, s); });
    if (err != hipSuccess) return from_hip(err);
  }
  if (dw) err = timed(NEL_K_BWD_DW, s, [&] { return launch_dw_group<true>(gw, s); });
  return from_hip(err);
}

nel_status nel_read_device_flags(const int32_t* dev_flags, int32_t* host_flags, void* stream) {
  if (!dev_flags || !host_flags) return NEL_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = hipMemcpyAsync(host_flags, dev_flags, sizeof(int32_t),
                                      hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(hipStreamSynchronize(s));
}

nel_status nel_clear_device_flags(int32_t* dev_flags, void* stream) {
  if (!dev_flags) return NEL_EINVAL;
  if (misaligned4(dev_flags)) return NEL_EALIGN;
  (void)hipGetLastError();
  return from_hip(launch_clear_flags(dev_flags, static_cast<hipStream_t>(stream)));
}

nel_status nel_timing_enable(int32_t on) {
  timing().on.store(on != 0, std::memory_order_relaxed);
  return NEL_OK;
}

nel_status nel_timing_reset(void) {
  Timing& T = timing();
  std::lock_guard<std::mutex> g(T.mu);
  for (auto& p : T.pending) {
    (void)hipEventSynchronize(p.b);
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  T.pending.clear();
  for (int k = 0; k < NEL_K_COUNT; ++k) {
    T.total_ms[k] = 0.0;
    T.launches[k] = 0;
  }
  return NEL_OK;
}

nel_status nel_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= NEL_K_COUNT || !total_ms || !launches) return NEL_EINVAL;
  Timing& T = timing();
  std::lock_guard<std::mutex> g(T.mu);
  nel_status st = NEL_OK;
  for (auto& p : T.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(p.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.a, p.b);
    if (e != hipSuccess) st = from_hip(e);
    T.total_ms[p.k] += ms;
    T.launches[p.k] += 1;
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  T.pending.clear();
  *total_ms = T.total_ms[kernel];
  *launches = T.launches[kernel];
  return st;
}

}  // extern "C"
