/*
 * nel.h -- C ABI of the Matryoshka multi-exit hot path on MI355X (gfx950).
 *
 * A Matryoshka suite nests M sub-models in one network: block m has width D_m
 * (D_1 < ... < D_M), every exit m has its own LM head W^m in R^{V x D_m}, and a
 * parameter-free junction joins block m to block m+1.  This library computes,
 * on one GPU, the junction, every exit's logits, and the loss in which the
 * largest exit's softmax teaches the smaller exits, together with the loss's
 * gradient with respect to every exit's logits.
 *
 * Sources (the paper's equations are referenced, not printed, on the pages):
 *   "Matryoshka Language Model Suites" (paper summary): paragraphs on the
 *     junction, on distillation and on speculative decoding;
 *   "Visualizing Core ideas": panels (b), (c) and (e);
 *   "Visualizing the core idea of Matryoshka LM Suites": bottom panel;
 *   copyedit of Sec. 2 "Modeling": notation x, e_m, D_0 = 0, W^m;
 *   "Is nesting the cheapest way to build a model suite?", follow-up 4:
 *     the 0.7 / 0.3 mix of next-token loss and cross-entropy to the largest exit.
 *
 * Conventions shared by every entry point
 *   - All tensors are device pointers to dense row-major arrays; the caller
 *     allocates and owns every buffer (inputs, outputs, workspace).  The
 *     library never allocates, frees or retains a pointer after returning.
 *   - Element type: NEL_BF16 (bfloat16 storage, fp32 arithmetic) or NEL_F32.
 *   - Base pointers of bf16/fp32 tensors (h, w, emb, junction output,
 *     dlogits, fp32 logits) and of the workspace must be 16-byte aligned;
 *     int32 arrays (ids, labels, argmax, accepted, flags) and the fp32 loss
 *     outputs need 4-byte alignment (NEL_EALIGN otherwise).  Rows whose
 *     length is not a multiple of 16 bytes take masked element paths, so
 *     any V >= 1 and D >= 1 are accepted.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it; no call synchronises except nel_read_device_flags and
 *     nel_timing_read.
 *   - A workspace is in use until the call's work on `stream` has finished.
 *     Calls that may run at the same time (on different streams) need
 *     separate workspaces; calls on one stream may share one.  The library
 *     keeps no device state between calls; its only host state is the
 *     timing record (nel_timing_*, see there) and the per-thread last HIP
 *     error.
 *   - Host-detectable errors are returned synchronously and nothing is
 *     launched.  Data errors found on the device (a token id or label outside
 *     [0, V)) set a bit in a device flag word (NEL_FLAG_*) and turn that
 *     token's outputs into NaN; the flag word is sticky (OR-ed), the caller
 *     clears it (nel_clear_device_flags or zero-initialised memory).
 *   - Token ids and labels are 0-based int32 in [0, V).
 */
#ifndef NEL_H
#define NEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NEL_OK = 0,
  NEL_EINVAL = -1,      /* bad scalar argument (alpha, n_exits, op, NULL required pointer) */
  NEL_ESHAPE = -2,      /* a size <= 0 where >= 1 is required, or widths not strictly increasing */
  NEL_EDTYPE = -3,      /* unknown element type */
  NEL_EALIGN = -4,      /* a base pointer below its required alignment */
  NEL_EWORKSPACE = -5,  /* workspace NULL or smaller than nel_workspace_size() */
  NEL_EHIP = -6,        /* the HIP runtime reported an error at launch */
  NEL_ETOOLARGE = -7    /* beyond the fixed scratch of nel_exit_heads_packed_noalloc */
} nel_status;

typedef enum { NEL_F32 = 0, NEL_BF16 = 1 } nel_dtype;

enum { NEL_FLAG_BAD_ID = 1, NEL_FLAG_BAD_LABEL = 2 };

enum { NEL_OP_LOSS = 0, NEL_OP_HEADS = 1 };

enum { NEL_MAX_EXITS = 8 };

/* Distillation divergences D(p, q), p = the teacher's softmax, q a smaller
 * exit's.  NEL_DIV_FORWARD is the method (summary's distillation paragraph;
 * follow-up 4 of "Is nesting the cheapest way to build a model suite?": 0.3
 * cross-entropy to the largest model).  The others are the swaps the same
 * follow-up proposes; its acceptance loss is read as the total variation,
 * 1 - beta with beta = sum_v min(p_v, q_v) the acceptance probability. */
typedef enum {
  NEL_DIV_FORWARD = 0,      /* -sum p log q */
  NEL_DIV_REVERSE_KL = 1,   /* sum q (log q - log p) */
  NEL_DIV_JS = 2,           /* (KL(p || m) + KL(q || m)) / 2, m = (p + q) / 2 */
  NEL_DIV_TV = 3            /* sum |p - q| / 2 */
} nel_divergence;

/* Junction modes: the method's junction and the two ablations of the paper
 * summary's junction paragraph and the key-visual explainer (200M scale):
 * dropping the norm match, and filling the new channels with zeros. */
typedef enum {
  NEL_JUNCTION_RESCALE = 0,     /* out = [h ||g|| / ||h||, g]  (the method) */
  NEL_JUNCTION_NO_RESCALE = 1,  /* out = [h, g] */
  NEL_JUNCTION_ZERO_FILL = 2    /* out = [h ||g|| / ||h||, 0]: the target norm is
                                   still the fresh embedding's */
} nel_junction_mode;

/*
 * Junction (the paper's Eq. 1, as stated in prose by the summary's junction
 * paragraph and the key-visual explainer's bottom panel; block inputs from the
 * copyedit of Sec. 2).  For every token t, with g = emb[ids[t]]:
 *     out[t, :d_in]     = h[t] * ||g||_2 / ||h[t]||_2       (0 if either norm is 0)
 *     out[t, d_in:d_out] = g                                 (bit-exact copy)
 * d_in == 0 is block 1's input: out[t] = emb[ids[t]] (h may be NULL).
 *   h:   [n_tokens, d_in]             dt     (input)
 *   ids: [n_tokens] int32 in [0,vocab)       (input)
 *   emb: [vocab, d_out - d_in]         dt     (input; the residual table e_{m+1})
 *   out: [n_tokens, d_out]             dt     (output; must not alias the inputs)
 *   mode: a nel_junction_mode (NEL_JUNCTION_RESCALE is the method)
 *   flags: device int32 flag word or NULL; a bad id sets NEL_FLAG_BAD_ID and
 *          writes a NaN row.
 * Norms are accumulated in fp32; each output element is rounded once.
 * Errors: NEL_ESHAPE if n_tokens < 0, d_in < 0, d_out <= d_in or vocab < 1;
 * NEL_EINVAL for an unknown mode.
 */
nel_status nel_junction(nel_dtype dt, int64_t n_tokens, int32_t d_in, int32_t d_out,
                        int32_t vocab, const void* h, const int32_t* ids, const void* emb,
                        void* out, int32_t mode, int32_t* flags, void* stream);

/*
 * Exit heads with greedy argmax (copyedit of Sec. 2: sub-model m ends in its
 * own head W^m; the summary's speculative-decoding paragraph: greedy drafting
 * and verification read the argmax of an exit's logits).  For each of the
 * n_exits exits e (any subset of a suite, widths d[e] strictly increasing):
 *     logits_e = h[e] · w[e]^T       fp32 accumulation, [n_tokens, vocab]
 *     argmax[e * n_tokens + t] = lowest index of the row maximum
 *   d:      host array [n_exits]
 *   h:      host array of n_exits device pointers, h[e] is [n_tokens, d[e]] dt
 *   w:      host array of n_exits device pointers, w[e] is [vocab, d[e]]   dt
 *   logits: NULL, or host array of n_exits device pointers to fp32 [n_tokens, vocab]
 *   argmax: NULL, or device int32 [n_exits, n_tokens]
 *   workspace: device, >= nel_workspace_size(NEL_OP_HEADS, ...) bytes
 */
nel_status nel_exit_heads(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                          const int32_t* d, const void* const* h, const void* const* w,
                          float* const* logits, int32_t* argmax, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * Greedy acceptance (summary's speculative-decoding paragraph: exit 1 drafts,
 * the largest exit verifies, draft length 6).  For each sequence b, with
 * P = positions tokens laid out [batch, positions]:
 *     accepted[b] = number of leading i < draft_len with
 *                   draft_argmax[b*P + i] == verify_argmax[b*P + i]
 * Requires 0 <= draft_len <= positions.  All arrays are device int32.
 */
nel_status nel_accept_prefix(int32_t batch, int32_t positions, int32_t draft_len,
                             const int32_t* draft_argmax, const int32_t* verify_argmax,
                             int32_t* accepted, void* stream);

/*
 * Sampled speculative verification ("Is nesting the cheapest way to build a
 * model suite?", follow-up 4: a drafted token is accepted with probability
 * beta = sum_v min(p_v, q_v); "Matryoshka Language Model Suites",
 * speculative-decoding paragraph: exit 1 drafts, the largest exit verifies,
 * also under nucleus sampling).  For sequence b and position i of P, p and q
 * are the draft and verifying exits' distributions: softmax(logits / T)
 * restricted to the nucleus (the most probable entries whose probability
 * reaches top_p, entries tied with the last one needed kept too) and
 * renormalised.  Then
 *     beta[b, i]    = sum_v min(p_v, q_v)                         (i < draft_len)
 *     accepted[b]   = number of leading i < draft_len with u_accept[b, i] p(x_i) < q(x_i),
 *                     x_i = draft_tokens[b, i]
 *     next_token[b] = after a rejection at k: a draw from max(0, q_k - p_k)
 *                     (from q_k if that is all zero); otherwise a draw from q
 *                     at position draft_len.  The draw is the first entry (in
 *                     vocabulary order) where the running sum of the weights
 *                     exceeds u_next[b] times their total.
 *   draft_logits, verify_logits: device fp32 [batch, positions, vocab] (e.g.
 *       the logits output of nel_exit_heads*), positions >= draft_len + 1
 *   draft_tokens, u_accept: device [batch, positions] (int32, fp32 in [0, 1))
 *   u_next: device fp32 [batch] in [0, 1);  beta: NULL or fp32 [batch, draft_len]
 *   accepted, next_token: device int32 [batch]
 *   flags: NULL or device flag word: a drafted token outside [0, vocab) sets
 *       NEL_FLAG_BAD_ID and counts as rejected
 *   workspace: >= nel_speculative_workspace(batch, draft_len) bytes.  When the
 *       call's work has completed, its first 2 * batch * (draft_len + 1) fp32
 *       quadruples hold the statistics of every row, the draft exit's first:
 *       quadruple (x * batch + b) * (draft_len + 1) + i, x = 0 draft / 1 verify,
 *       is {max_v fl(l_v / T), nucleus mass sum_{kept} e_v, the threshold (the
 *       smallest e_v kept; 0 when top_p = 1), the softmax mass sum_v e_v},
 *       with e_v = exp(fl(l_v / T) - max) in fp32 and entry v kept iff
 *       e_v >= the threshold.  Nothing else is returned there.
 * Every decision is taken in fp32 from the given logits.  Requires
 * vocab <= 32768 (NEL_ESHAPE), temperature > 0 and 0 < top_p <= 1 (NEL_EINVAL).
 */
nel_status nel_speculative_verify(int32_t batch, int32_t positions, int32_t draft_len,
                                  int32_t vocab, const float* draft_logits,
                                  const float* verify_logits, const int32_t* draft_tokens,
                                  const float* u_accept, const float* u_next, float temperature,
                                  float top_p, float* beta, int32_t* accepted,
                                  int32_t* next_token, int32_t* flags, void* workspace,
                                  size_t ws_bytes, void* stream);
size_t nel_speculative_workspace(int32_t batch, int32_t draft_len);

/*
 * Matryoshka loss with online distillation and its logit gradients (summary's
 * distillation and limitations paragraphs; follow-up 4's 0.7/0.3 mix;
 * main-visual explainer panel (b): distillation only into smaller exits).
 * Exit n_exits-1 is the teacher M; p = softmax(l_M) is under stop-gradient.
 * Per token t and exit m, with l_m = h[m] · w[m]^T (fp32 accumulation) and
 * q_m = softmax(l_m):
 *     CE_m   = logsumexp(l_m) - l_m[y_t]
 *     Dist_m = D(p, q_m)                                  (m < M; 0 for M)
 *              NEL_DIV_FORWARD: logsumexp(l_m) - sum_v p_v l_m,v
 *     L_m    = (1 - alpha_d) CE_m + alpha_d Dist_m       (m < M),  L_M = CE_M
 *     total  = sum_m lambda_m L_m
 *   exit_weights: NULL (every lambda_m = 1, the summary's equal weights) or a
 *               host array of n_exits finite values >= 0 (the reweighting
 *               of the limitations paragraph)
 *   divergence: a nel_divergence; other than NEL_DIV_FORWARD it needs dlogits
 *               (its pass reads every exit's stored shifted logits)
 *   token_loss: NULL, or device fp32 [n_exits, 3, n_tokens] = (CE, Dist, L)
 *   mean_loss:  device fp32 [3*n_exits + 1]: mean over tokens of CE_0..CE_{M-1},
 *               then Dist_0.., then L_0.., then the total (fixed-order sums)
 *   dlogits:    NULL (loss only), or host array of n_exits device pointers,
 *               dlogits[e] is [n_tokens, vocab] of type dt, written with
 *               grad_scale * d(sum_t total_t)/d l_e:
 *                 m < M: grad_scale lambda_m ((1-alpha_d)(q_m - onehot(y)) + alpha_d dD/dl_m)
 *                        (NEL_DIV_FORWARD: dD/dl_m = q_m - p)
 *                 M:     grad_scale lambda_M (p - onehot(y))
 *   labels: device int32 [n_tokens]; a label outside [0,vocab) sets
 *           NEL_FLAG_BAD_LABEL in the workspace's first word and NaNs that token.
 *   workspace: device, >= nel_workspace_size(NEL_OP_LOSS, ...) bytes; its
 *           first int32 is the device flag word.
 * No fp32 logit tensor is ever written to memory.  With NEL_DIV_FORWARD the
 * distillation term comes from fp32 logits; the other divergences are summed
 * from the stored shifted logits (fp16 for dt = NEL_BF16).
 * Errors: NEL_EINVAL if alpha_d is outside [0,1], n_exits outside [1,8], a
 * weight is negative or not finite, the divergence is unknown, or it needs
 * dlogits and they are NULL.
 */
nel_status nel_matryoshka_loss(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                               const int32_t* d, const void* const* h, const void* const* w,
                               const int32_t* labels, float alpha_d, float grad_scale,
                               const float* exit_weights, int32_t divergence,
                               float* token_loss, float* mean_loss, void* const* dlogits,
                               void* workspace, size_t ws_bytes, void* stream);

/*
 * MFMA-tiled head weights.  The contraction of every exit head (copyedit of
 * Sec. 2: sub-model m ends in its own head W^m) runs fastest when each matrix
 * core operand is one contiguous 1 KB read, so a bf16 head W [vocab, d] may be
 * rewritten once into the tiled layout below and then used by the *_packed
 * entry points, which compute exactly what their row-major counterparts do.
 * Requires dt == NEL_BF16, vocab % 32 == 0 and below 2^24, d % 64 == 0 and
 * below 2^24 (NEL_ESHAPE).  The layout, for row
 * block rb < vocab/16, column block kb < d/32, lane l < 64, j < 8:
 *     packed[((rb * (d/32) + kb) * 64 + l) * 8 + j] = w[16 rb + l % 16][32 kb + 8 (l / 16) + j]
 * (one A operand of the 16x16x32 bf16 matrix instruction per 1 KB block).
 *   w:        device bf16 [vocab, d] (input)
 *   w_packed: device bf16, vocab * d elements (output; must not overlap w)
 * Errors: NEL_EDTYPE unless bf16; NEL_ESHAPE if vocab or d breaks the rule
 * above; NEL_EINVAL for NULL or overlapping buffers; NEL_EALIGN below 16 bytes.
 */
nel_status nel_pack_weights(nel_dtype dt, int32_t vocab, int32_t d, const void* w,
                            void* w_packed, void* stream);

/*
 * nel_matryoshka_loss with every w[e] in the tiled layout of
 * nel_pack_weights.  Same arguments, outputs and errors, plus: dt must be
 * NEL_BF16 (NEL_EDTYPE), vocab % 32 == 0 and every d[e] % 64 == 0, both
 * below 2^24 (NEL_ESHAPE), and dlogits must be given (NEL_EINVAL): between the head GEMM
 * and the final gradient pass the dlogits buffers hold 16-bit scratch.  With
 * NEL_DIV_FORWARD the teacher's holds its softmax weights exp(l_M - m) (m the
 * 256-entry tile maximum) and the smaller exits' hold l - m, all fp16; the
 * gradient pass forms the teacher-weighted logit sums of Dist from them.  The
 * other divergences store l - m in fp16 for every exit.  Every dlogits buffer
 * is scratch until the call's work on `stream` has completed.
 */
nel_status nel_matryoshka_loss_packed(nel_dtype dt, int32_t n_exits, int64_t n_tokens,
                                      int32_t vocab, const int32_t* d, const void* const* h,
                                      const void* const* w_packed, const int32_t* labels,
                                      float alpha_d, float grad_scale, const float* exit_weights,
                                      int32_t divergence, float* token_loss, float* mean_loss,
                                      void* const* dlogits, void* workspace, size_t ws_bytes,
                                      void* stream);

/*
 * nel_exit_heads with every w[e] in the tiled layout of nel_pack_weights
 * (dt NEL_BF16, vocab % 32 == 0, every d[e] % 64 == 0, both below 2^24; same
 * outputs and errors).
 */
nel_status nel_exit_heads_packed(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                                 const int32_t* d, const void* const* h,
                                 const void* const* w_packed, float* const* logits,
                                 int32_t* argmax, void* workspace, size_t ws_bytes, void* stream);

/*
 * nel_exit_heads_packed for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, outputs and errors, without the workspace: the
 * per-tile partial results live in a fixed device array of
 * NEL_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  It calls no allocating routine (nor the timing
 * hooks, which create events).  The caller still passes inputs and outputs.
 *   - A request whose partial results exceed the array is NEL_ETOOLARGE (with
 *     nothing launched): it needs 256 + 8 * n_exits * n_tokens * ceil(vocab / 128)
 *     bytes, e.g. up to 4095 tokens for two exits at vocab 32768.
 *   - Every call on one GPU shares that GPU's array, and nothing in it has to
 *     start at zero (each call writes every value it reads).  Calls that
 *     overlap on one GPU (other streams, other threads) race: serialise them.
 *   - `stream` must belong to the current device (NEL_EINVAL otherwise).
 *   - The array's device address is looked up on the first call on a device
 *     (hipGetSymbolAddress, no allocation).
 */
enum { NEL_NOALLOC_SCRATCH_BYTES = 16 << 20 };
nel_status nel_exit_heads_packed_noalloc(nel_dtype dt, int32_t n_exits, int64_t n_tokens,
                                         int32_t vocab, const int32_t* d, const void* const* h,
                                         const void* const* w_packed, float* const* logits,
                                         int32_t* argmax, void* stream);

/*
 * Backward of the junction (nel_junction).  With g = emb[ids[t]], a = ||h[t]||,
 * b = ||g||, the forward out[t] = [h[t] b / a, g] and the upstream gradient
 * dout[t] = [dh_up, dg_up] (split at d_in), the chain rule gives
 *     dh[t]   = (b / a) (dh_up - h[t] (h[t] . dh_up) / a^2)        (0 if a or b is 0)
 *     demb[v] = sum_{t: ids[t] = v} (dg_up[t] + c_t g / b),  c_t = (h[t] . dh_up) / a
 * ("Matryoshka Language Model Suites", junction paragraph, for the forward).
 * stop_grad != 0 is arm (B) of follow-up 2 on "Is nesting the cheapest way to
 * build a model suite?": no gradient reaches h through the junction (dh = 0)
 * while the embedding still receives both terms.  mode (nel_junction_mode)
 * selects the forward it differentiates: NEL_JUNCTION_NO_RESCALE gives
 * dh = dh_up and demb[v] = sum dg_up; NEL_JUNCTION_ZERO_FILL drops the dg_up
 * term (the zeros do not depend on emb).
 *   h:     [n_tokens, d_in] dt, or NULL when d_in == 0 (block 1)
 *   ids:   [n_tokens] int32;  emb: [vocab, d_out - d_in] dt;  dout: [n_tokens, d_out] dt
 *   dh:    NULL or [n_tokens, d_in] dt (must be NULL when d_in == 0)
 *   demb:  NULL or fp32 [vocab, d_out - d_in], every row written (0 for ids
 *          no token uses).  Each row's tokens are taken in token order, in
 *          consecutive groups of 64 summed in order, and the group sums are
 *          added in order: reruns are bit-identical
 *   flags: device flag word or NULL; a bad id sets NEL_FLAG_BAD_ID, NaNs its dh
 *          row and contributes nothing to demb
 *   workspace: >= nel_junction_backward_workspace(n_tokens, d_in, d_out, vocab)
 *          bytes (grows with n_tokens * vocab / 256 and with the embedding width)
 * n_tokens above 2^30 is NEL_ESHAPE.
 */
nel_status nel_junction_backward(nel_dtype dt, int64_t n_tokens, int32_t d_in, int32_t d_out,
                                 int32_t vocab, const void* h, const int32_t* ids,
                                 const void* emb, const void* dout, int32_t stop_grad,
                                 int32_t mode, void* dh, float* demb, int32_t* flags,
                                 void* workspace, size_t ws_bytes, void* stream);
/* Bytes of workspace nel_junction_backward needs (0 on bad arguments). */
size_t nel_junction_backward_workspace(int64_t n_tokens, int32_t d_in, int32_t d_out,
                                       int32_t vocab);

/*
 * Backward of one exit head (the step after the loss: l = h W^T with W the
 * exit's head, copyedit of Sec. 2 "Modeling"; G = dL/dl from
 * nel_matryoshka_loss*).  By the chain rule, with fp32 accumulation:
 *     dh = G W       [n_tokens, d]  in dt (bf16)
 *     dw = G^T h     [vocab, d]     fp32
 *   dlogits: device bf16 [n_tokens, vocab] (G, input)
 *   h:       device bf16 [n_tokens, d]     (the exit's block output, input)
 *   w:       device bf16 [vocab, d]        (the head, row-major, input)
 *   dh, dw:  device outputs, each may be NULL (not both); they must not alias
 *            the inputs or the workspace
 *   workspace: device, >= nel_head_backward_workspace() bytes (the
 *            transposed, MFMA-tiled copies of W and h; G is read in place)
 * Requires dt == NEL_BF16 (NEL_EDTYPE), vocab and d multiples of 64, d below
 * 2^22 and the padded token count below 2^24 (NEL_ESHAPE).  n_tokens == 0
 * sets dw to 0.
 */
nel_status nel_head_backward(nel_dtype dt, int64_t n_tokens, int32_t vocab, int32_t d,
                             const void* dlogits, const void* h, const void* w, void* dh,
                             float* dw, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace nel_head_backward needs (0 on bad arguments). */
size_t nel_head_backward_workspace(int64_t n_tokens, int32_t vocab, int32_t d);

/*
 * nel_head_backward for every exit of a suite at once: the same outputs,
 * bit-identical, but each of the two GEMMs (dh for all exits, then dw for
 * all exits) is one launch, so one exit's workgroups fill another's last
 * partial round on the device.
 *   d:       host array [n_exits] of widths (each a multiple of 64)
 *   dlogits, h, w: host arrays of n_exits device pointers, as in nel_head_backward
 *   dh, dw:  NULL (skip that output for every exit) or host arrays of n_exits
 *            device pointers, none NULL; not both NULL
 *   workspace: >= nel_heads_backward_workspace() bytes
 * Errors as nel_head_backward; NEL_EINVAL for n_exits outside [1, 8] or a
 * NULL entry.
 */
nel_status nel_heads_backward(nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab,
                              const int32_t* d, const void* const* dlogits,
                              const void* const* h, const void* const* w, void* const* dh,
                              float* const* dw, void* workspace, size_t ws_bytes, void* stream);
/* Bytes of workspace nel_heads_backward needs (0 on bad arguments). */
size_t nel_heads_backward_workspace(int32_t n_exits, int64_t n_tokens, int32_t vocab,
                                    const int32_t* d);

/*
 * The loss and the backward of every exit head in one call, with the logit
 * gradients G_e never written to memory.  G_e is the gradient
 * nel_matryoshka_loss_packed (NEL_DIV_FORWARD) writes into dlogits[e], i.e.
 * grad_scale lambda_e d(sum_t total_t)/d l_e with the teacher under
 * stop-gradient ("Matryoshka Language Model Suites", distillation paragraph;
 * the backward through l = h W^T follows from the head of the copyedit of
 * Sec. 2 "Modeling"):
 *     dh[e] = G_e W_e      [n_tokens, d_e] bf16
 *     dw[e] = G_e^T h_e    [vocab, d_e]    fp32
 * The head GEMM leaves its 16-bit scratch in scratch[e]; the dh and dw GEMMs
 * form each 64-entry slice of G_e from it and per-row constants in
 * registers, with the arithmetic of the gradient pass, so G_e is bit for
 * bit the one nel_matryoshka_loss_packed stores (same inputs, dlogits =
 * scratch): dh is then bit-identical to nel_heads_backward on the stored
 * gradients, and dw sums the same products in another fp32 order.
 *   h, labels, alpha_d, grad_scale, exit_weights, token_loss, mean_loss:
 *            as nel_matryoshka_loss (the divergence is NEL_DIV_FORWARD)
 *   w:        host array of n_exits device bf16 [vocab, d_e] (row-major heads,
 *            read by the dh GEMM's transposing pack)
 *   w_packed: the same heads in the layout of nel_pack_weights
 *   scratch:  host array of n_exits device buffers of n_tokens * vocab 16-bit
 *            entries (no alias); their contents on return are scratch
 *   dh, dw:   NULL (skip that output for every exit) or host arrays of n_exits
 *            device pointers, none NULL (dh's may be when n_tokens is 0); not
 *            both NULL
 *   workspace: >= nel_loss_backward_workspace() bytes; its first int32 is the
 *            device flag word (NEL_FLAG_BAD_LABEL: that token's losses, its
 *            rows of dh and, through the sum over tokens, all of dw are NaN)
 * Requires dt == NEL_BF16 (NEL_EDTYPE); vocab and every d_e multiples of 64,
 * d_e below 2^22, the padded token count below 2^24 (NEL_ESHAPE).  Other
 * errors as nel_matryoshka_loss_packed and nel_heads_backward; on any error
 * nothing is launched.  n_tokens == 0 writes the means and sets dw to 0.
 */
nel_status nel_matryoshka_loss_backward_packed(
    nel_dtype dt, int32_t n_exits, int64_t n_tokens, int32_t vocab, const int32_t* d,
    const void* const* h, const void* const* w, const void* const* w_packed,
    const int32_t* labels, float alpha_d, float grad_scale, const float* exit_weights,
    float* token_loss, float* mean_loss, void* const* scratch, void* const* dh,
    float* const* dw, void* workspace, size_t ws_bytes, void* stream);
/* Bytes of workspace nel_matryoshka_loss_backward_packed needs (0 on bad arguments). */
size_t nel_loss_backward_workspace(int32_t n_exits, int64_t n_tokens, int32_t vocab,
                                   const int32_t* d);

/* Bytes of device workspace an op needs (0 on bad arguments). */
size_t nel_workspace_size(int32_t op, int32_t n_exits, int64_t n_tokens, int32_t vocab);

/* Copy the device flag word to *host_flags; synchronises `stream`. */
nel_status nel_read_device_flags(const int32_t* dev_flags, int32_t* host_flags, void* stream);

/* Zero the device flag word (a one-thread kernel on `stream`). */
nel_status nel_clear_device_flags(int32_t* dev_flags, void* stream);

/* Static text for a status code. */
const char* nel_status_string(nel_status s);

/* Name of the HIP error behind the calling thread's most recent NEL_EHIP
 * ("none" if there was none); static storage. */
const char* nel_last_hip_error(void);

/*
 * Measurement hooks.  While enabled, every kernel launch is bracketed by a
 * pair of hipEvents recorded on the stream it is launched on, and
 * nel_timing_read sums their elapsed times per kernel.  Kernel ids:
 * 0 junction, 1 heads+loss statistics GEMM, 2 loss merge, 3 means,
 * 4 dlogits finalize, 5 heads+argmax GEMM, 6 argmax merge, 7 accept,
 * 8 weight packing, 9 head-backward operand packs, 10 dH GEMM, 11 dW GEMM,
 * 12 junction backward, 13 sampled speculative verification, 14 divergence pass,
 * 15 gradient row constants (fused loss backward; that call's gradient pass,
 * which then writes no gradients, counts as 4).
 * The record is process-global.  A lock guards it, so launching and reading
 * from several threads is free of data races, but launches from every thread
 * and stream are summed together: for benchmarks, with one thread launching.
 */
enum { NEL_K_JUNCTION = 0, NEL_K_HEADS_LOSS = 1, NEL_K_MERGE = 2, NEL_K_MEANS = 3,
       NEL_K_FINALIZE = 4, NEL_K_HEADS_ARGMAX = 5, NEL_K_ARGMAX_MERGE = 6,
       NEL_K_ACCEPT = 7, NEL_K_PACK = 8, NEL_K_BWD_PACK = 9, NEL_K_BWD_DH = 10,
       NEL_K_BWD_DW = 11, NEL_K_JUNCTION_BWD = 12, NEL_K_SPECULATIVE = 13,
       NEL_K_DIVERGENCE = 14, NEL_K_GRAD_CONSTS = 15, NEL_K_COUNT = 16 };
nel_status nel_timing_enable(int32_t on);
/* Synchronises the device, then returns the summed milliseconds and the
 * number of timed launches of `kernel` since the last reset. */
nel_status nel_timing_read(int32_t kernel, double* total_ms, int64_t* launches);
nel_status nel_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* NEL_H */
