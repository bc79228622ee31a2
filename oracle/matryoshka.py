"""Float64 NumPy definitions of the junction, the exit heads, the
Matryoshka distillation loss with its logit gradients, greedy argmax and
accepted-prefix length.  Test infrastructure only (see the package header).

Nothing here is blocked, fused or reordered beyond the definitions; the only
concession to size is ``forward_tokens``, which evaluates the same
definitions on a chosen subset of tokens (tokens are independent).
"""
from __future__ import annotations

import contextlib
from typing import Dict, List, Optional, Sequence

import numpy as np

# Working precision of every definition below: float64 for all parity use.
# The benchmark's CPU baseline also times the same definitions in float32
# (``working_precision``); that changes the type the steps run in, not the
# steps.
_DTYPE = np.float64


def _real(x) -> np.ndarray:
    return np.asarray(x, dtype=_DTYPE)


@contextlib.contextmanager
def working_precision(dtype):
    """Run the definitions in ``dtype`` (np.float32 for the CPU speed
    baseline) inside the block; float64 again afterwards."""
    global _DTYPE
    old = _DTYPE
    _DTYPE = np.dtype(dtype).type
    try:
        yield
    finally:
        _DTYPE = old


# ---------------------------------------------------------------------------
# Junction
# ---------------------------------------------------------------------------
# Junction modes: the method's junction and the two ablations the paper
# summary and the key-visual explainer report at 200M scale (dropping the
# norm match; filling the new channels with zeros).
JUNCTION_RESCALE, JUNCTION_NO_RESCALE, JUNCTION_ZERO_FILL = 0, 1, 2


def junction(h: Optional[np.ndarray], ids: np.ndarray, emb: np.ndarray,
             mode: int = JUNCTION_RESCALE) -> np.ndarray:
    """Parameter-free junction between block m and block m+1.

    "Matryoshka Language Model Suites", junction paragraph, and the key-visual
    explainer's bottom panel: the m-th output is rescaled to the L2 norm of
    the fresh embedding of the same token and the two are concatenated along
    channels; no parameters.  Copyedit of Sec. 2 "Modeling": block m+1 reads
    the previous block's output together with its own residual table
    e_{m+1} applied to the original tokens x; with D_0 = 0 block 1 reads
    e_1[x] alone.

    Readings: per token, L2 over channels; no epsilon; the rescaled output
    fills the first D_m channels and the embedding the last
    D_{m+1} - D_m; if either norm is zero the rescaled half is zero.

    Ablation modes (same passages, the 200M ablation sentences):
      JUNCTION_NO_RESCALE: out = [h, g]   (the norm match dropped)
      JUNCTION_ZERO_FILL:  out = [h b / a, 0]   (the new channels are zeros;
        reading: the rescale target stays the fresh embedding's norm b, since
        rescaling to the norm of the zeros would erase h altogether)

    h:   [N, D_in] (None or D_in == 0 for block 1); ids: [N] in [0, V);
    emb: [V, D_out - D_in].  Returns float64 [N, D_out].
    """
    g = _real(emb)[np.asarray(ids, dtype=np.int64)]
    fill = np.zeros_like(g) if mode == JUNCTION_ZERO_FILL else g
    if h is None or np.asarray(h).shape[1] == 0:
        return fill
    hf = _real(h)
    if mode == JUNCTION_NO_RESCALE:
        return np.concatenate([hf, g], axis=1)
    a = np.sqrt(np.sum(hf * hf, axis=1))
    b = np.sqrt(np.sum(g * g, axis=1))
    scale = np.zeros_like(a)
    ok = (a > 0) & (b > 0)
    scale[ok] = b[ok] / a[ok]
    return np.concatenate([hf * scale[:, None], fill], axis=1)


def junction_backward(h: Optional[np.ndarray], ids: np.ndarray, emb: np.ndarray,
                      dout: np.ndarray, stop_grad: bool = False,
                      mode: int = JUNCTION_RESCALE):
    """Gradients of `junction` by the chain rule, given dL/dout.

    Forward per token: g = e[x], a = ||h||, b = ||g||, out = [h b / a, g]
    (junction paragraph of the paper summary; 0 rescaled half if a or b is 0).
    With dout = [du, dg] split at d_in:
        dL/dh   = (b / a) (du - h (h . du) / a^2)
        dL/dg   = dg + ((h . du) / a) g / b      (d||g||/dg = g / ||g||)
    and dL/de[v] sums dL/dg over the tokens with id v.  The ablation modes
    drop terms: JUNCTION_NO_RESCALE has dL/dh = du and dL/dg = dg;
    JUNCTION_ZERO_FILL has no dg term (the zeros do not depend on e).
    stop_grad (arm (B) of follow-up 2 on the follow-ups page: every block
    learns only from its own exit) treats h as a constant: dL/dh = 0, dL/dg
    unchanged.  Returns (dh or None when h is None, demb [V, d_out - d_in]).
    """
    g = _real(emb)[ids]
    dout = _real(dout)
    d_in = 0 if h is None else h.shape[1]
    du, dg = dout[:, :d_in], dout[:, d_in:]
    demb = np.zeros_like(_real(emb))
    if mode != JUNCTION_ZERO_FILL:
        np.add.at(demb, ids, dg)
    if h is None:
        return None, demb
    h = _real(h)
    if mode == JUNCTION_NO_RESCALE:
        return (np.zeros_like(h) if stop_grad else du.copy()), demb
    a = np.linalg.norm(h, axis=1)
    b = np.linalg.norm(g, axis=1)
    live = (a > 0) & (b > 0)
    hd = np.sum(h * du, axis=1)
    sa = np.where(live, a, 1.0)
    sb = np.where(live, b, 1.0)
    dh = np.where(live, b / sa, 0.0)[:, None] * (du - h * (hd / sa ** 2)[:, None])
    if stop_grad:
        dh = np.zeros_like(h)
    c = np.where(live, hd / sa, 0.0)
    np.add.at(demb, ids, (c / sb)[:, None] * g)
    return dh, demb


# ---------------------------------------------------------------------------
# Heads
# ---------------------------------------------------------------------------
def heads(hs: Sequence[np.ndarray], ws: Sequence[np.ndarray]) -> List[np.ndarray]:
    """Per-exit linear LM heads: l_m = h_m W^m^T.

    Copyedit of Sec. 2 "Modeling": sub-model m is blocks 1..m followed by its
    own head W^m in R^{V x D_m}; the heads are not nested.  Reading: no bias,
    no final norm inside the op; logits are token-major [N, V].
    """
    return [_real(h) @ _real(w).T for h, w in zip(hs, ws)]


def head_backward(g: np.ndarray, h: np.ndarray, w: np.ndarray):
    """Backward of one linear head l = h W^T (the head of `heads`): with
    G = dL/dl, the chain rule gives dL/dh = G W and dL/dW = G^T h.

    Copyedit of Sec. 2 "Modeling" for the head; G is what `matryoshka_grad`
    returns for that exit (the teacher's under stop-gradient).  Returns
    (dh [N, D], dw [V, D]).
    """
    gr = _real(g)
    return gr @ _real(w), gr.T @ _real(h)


# ---------------------------------------------------------------------------
# Softmax pieces
# ---------------------------------------------------------------------------
def logsumexp(l: np.ndarray) -> np.ndarray:
    """log sum_v exp(l_v) over the last axis, two passes with the max shift."""
    l = _real(l)
    mx = np.max(l, axis=-1, keepdims=True)
    return (mx + np.log(np.sum(np.exp(l - mx), axis=-1, keepdims=True)))[..., 0]


def softmax(l: np.ndarray) -> np.ndarray:
    l = _real(l)
    return np.exp(l - logsumexp(l)[..., None])


# ---------------------------------------------------------------------------
# Loss and gradients
# ---------------------------------------------------------------------------
# Distillation divergences D(p, q) between the teacher p = softmax(l_M) and a
# student q = softmax(l_m).  DIV_FORWARD is the method's cross-entropy to the
# teacher (summary's distillation paragraph; follow-up 4's 0.3 term); the
# others are the swaps follow-up 4 of "Is nesting the cheapest way to build a
# model suite?" proposes: reverse KL, Jensen-Shannon, and an acceptance loss,
# read as the total-variation distance 1 - beta = 1 - sum_v min(p_v, q_v)
# (beta is the acceptance probability the same follow-up defines).
DIV_FORWARD, DIV_REVERSE_KL, DIV_JS, DIV_TV = 0, 1, 2, 3


def _xlogy(x, y):
    """x log y with 0 log 0 = 0."""
    return np.where(x > 0, x * np.log(np.where(x > 0, y, 1.0)), 0.0)


def divergence(p: np.ndarray, q: np.ndarray, kind: int) -> np.ndarray:
    """D(p, q) per row (last axis = vocabulary), p the teacher, q the student.
        DIV_FORWARD:    -sum p log q
        DIV_REVERSE_KL: sum q (log q - log p)
        DIV_JS:         (KL(p || m) + KL(q || m)) / 2,  m = (p + q) / 2
        DIV_TV:         sum |p - q| / 2  =  1 - sum min(p, q)
    """
    p, q = _real(p), _real(q)
    if kind == DIV_FORWARD:
        return -np.sum(_xlogy(p, q), axis=-1)
    if kind == DIV_REVERSE_KL:
        return np.sum(_xlogy(q, q) - _xlogy(q, p), axis=-1)
    if kind == DIV_JS:
        m = 0.5 * (p + q)
        return 0.5 * np.sum(_xlogy(p, p) - _xlogy(p, m) + _xlogy(q, q) - _xlogy(q, m), axis=-1)
    if kind == DIV_TV:
        return 0.5 * np.sum(np.abs(p - q), axis=-1)
    raise ValueError(kind)


def divergence_grad(p: np.ndarray, q: np.ndarray, kind: int) -> np.ndarray:
    """dD/dl for q = softmax(l), p held fixed (the teacher under stop-gradient).
    With r_v = dD/dq_v, the softmax's chain rule gives q_v (r_v - sum_u q_u r_u):
        DIV_FORWARD:    r = -p / q               ->  q - p
        DIV_REVERSE_KL: r = log q - log p + 1    ->  q (log q - log p - D)
        DIV_JS:         r = log(q / m) / 2
        DIV_TV:         r = sign(q - p) / 2      (0 where q = p)
    """
    p, q = _real(p), _real(q)
    if kind == DIV_FORWARD:
        return q - p
    if kind == DIV_REVERSE_KL:
        r = np.log(q) - np.log(p)
    elif kind == DIV_JS:
        r = 0.5 * (np.log(q) - np.log(0.5 * (p + q)))
    elif kind == DIV_TV:
        r = 0.5 * np.sign(q - p)
    else:
        raise ValueError(kind)
    return q * (r - np.sum(q * r, axis=-1, keepdims=True))


def matryoshka_loss(logits: Sequence[np.ndarray], labels: np.ndarray, alpha: float,
                    exit_weights: Optional[Sequence[float]] = None,
                    div: int = DIV_FORWARD) -> Dict:
    """Per-exit next-token cross-entropy plus online distillation.

    "Matryoshka Language Model Suites", distillation paragraph: the largest
    exit's softmax is the teacher and every smaller exit gets a token-level
    cross-entropy to it, weighted alpha_d = 0.3 and mixed with its own LM
    loss (follow-up 4 of "Is nesting the cheapest way ...": 0.7 next-token
    plus 0.3 cross-entropy to the largest model).  Main-visual explainer,
    panel (b): distillation goes only into the smaller exits.  Limitations
    paragraph: per-sub-model losses are summed with equal weight, and
    reweighting them is the fix a 200M sweep points to (exit_weights lambda,
    default all 1).

        CE_m   = LSE(l_m) - l_m[y]
        Dist_m = D(p, softmax(l_m)),  p = softmax(l_M)          (m < M)
                 (DIV_FORWARD: -sum_v p_v log softmax(l_m)_v = LSE(l_m) - sum_v p_v l_m,v)
        L_m    = (1 - alpha) CE_m + alpha Dist_m               (m < M)
        L_M    = CE_M,          total = sum_m lambda_m L_m

    Returns per-token arrays ce, dist (0 for the teacher), loss [M, N],
    total [N], and their means over tokens.
    """
    M = len(logits)
    y = np.asarray(labels, dtype=np.int64)
    n = y.shape[0]
    lam = np.ones(M) if exit_weights is None else _real(exit_weights)
    rows = np.arange(n)
    ls = [_real(l) for l in logits]
    lse = np.stack([logsumexp(l) for l in ls])                   # [M, N]
    ce = np.stack([lse[m] - ls[m][rows, y] for m in range(M)])   # [M, N]
    p = np.exp(ls[-1] - lse[-1][:, None])
    dist = np.zeros((M, n))
    for m in range(M - 1):
        if div == DIV_FORWARD:
            dist[m] = lse[m] - np.sum(p * ls[m], axis=1)
        else:
            dist[m] = divergence(p, np.exp(ls[m] - lse[m][:, None]), div)
    loss = np.empty((M, n))
    loss[: M - 1] = (1.0 - alpha) * ce[: M - 1] + alpha * dist[: M - 1]
    loss[M - 1] = ce[M - 1]
    total = np.sum(lam[:, None] * loss, axis=0)
    return {
        "lse": lse, "ce": ce, "dist": dist, "loss": loss, "total": total,
        "mean_ce": ce.mean(axis=1), "mean_dist": dist.mean(axis=1),
        "mean_loss": loss.mean(axis=1), "mean_total": float(total.mean()) if n else 0.0,
    }


def matryoshka_grad(logits: Sequence[np.ndarray], labels: np.ndarray, alpha: float,
                    grad_scale: float = 1.0, exit_weights: Optional[Sequence[float]] = None,
                    div: int = DIV_FORWARD) -> List[np.ndarray]:
    """d(grad_scale * sum_t total_t) / d l_m for every exit.

    The teacher's distribution enters the smaller exits' losses under
    stop-gradient, so exit M's gradient is that of CE_M alone:

        g_m = grad_scale lambda_m ((1 - alpha)(q_m - onehot(y)) + alpha dD/dl_m)   (m < M)
        g_M = grad_scale lambda_M (p - onehot(y))
    (DIV_FORWARD: dD/dl_m = q_m - p, so g_m = q_m - (1 - alpha) onehot(y) - alpha p.)
    """
    M = len(logits)
    y = np.asarray(labels, dtype=np.int64)
    lam = np.ones(M) if exit_weights is None else _real(exit_weights)
    rows = np.arange(y.shape[0])
    p = softmax(logits[-1])
    out = []
    for m in range(M):
        if m == M - 1:
            g = p.copy()
            g[rows, y] -= 1.0
        elif div == DIV_FORWARD:
            g = softmax(logits[m]) - alpha * p
            g[rows, y] -= 1.0 - alpha
        else:
            q = softmax(logits[m])
            g = (1.0 - alpha) * q + alpha * divergence_grad(p, q, div)
            g[rows, y] -= 1.0 - alpha
        out.append(grad_scale * lam[m] * g)
    return out


# ---------------------------------------------------------------------------
# Greedy speculative verification
# ---------------------------------------------------------------------------
def argmax_lowest(l: np.ndarray) -> np.ndarray:
    """Greedy token: index of the largest logit, the lowest index on ties."""
    l = _real(l)
    mx = np.max(l, axis=-1, keepdims=True)
    idx = np.arange(l.shape[-1])
    return np.min(np.where(l == mx, idx, l.shape[-1]), axis=-1).astype(np.int64)


def accept_prefix(draft: np.ndarray, verify: np.ndarray, draft_len: int) -> np.ndarray:
    """Accepted draft length per sequence under greedy verification.

    "Matryoshka Language Model Suites", speculative-decoding paragraphs: exit 1
    drafts and exit M verifies, draft length 6, greedy decoding.  Reading:
    in one verify pass over P = draft_len + 1 positions, draft token i is
    accepted while exit 1's greedy token equals exit M's greedy token at every
    position up to i; the count is the number of leading matches among the
    first draft_len positions.  draft, verify: int [B, P].
    """
    d = np.asarray(draft)
    v = np.asarray(verify)
    B = d.shape[0]
    out = np.zeros(B, dtype=np.int64)
    for b in range(B):
        k = 0
        while k < draft_len and d[b, k] == v[b, k]:
            k += 1
        out[b] = k
    return out


def nucleus(l: np.ndarray, temperature: float = 1.0, top_p: float = 1.0) -> np.ndarray:
    """Sampling distribution of one exit at one position (last axis = vocabulary).

    softmax(l / temperature), restricted to the nucleus and renormalised: the
    most probable entries whose probabilities reach top_p (the pages report
    nucleus sampling for speculative decoding without its settings, so both
    are parameters).  Reading for ties: every entry whose probability equals
    that of the last entry needed is kept too, so the set does not depend on
    an ordering of equal values.  top_p >= 1 keeps everything.
    """
    p = softmax(_real(l) / temperature)
    if top_p >= 1.0:
        return p
    flat = p.reshape(-1, p.shape[-1])
    out = np.empty_like(flat)
    for i, row in enumerate(flat):
        srt = np.sort(row)[::-1]
        k = min(int(np.searchsorted(np.cumsum(srt), top_p)), row.size - 1)
        keep = np.where(row >= srt[k], row, 0.0)
        out[i] = keep / keep.sum()
    return out.reshape(p.shape)


def sample_inverse_cdf(w: np.ndarray, u: float) -> int:
    """The entry v of weights w >= 0 (vocabulary order) where the running sum
    first exceeds u * sum(w); u in [0, 1).  Entries of weight 0 are never drawn."""
    w = _real(w)
    c = np.cumsum(w)
    v = int(np.searchsorted(c, u * c[-1], side="right"))
    nz = np.nonzero(w > 0)[0]
    return int(min(v, nz[-1]))


def speculative_verify(draft_logits: np.ndarray, verify_logits: np.ndarray,
                       draft_tokens: np.ndarray, u_accept: np.ndarray, u_next: np.ndarray,
                       draft_len: int, temperature: float = 1.0, top_p: float = 1.0):
    """Speculative sampling with the draft exit's distribution p and the
    verifying exit's q at every position (follow-up 4 of the follow-ups page:
    a drafted token is accepted with probability beta = sum_v min(p_v, q_v),
    after Leviathan et al.; the paper summary's speculative-decoding paragraph
    for the nested draft / verifier pair under nucleus sampling).

    Per sequence b, positions i < draft_len hold drafted tokens x_i:
      beta[b, i] = sum_v min(p_v, q_v)                      (p, q = nucleus(...))
      x_i is accepted iff u_accept[b, i] * p(x_i) < q(x_i)  (probability min(1, q/p))
      accepted[b] = number of leading accepted tokens
      next[b]: after the first rejection at k, a draw from max(0, q_k - p_k)
               (from q_k if that is all zero); if all are accepted, a draw from
               q at position draft_len; draws by sample_inverse_cdf(., u_next[b]).
    draft_logits, verify_logits: [B, P, V] with P >= draft_len + 1.
    Returns (beta [B, draft_len], accepted [B], next [B]).
    """
    dl = _real(draft_logits)
    vl = _real(verify_logits)
    B = dl.shape[0]
    beta = np.zeros((B, draft_len))
    acc = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    for b in range(B):
        p = nucleus(dl[b, :draft_len + 1], temperature, top_p)
        q = nucleus(vl[b, :draft_len + 1], temperature, top_p)
        beta[b] = np.minimum(p[:draft_len], q[:draft_len]).sum(axis=1)
        k = 0
        while k < draft_len:
            x = int(draft_tokens[b, k])
            if u_accept[b, k] * p[k, x] < q[k, x]:
                k += 1
            else:
                break
        acc[b] = k
        if k < draft_len:
            r = np.maximum(q[k] - p[k], 0.0)
            w = r if r.sum() > 0 else q[k]
        else:
            w = q[draft_len]
        nxt[b] = sample_inverse_cdf(w, float(u_next[b]))
    return beta, acc, nxt


# ---------------------------------------------------------------------------
# Chunked evaluation on a subset of tokens
# ---------------------------------------------------------------------------
def forward_tokens(hs: Sequence[np.ndarray], ws: Sequence[np.ndarray], labels: np.ndarray,
                   alpha: float, grad_scale: float = 1.0, rows=None, chunk: int = 1024,
                   want_grad: bool = True, exits: Optional[Sequence[int]] = None,
                   exit_weights: Optional[Sequence[float]] = None, div: int = DIV_FORWARD):
    """Heads, losses and gradients for the tokens ``rows`` (default: all),
    ``chunk`` tokens at a time.  Returns (loss dict over the rows, list of
    per-exit gradient arrays [len(rows), V] or None)."""
    n = hs[0].shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    sel = list(range(len(hs))) if exits is None else list(exits)
    parts = []
    grads = [[] for _ in sel] if want_grad else None
    for s in range(0, len(rows), chunk):
        r = rows[s:s + chunk]
        lg = heads([hs[m][r] for m in sel], [ws[m] for m in sel])
        parts.append(matryoshka_loss(lg, labels[r], alpha, exit_weights, div))
        if want_grad:
            for j, g in enumerate(matryoshka_grad(lg, labels[r], alpha, grad_scale, exit_weights,
                                                  div)):
                grads[j].append(g)
    keys = ("lse", "ce", "dist", "loss")
    res = {k: np.concatenate([p[k] for p in parts], axis=1) for k in keys}
    res["total"] = np.concatenate([p["total"] for p in parts])
    for k in ("ce", "dist", "loss"):
        res["mean_" + k] = res[k].mean(axis=1)
    res["mean_total"] = float(res["total"].mean())
    if want_grad:
        grads = [np.concatenate(g, axis=0) for g in grads]
    return res, grads


def loss_backward(hs: Sequence[np.ndarray], ws: Sequence[np.ndarray], labels: np.ndarray,
                  alpha: float, grad_scale: float = 1.0,
                  exit_weights: Optional[Sequence[float]] = None, chunk: int = 1024):
    """The loss and the backward of every exit head in one pass over the
    tokens, the logit gradients never kept beyond a chunk of ``chunk`` tokens.

    For each chunk: the heads (``heads``), the losses (``matryoshka_loss``),
    G_m = ``matryoshka_grad`` (teacher under stop-gradient; "Matryoshka
    Language Model Suites", distillation paragraph), then by the chain rule
    through l_m = h_m W^m^T (``head_backward``) the chunk's rows of
    dh_m = G_m W^m and its share of dW^m = sum over tokens of G_m[t]^T h_m[t].
    Returns (loss dict as ``forward_tokens``, [dh_m [N, D_m]], [dW^m [V, D_m]]).
    """
    n = hs[0].shape[0]
    res, _ = forward_tokens(hs, ws, labels, alpha, grad_scale, chunk=chunk, want_grad=False,
                            exit_weights=exit_weights)
    dhs = [np.zeros((n, h.shape[1]), dtype=_DTYPE) for h in hs]
    dws = [np.zeros(np.shape(w), dtype=_DTYPE) for w in ws]
    for s in range(0, n, chunk):
        r = slice(s, min(n, s + chunk))
        lg = heads([h[r] for h in hs], ws)
        for m, g in enumerate(matryoshka_grad(lg, labels[r], alpha, grad_scale, exit_weights)):
            dh, dw = head_backward(g, hs[m][r], ws[m])
            dhs[m][r] = dh
            dws[m] += dw
    return res, dhs, dws
