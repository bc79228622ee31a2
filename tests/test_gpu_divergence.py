"""Per-exit loss weights and the other distillation divergences (reverse KL,
Jensen-Shannon, total variation) through nel_matryoshka_loss and
nel_matryoshka_loss_packed, against the oracle.

Bars.  Losses as for the main path: every per-token CE, Dist and L within
1e-3 max(1, |ref|) for bf16 inputs and 1e-4 for fp32.  The other divergences
are summed from the stored tile-shifted logits s = l - m_tile, kept in fp16
for bf16 inputs (relative rounding 2^-11, |s| <= l_max - l) and in fp32 for
fp32 inputs.  Gradients use the main path's bars: 2e-2 max-abs for bf16,
1e-4 for fp32.  For TV, an entry where q - p is within the rounding of the
stored s has no decided sign: there the gradient must match the one for some
sign (+, - or 0) of that entry, with the oracle's row constant."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DevSuite, GRAD_TOL, LOSS_TOL, assert_grad_close, assert_loss_close, log,
                      sample_rows, to_np)

pytestmark = pytest.mark.gpu

DIVS = [oracle.DIV_REVERSE_KL, oracle.DIV_JS, oracle.DIV_TV]
LAM = [0.5, 2.0, 1.25]


def _lse(l):
    mx = l.max(axis=1, keepdims=True)
    return mx + np.log(np.exp(l - mx).sum(axis=1, keepdims=True))


def rounding(l, dtype):
    """Error of log-probabilities read back from the stored s: per entry."""
    if dtype == "f32":
        return 2.0 ** -22 * (np.abs(l) + np.abs(_lse(l)))
    return 2.0 ** -11 * (l.max(axis=1, keepdims=True) - l) + 2.0 ** -22 * np.abs(_lse(l))


def tv_undecided(l_s, l_t, dtype):
    q, p = np.exp(l_s - _lse(l_s)), np.exp(l_t - _lse(l_t))
    return np.abs(q - p) <= 2.0 * (q * rounding(l_s, dtype) + p * rounding(l_t, dtype)) + 1e-12


def rkl_grad_bar(s, r, m, alpha, lam):
    """First-order bound of the reverse-KL student gradient's error, for logits
    so spread that the gradient alpha lam q (log q - log p - K) is ill
    conditioned.  Per entry, the error of a log-probability read back by the
    kernel is e = (stored-s rounding) + 2 x (the row's fp32 accumulation bound
    of the logits, which also bounds the log-sum-exp's).  Then
        dq = q e_q,  dr = e_q + e_p,  dK = sum_u q_u (e_q,u |r_u| + dr_u),
        dg = lam ((1 - alpha) dq + alpha (dq |r - K| + q (dr + dK))),
    and the bar is 2 dg plus the main path's bar and the output's rounding."""
    from gpu_util import head_error_bound_ordered
    M = s.n_exits
    ls = oracle.heads([s.h[m][r]], [s.w[m]])[0]
    lt = oracle.heads([s.h[M - 1][r]], [s.w[M - 1]])[0]
    es = rounding(ls, s.dtype) + 2 * head_error_bound_ordered(s.h[m][r], s.w[m]).max(1, keepdims=True)
    et = rounding(lt, s.dtype) + 2 * head_error_bound_ordered(s.h[M - 1][r], s.w[M - 1]).max(1, keepdims=True)
    lq, lp = ls - _lse(ls), lt - _lse(lt)
    q = np.exp(lq)
    rr = lq - lp
    K = np.sum(q * rr, axis=1, keepdims=True)
    dq = q * es
    dr = es + et
    dK = np.sum(q * (es * np.abs(rr) + dr), axis=1, keepdims=True)
    dg = lam[m] * ((1 - alpha) * dq + alpha * (dq * np.abs(rr - K) + q * (dr + dK)))
    g = lam[m] * ((1 - alpha) * q + alpha * q * (rr - K))
    out_round = np.abs(g) * (2.0 ** -8 if s.dtype == "bf16" else 2.0 ** -23)
    return 2 * dg + GRAD_TOL[s.dtype] + out_round


def run(nel, ds, alpha, div, lam, packed):
    import torch
    if packed:
        pw = [nel.pack_weights(w) for w in ds.w]
        mean, tok, dl = nel.matryoshka_loss_packed(ds.h, pw, ds.labels, alpha_d=alpha,
                                                   exit_weights=lam, divergence=div)
    else:
        mean, tok, dl = nel.matryoshka_loss(ds.h, ds.w, ds.labels, alpha_d=alpha,
                                            exit_weights=lam, divergence=div)
    torch.cuda.synchronize()
    return to_np(mean), to_np(tok), dl


def check(nel, s, alpha, div, lam, packed=False, rows=None, conditioned=False):
    """Every token (or the sampled rows) of every exit against the oracle.
    conditioned: hold the reverse-KL student gradients to rkl_grad_bar."""
    import torch
    ds = DevSuite(s)
    mean, tok, dl = run(nel, ds, alpha, div, lam, packed)
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, alpha, rows=rows, exit_weights=lam,
                                       div=div)
    r = np.arange(s.n_tokens) if rows is None else rows
    M = s.n_exits
    tol = LOSS_TOL[s.dtype]
    assert_loss_close(tok[:, 0, r], ref["ce"], tol, "CE")
    lg = oracle.heads([s.h[m][r] for m in range(M)], s.w)
    undecided = 0
    worst = 0.0
    for m in range(M - 1):
        worst = max(worst, assert_loss_close(tok[m, 1, r], ref["dist"][m], tol, f"Dist exit {m}"))
        assert_loss_close(tok[m, 2, r], ref["loss"][m], tol, f"L exit {m}")
    assert_loss_close(tok[M - 1, 2, r], ref["loss"][M - 1], tol, "L teacher")
    if rows is None:
        want_total = float(np.mean(np.sum(np.asarray(lam)[:, None] * ref["loss"], axis=0)))
        assert abs(mean[3 * M] - want_total) <= 2e-3 * max(1.0, abs(want_total)), "total mean"
    for m in range(M):
        g = to_np(dl[m][torch.from_numpy(r).cuda()] if rows is not None else dl[m])
        if div == oracle.DIV_TV and m < M - 1:
            amb = tv_undecided(lg[m], lg[-1], s.dtype)
            undecided += int(amb.sum())
            # the gradient for each sign of an undecided entry: lambda alpha q (sigma - K)
            # moves by lambda alpha q per half unit of sigma
            q = np.exp(lg[m] - _lse(lg[m]))
            step = 0.5 * lam[m] * alpha * q
            sig = 0.5 * np.sign(q - np.exp(lg[-1] - _lse(lg[-1])))
            ok = np.zeros_like(amb)
            for alt in (-0.5, 0.0, 0.5):
                cand = grads[m] + 2.0 * step * (alt - sig)
                ok |= np.abs(g - cand) <= GRAD_TOL[s.dtype]
            assert np.all(ok[amb]), f"dlogits exit {m}: an undecided TV entry fits no sign"
            g = np.where(amb, grads[m], g)
        if conditioned and div == oracle.DIV_REVERSE_KL and m < M - 1:
            assert np.all(np.isfinite(g)), f"dlogits exit {m}: non-finite values"
            bar = rkl_grad_bar(s, r, m, alpha, lam)
            err = np.abs(g - grads[m])
            assert np.all(err <= bar), f"dlogits exit {m}: worst {np.max(err / bar):.3g} x bar"
            continue
        assert_grad_close(g, grads[m], GRAD_TOL[s.dtype], f"dlogits exit {m}")
    log(f"  worst scaled Dist error {worst:.2e} (bar {tol})")
    return undecided


@pytest.mark.parametrize("div", DIVS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_divergence_row_major(nel, div, dtype):
    s = synth.make_suite((64, 136, 200), 300, 2, 100, dtype=dtype, seed=101)
    und = check(nel, s, 0.3, div, LAM)
    log(f"[div] row-major {dtype} div={div}: ok, TV entries of undecided sign {und}")


@pytest.mark.parametrize("div", DIVS)
def test_divergence_packed(nel, div):
    s = synth.make_suite((64, 128, 192), 512, 3, 100, seed=102)   # ragged token tiles
    und = check(nel, s, 0.4, div, LAM, packed=True)
    log(f"[div] packed div={div}: ok, TV entries of undecided sign {und}")


def test_divergence_element_path(nel):
    """A vocabulary that is not a multiple of the 16-byte chunk (fp32: 4)."""
    s = synth.make_suite((13, 40), 301, 1, 77, dtype="f32", seed=103)
    check(nel, s, 0.5, oracle.DIV_JS, [1.0, 0.75])
    check(nel, s, 1.0, oracle.DIV_REVERSE_KL, [3.0, 0.5])


@pytest.mark.parametrize("packed", [False, True])
def test_exit_weights_forward_divergence(nel, packed):
    """The method's divergence with reweighted exits: gradients and the total scale."""
    s = synth.make_suite((64, 128, 192), 512, 2, 64, seed=104)
    check(nel, s, 0.3, oracle.DIV_FORWARD, [0.2, 1.0, 3.0], packed=packed)
    check(nel, s, 0.3, oracle.DIV_FORWARD, [1.0, 0.0, 1.0], packed=packed)   # a switched-off exit


@pytest.mark.parametrize("div", DIVS)
def test_divergence_benchmark_shape_sampled(nel, div):
    """The benchmark workload (16,384 tokens, V = 32,768, widths 1024 / 2304 /
    4352) on the packed path: sampled full rows of every exit."""
    s = synth.make_workload(2)
    rows = sample_rows(s.n_tokens, 12, 105 + div)
    log(f"[div] benchmark shape n={s.n_tokens} div={div} rows={len(rows)}")
    check(nel, s, 0.3, div, LAM, packed=True, rows=rows)


@pytest.mark.parametrize("packed,dtype", [(False, "f32"), (False, "bf16"), (True, "bf16")],
                         ids=["row-major-f32", "row-major-bf16", "packed-bf16"])
def test_divergences_with_underflowing_probabilities(nel, packed, dtype):
    """Block outputs scaled by 64, so the logits of a row span several hundred:
    most entries have log-probabilities far below -70 under both the teacher
    and the student, where p + q < 2^-100 and the Jensen-Shannon mixture's log
    takes its log-sum-exp form.  Every divergence stays finite and matches the
    oracle at the same bars, except the reverse-KL gradient: alpha lam q
    (log q - log p - K) carries |log q - log p| of several hundred here, which
    multiplies the fp32 logits' own rounding, so it is held to the first-order
    bar of rkl_grad_bar instead of a fixed one."""
    s = synth.make_suite((64, 128, 192), 512, 2, 64, dtype=dtype, seed=106)
    s.h = [synth.round_to_bf16(h * 64.0) if dtype == "bf16" else (h * 64.0).astype(np.float32)
           for h in s.h]
    l = oracle.heads(s.h, s.w)
    lp = [x - _lse(x) for x in l]
    frac = float(np.mean((lp[0] < -70) & (lp[-1] < -70)))
    log(f"[div] underflow case {dtype} packed={packed}: entries with both log-probs < -70: {frac:.2f}")
    assert frac > 0.5
    for div in DIVS:
        check(nel, s, 0.3, div, LAM, packed=packed, conditioned=True)
