"""Per-exit loss weights and the other distillation divergences (reverse KL,
Jensen-Shannon, total variation) through nel_matryoshka_loss and
nel_matryoshka_loss_packed, against the oracle.

Bars.  CE as for the main path.  The other divergences are summed from the
stored tile-shifted logits s = l - m_tile.  In fp32 these are exact to fp32
rounding: D to 1e-4 max(1, |ref|).  In bf16 each s is rounded with relative
error 2^-9, and |s| <= l_max - l.  The bar is twice that rounding propagated
to first order through D, computed from the oracle's values:
    reverse KL  sum_v q |lq - lp + 1| e_q + q e_p
    JS          sum_v (q |lq - lm| e_q + p |lp - lm| e_p) / 2
    TV          sum_v (q e_q + p e_p) / 2
with lq, lp, lm = log q, log p, log((p + q) / 2) and e = 2^-9 (l_max - l),
plus 1e-5 for the fp32 sums.  L_m takes alpha times that on top of the CE
bar.  Gradients use the main path's bars: 2e-2 max-abs for bf16, 1e-4 for
fp32.  For TV, an entry where q - p is within its rounding has no decided
sign: there the gradient must match the one for some sign (+, - or 0) of
that entry, with the oracle's row constant."""
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
    """Error of log-probabilities read back from stored s: per entry."""
    if dtype == "f32":
        return 2.0 ** -22 * (np.abs(l) + np.abs(_lse(l)))
    return 2.0 ** -9 * (l.max(axis=1, keepdims=True) - l) + 2.0 ** -22 * np.abs(_lse(l))


def div_bound(l_s, l_t, div, dtype):
    lq, lp = l_s - _lse(l_s), l_t - _lse(l_t)
    q, p = np.exp(lq), np.exp(lp)
    eq, ep = rounding(l_s, dtype), rounding(l_t, dtype)
    if div == oracle.DIV_REVERSE_KL:
        b = np.sum(q * np.abs(lq - lp + 1) * eq + q * ep, axis=1)
    elif div == oracle.DIV_JS:
        lm = np.logaddexp(lq, lp) - np.log(2.0)
        b = 0.5 * np.sum(q * np.abs(lq - lm) * eq + p * np.abs(lp - lm) * ep, axis=1)
    else:
        b = 0.5 * np.sum(q * eq + p * ep, axis=1)
    return 2.0 * b + 1e-5


def tv_undecided(l_s, l_t, dtype):
    q, p = np.exp(l_s - _lse(l_s)), np.exp(l_t - _lse(l_t))
    return np.abs(q - p) <= 2.0 * (q * rounding(l_s, dtype) + p * rounding(l_t, dtype)) + 1e-12


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


def check(nel, s, alpha, div, lam, packed=False, rows=None):
    """Every token (or the sampled rows) of every exit against the oracle."""
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
    for m in range(M - 1):
        if s.dtype == "f32":
            bnd = 1e-4 * np.maximum(1.0, np.abs(ref["dist"][m]))
        else:
            bnd = div_bound(lg[m], lg[-1], div, s.dtype)
        err = np.abs(tok[m, 1, r] - ref["dist"][m])
        assert np.all(err <= bnd), f"Dist exit {m}: worst {np.max(err / bnd):.3g} x bar"
        lbar = tol * np.maximum(1.0, np.abs(ref["loss"][m])) + alpha * bnd
        assert np.all(np.abs(tok[m, 2, r] - ref["loss"][m]) <= lbar), f"L exit {m}"
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
        assert_grad_close(g, grads[m], GRAD_TOL[s.dtype], f"dlogits exit {m}")
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


def test_divergence_benchmark_shape_sampled(nel):
    """The benchmark workload (16,384 tokens, V = 32,768, widths 1024 / 2304 /
    4352) on the packed path with Jensen-Shannon: sampled full rows."""
    s = synth.make_workload(2)
    rows = sample_rows(s.n_tokens, 12, 105)
    log(f"[div] benchmark shape n={s.n_tokens} rows={len(rows)}")
    check(nel, s, 0.3, oracle.DIV_JS, LAM, packed=True, rows=rows)
