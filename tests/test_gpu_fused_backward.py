"""The loss and every exit head's backward with the logit gradients G formed
inside the dh and dW GEMMs (nel_matryoshka_loss_backward_packed), checked
(a) against the stored-gradient path (nel_matryoshka_loss_packed then
nel_heads_backward): dh bit for bit (one GEMM loop, the same gradients), dW
within the reordering bound 2 gamma_n |G~|^T |h| (the same bf16 products
summed in fp32 by two different loops), and (b) against the oracle's
composition oracle.loss_backward.

Bars for (b), per element, by the triangle inequality through the GPU's own
stored gradients G~ (which the loss tests hold to the oracle's G within the
dlogits bar):
    |dh - dh_ref| <= |G~ - G| |W| + gamma_K |G~| |W| + 2^-8 |dh|   (bf16 output)
    |dW - dW_ref| <= |G~ - G|^T |h| + gamma_n |G~|^T |h|
with gamma_K = 2 K 2^-24 (fp32 accumulation in any order; bf16 products are
exact in fp32).  The losses are held to rel 1e-3 as everywhere."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DevSuite, GRAD_TOL, assert_grad_close, assert_loss_close, log, to_np

pytestmark = pytest.mark.gpu


def gamma(K):
    return 2.0 * K * 2.0 ** -24


def run_both(nel, ds, alpha, gs, lam, want_dh=True, want_dw=True):
    import torch
    pw = [nel.pack_weights(w) for w in ds.w]
    mean_f, tok_f, dh_f, dw_f = nel.loss_backward_packed(
        ds.h, ds.w, pw, ds.labels, alpha_d=alpha, grad_scale=gs, exit_weights=lam,
        want_dh=want_dh, want_dw=want_dw)
    mean_u, tok_u, dl = nel.matryoshka_loss_packed(ds.h, pw, ds.labels, alpha_d=alpha,
                                                   grad_scale=gs, exit_weights=lam)
    dh_u, dw_u = nel.heads_backward(dl, ds.h, ds.w, want_dh=want_dh, want_dw=want_dw)
    torch.cuda.synchronize()
    return (mean_f, tok_f, dh_f, dw_f), (mean_u, tok_u, dl, dh_u, dw_u)


def assert_matches_stored(nel, ds, fused, unfused):
    """dh bit for bit; dW within 2 gamma_n |G~|^T |h| of the stored-gradient
    dW (the bound's product runs in fp32 on the GPU: its own rounding is far
    below the factor 2 it carries)."""
    import torch
    _, _, dh_f, dw_f = fused
    _, _, dl, dh_u, dw_u = unfused
    if dh_f is None:
        assert dh_u is None
    else:
        for m, (a, b) in enumerate(zip(dh_f, dh_u)):
            same = torch.equal(a.view(torch.int16), b.view(torch.int16))
            assert same, f"dh exit {m}: fused differs from the stored-gradient path"
    if dw_f is None:
        assert dw_u is None
        return
    for m, (a, b) in enumerate(zip(dw_f, dw_u)):
        n = dl[m].shape[0]
        bound = 2.0 * gamma(n) * (dl[m].float().abs().t().contiguous() @ ds.h[m].float().abs())
        err = (a - b).abs()
        assert bool(torch.all(err <= bound + 1e-30)), (
            f"dW exit {m}: fused differs from the stored-gradient dW by "
            f"{float((err / (bound + 1e-30)).max()):.3g} x the reordering bound")
        assert bool(torch.isfinite(a).all()) == bool(torch.isfinite(b).all())


CASES = [
    # name, widths (multiples of 64), V, batch, seq, alpha, grad_scale, exit weights, seed
    ("3exit-ragged", (64, 128, 192), 512, 3, 67, 0.3, 1.0, None, 71),
    ("weighted-scaled", (64, 192), 1024, 2, 100, 0.7, 0.25, (0.5, 2.0), 72),
    ("one-exit", (128,), 256, 1, 65, 0.3, 1.0, None, 73),
    ("vocab-64", (64, 128), 64, 1, 65, 1.0, 1.0, None, 74),
    ("alpha-0", (64, 128, 256), 768, 2, 64, 0.0, 1.0, (1.0, 0.0, 1.5), 75),
    # a negative upstream gradient: every exit's sign flips, one weight is 0
    ("negative-scale", (64, 128, 192), 512, 2, 70, 0.3, -0.75, (1.0, 0.0, 2.0), 76),
]


@pytest.mark.parametrize("name,widths,V,B,S,alpha,gs,lam,seed", CASES, ids=[c[0] for c in CASES])
def test_fused_backward_small(nel, name, widths, V, B, S, alpha, gs, lam, seed):
    s = synth.make_suite(widths, V, B, S, seed=seed)
    log(f"[fused-bwd] {name}: n={s.n_tokens} V={V} widths={widths} alpha={alpha} gs={gs} lam={lam}")
    ds = DevSuite(s)
    fused, unfused = run_both(nel, ds, alpha, gs, lam)
    assert_matches_stored(nel, ds, fused, unfused)
    mean_f, tok_f, dh_f, dw_f = fused
    dl = unfused[2]
    ref, dh_ref, dw_ref = oracle.loss_backward(s.h, s.w, s.labels, alpha, grad_scale=gs,
                                               exit_weights=lam)
    tok = to_np(tok_f)
    assert_loss_close(tok[:, 0], ref["ce"], 1e-3, "CE")
    assert_loss_close(tok[:, 1], ref["dist"], 1e-3, "Dist")
    assert_loss_close(tok[:, 2], ref["loss"], 1e-3, "L")
    want_mean = np.concatenate([ref["mean_ce"], ref["mean_dist"], ref["mean_loss"],
                                [ref["mean_total"]]])
    assert_loss_close(to_np(mean_f), want_mean, 1e-3, "means")
    g_ref = oracle.matryoshka_grad(oracle.heads(s.h, s.w), s.labels, alpha, gs, lam)
    n = s.n_tokens
    for m in range(s.n_exits):
        gt = to_np(dl[m])   # the stored gradients, which the fused GEMMs form bit for bit
        assert_grad_close(gt, g_ref[m], GRAD_TOL["bf16"] * max(1.0, abs(gs)), f"G exit {m}")
        dG = np.abs(gt - g_ref[m])
        w, h = s.w[m].astype(np.float64), s.h[m].astype(np.float64)
        got = to_np(dh_f[m])
        tol = dG @ np.abs(w) + gamma(V) * (np.abs(gt) @ np.abs(w))
        tol = tol + 2.0 ** -8 * (np.abs(dh_ref[m]) + tol) + 1e-30
        err = np.abs(got - dh_ref[m])
        assert np.all(err <= tol), f"dh exit {m}: worst {np.max(err / tol):.3g} x bar"
        got = to_np(dw_f[m])
        tol = dG.T @ np.abs(h) + gamma(n) * (np.abs(gt).T @ np.abs(h)) + 1e-30
        err = np.abs(got - dw_ref[m])
        assert np.all(err <= tol), f"dW exit {m}: worst {np.max(err / tol):.3g} x bar"
        ref_norm = np.linalg.norm(dh_ref[m])
        if ref_norm > 0:
            log(f"  exit {m}: |dh - ref| / |ref| = "
                f"{np.linalg.norm(to_np(dh_f[m]) - dh_ref[m]) / ref_norm:.3g}")


def test_fused_backward_single_outputs(nel):
    s = synth.make_suite((64, 128), 512, 2, 70, seed=76)
    ds = DevSuite(s)
    for want_dh, want_dw in ((True, False), (False, True)):
        fused, unfused = run_both(nel, ds, 0.3, 1.0, None, want_dh=want_dh, want_dw=want_dw)
        assert (fused[2] is None) != want_dh and (fused[3] is None) != want_dw
        assert_matches_stored(nel, ds, fused, unfused)


def test_fused_backward_bad_label_is_nan_and_flagged(nel):
    import torch
    s = synth.make_suite((64, 128), 256, 1, 40, seed=77)
    ds = DevSuite(s)
    ds.labels[5] = 256          # outside the vocabulary
    ws = torch.zeros(nel.loss_backward_workspace_size(s.n_tokens, 256, [64, 128]),
                     dtype=torch.uint8, device="cuda:0")
    pw = [nel.pack_weights(w) for w in ds.w]
    mean, tok, dhs, dws = nel.loss_backward_packed(ds.h, ds.w, pw, ds.labels, workspace=ws)
    torch.cuda.synchronize()
    assert nel.read_flags(ws) & nel.FLAG_BAD_LABEL
    for m in range(2):
        dh = to_np(dhs[m])
        assert np.all(np.isnan(dh[5])), "the bad token's dh row is NaN"
        assert np.all(np.isfinite(np.delete(dh, 5, axis=0))), "other rows stay finite"
        assert np.all(np.isnan(to_np(dws[m]))), "every dW entry sums the bad token's row"
        assert np.all(np.isnan(to_np(tok)[m, :, 5]))


def test_fused_backward_no_tokens(nel):
    import torch
    V, widths = 128, (64, 128)
    hs = [torch.empty(0, d, dtype=torch.bfloat16, device="cuda:0") for d in widths]
    ws = [torch.ones(V, d, dtype=torch.bfloat16, device="cuda:0") for d in widths]
    pw = [nel.pack_weights(w) for w in ws]
    labels = torch.empty(0, dtype=torch.int32, device="cuda:0")
    dws = [torch.full((V, d), 7.0, dtype=torch.float32, device="cuda:0") for d in widths]
    mean, tok, dhs, dws = nel.loss_backward_packed(hs, ws, pw, labels, dws=dws)
    torch.cuda.synchronize()
    for m in range(2):
        assert dhs[m].shape == (0, widths[m])
        assert float(dws[m].abs().max()) == 0.0


def test_fused_backward_benchmark_shape(nel):
    """500M-1.5B-3B-3exit (16,384 tokens, V = 32,768): dh bit-identical to
    the stored-gradient path and dW within its reordering bound, on every
    entry, and 24 sampled tokens' dh rows against the oracle by the bar above."""
    import torch
    s = synth.make_workload(2)
    log(f"[fused-bwd] workload 2: n={s.n_tokens} V={s.vocab} widths={s.widths}")
    ds = DevSuite(s)
    fused, unfused = run_both(nel, ds, 0.3, 1.0, None)
    assert_matches_stored(nel, ds, fused, unfused)
    rows = np.unique(np.concatenate([[0, 1, s.n_tokens - 1],
                                     np.random.default_rng(78).choice(s.n_tokens, 21, replace=False)]))
    lg = oracle.heads([h[rows] for h in s.h], s.w)
    g_ref = oracle.matryoshka_grad(lg, s.labels[rows], 0.3)
    idx = torch.from_numpy(rows).to("cuda:0")
    for m in range(s.n_exits):
        w = s.w[m].astype(np.float64)
        dh_ref = g_ref[m] @ w
        gt = to_np(unfused[2][m].index_select(0, idx))
        got = to_np(fused[2][m].index_select(0, idx))
        dG = np.abs(gt - g_ref[m])
        tol = dG @ np.abs(w) + gamma(s.vocab) * (np.abs(gt) @ np.abs(w))
        tol = tol + 2.0 ** -8 * (np.abs(dh_ref) + tol) + 1e-30
        err = np.abs(got - dh_ref)
        assert np.all(err <= tol), f"dh exit {m}: worst {np.max(err / tol):.3g} x bar"
        log(f"  exit {m}: sampled |dh - ref| / |ref| = "
            f"{np.linalg.norm(got - dh_ref) / np.linalg.norm(dh_ref):.3g}")
    del fused, unfused
    torch.cuda.empty_cache()
