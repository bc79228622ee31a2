"""Pins for the CPU oracle: brute force, closed forms, library special cases
and invariants, each chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign or index, a reversed distillation direction, a transposed
operand) fails at least one of them."""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch
import torch.nn.functional as F

import oracle
import synth


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------- LSE
@pytest.mark.parametrize("V", [1, 2, 3, 7, 16])
def test_lse_brute_force(V):
    r = rng(V)
    for scale, shift in [(1.0, 0.0), (10.0, 0.0), (3.0, 700.0), (3.0, -700.0)]:
        l = r.standard_normal((5, V)) * scale + shift
        got = oracle.logsumexp(l)
        for i in range(5):
            m = max(l[i])
            want = m + math.log(math.fsum(math.exp(x - m) for x in l[i]))
            assert got[i] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_lse_shift_invariance():
    l = rng(1).standard_normal((4, 33))
    np.testing.assert_allclose(oracle.logsumexp(l + 17.25), oracle.logsumexp(l) + 17.25, rtol=1e-14)


# --------------------------------------------------------------------- CE
def _torch_ce(l, y):
    return F.cross_entropy(torch.from_numpy(l), torch.from_numpy(y.astype(np.int64)),
                           reduction="none").numpy()


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_ce_is_library_cross_entropy_at_alpha_zero(M):
    r = rng(M)
    V, N = 37, 11
    ls = [r.standard_normal((N, V)) * 3 for _ in range(M)]
    y = r.integers(0, V, N)
    out = oracle.matryoshka_loss(ls, y, 0.0)
    for m in range(M):
        np.testing.assert_allclose(out["ce"][m], _torch_ce(ls[m], y), rtol=1e-12)
        np.testing.assert_allclose(out["loss"][m], _torch_ce(ls[m], y), rtol=1e-12)
    np.testing.assert_allclose(out["total"], sum(_torch_ce(l, y) for l in ls), rtol=1e-12)


def test_single_exit_is_plain_lm_loss_for_any_alpha():
    r = rng(5)
    l = r.standard_normal((9, 20)) * 2
    y = r.integers(0, 20, 9)
    for a in (0.0, 0.3, 1.0):
        out = oracle.matryoshka_loss([l], y, a)
        np.testing.assert_allclose(out["total"], _torch_ce(l, y), rtol=1e-12)
        assert np.all(out["dist"] == 0)


# --------------------------------------------------------------------- distillation
def test_distillation_equals_teacher_entropy_when_logits_equal():
    r = rng(7)
    N, V = 6, 50
    lt = r.standard_normal((N, V)) * 4
    y = r.integers(0, V, N)
    out = oracle.matryoshka_loss([lt.copy(), lt.copy(), lt], y, 0.3)
    p = scipy.special.softmax(lt, axis=1)
    H = scipy.stats.entropy(p, axis=1)
    np.testing.assert_allclose(out["dist"][0], H, rtol=1e-12)
    np.testing.assert_allclose(out["dist"][1], H, rtol=1e-12)


def test_distillation_is_entropy_plus_kl_teacher_to_student():
    """Dist_m = H(p) + KL(p || q_m): the teacher's distribution is the target."""
    r = rng(8)
    N, V = 8, 40
    ls = [r.standard_normal((N, V)) * s for s in (1.0, 2.0, 3.0)]
    y = r.integers(0, V, N)
    out = oracle.matryoshka_loss(ls, y, 0.3)
    p = scipy.special.softmax(ls[2], axis=1)
    H = scipy.stats.entropy(p, axis=1)
    for m in range(2):
        q = scipy.special.softmax(ls[m], axis=1)
        kl = scipy.special.rel_entr(p, q).sum(axis=1)
        np.testing.assert_allclose(out["dist"][m], H + kl, rtol=1e-11)
        assert np.all(out["dist"][m] >= H - 1e-12)       # Gibbs


def test_alpha_one_loss_is_distillation_and_mix_is_linear():
    r = rng(9)
    ls = [r.standard_normal((5, 30)) * 2 for _ in range(3)]
    y = r.integers(0, 30, 5)
    o1 = oracle.matryoshka_loss(ls, y, 1.0)
    np.testing.assert_allclose(o1["loss"][:2], o1["dist"][:2], rtol=1e-14)
    np.testing.assert_allclose(o1["loss"][2], o1["ce"][2], rtol=1e-14)
    o3 = oracle.matryoshka_loss(ls, y, 0.3)
    np.testing.assert_allclose(o3["loss"][:2], 0.7 * o3["ce"][:2] + 0.3 * o3["dist"][:2], rtol=1e-13)
    # the teacher's own loss never depends on alpha
    np.testing.assert_allclose(o1["loss"][2], o3["loss"][2], rtol=0)


# --------------------------------------------------------------------- gradients
@pytest.mark.parametrize("V", [2, 5, 16])
@pytest.mark.parametrize("alpha", [0.0, 0.3, 1.0])
def test_gradients_central_differences(V, alpha):
    r = rng(V + int(alpha * 10))
    M, N = 3, 4
    ls = [r.standard_normal((N, V)) * 2 for _ in range(M)]
    y = r.integers(0, V, N)
    gs = 0.5
    g = oracle.matryoshka_grad(ls, y, alpha, gs)
    eps = 1e-6
    for m in range(M):
        for t in range(N):
            for v in range(V):
                lp = [l.copy() for l in ls]
                lm = [l.copy() for l in ls]
                lp[m][t, v] += eps
                lm[m][t, v] -= eps
                if m < M - 1:
                    fp = oracle.matryoshka_loss(lp, y, alpha)["total"].sum()
                    fm = oracle.matryoshka_loss(lm, y, alpha)["total"].sum()
                else:   # teacher under stop-gradient: only its own CE
                    fp = oracle.matryoshka_loss(lp, y, alpha)["ce"][M - 1].sum()
                    fm = oracle.matryoshka_loss(lm, y, alpha)["ce"][M - 1].sum()
                fd = gs * (fp - fm) / (2 * eps)
                assert g[m][t, v] == pytest.approx(fd, abs=2e-8)


def test_gradient_rows_sum_to_zero_and_teacher_ignores_alpha():
    r = rng(11)
    ls = [r.standard_normal((6, 64)) * 3 for _ in range(4)]
    y = r.integers(0, 64, 6)
    g03 = oracle.matryoshka_grad(ls, y, 0.3)
    g1 = oracle.matryoshka_grad(ls, y, 1.0)
    for g in g03 + g1:
        np.testing.assert_allclose(g.sum(axis=1), 0, atol=1e-14)
    np.testing.assert_array_equal(g03[-1], g1[-1])
    p = scipy.special.softmax(ls[-1], axis=1)
    for m in range(3):
        np.testing.assert_allclose(g1[m], scipy.special.softmax(ls[m], axis=1) - p, atol=1e-15)


def test_gradient_matches_torch_autograd_with_detached_teacher():
    r = rng(12)
    ls = [torch.tensor(r.standard_normal((5, 23)) * 2, requires_grad=True) for _ in range(3)]
    y = torch.tensor(r.integers(0, 23, 5))
    p = torch.softmax(ls[-1], dim=1).detach()
    tot = F.cross_entropy(ls[-1], y, reduction="sum")
    for m in range(2):
        ce = F.cross_entropy(ls[m], y, reduction="sum")
        dist = -(p * torch.log_softmax(ls[m], dim=1)).sum()
        tot = tot + 0.7 * ce + 0.3 * dist
    tot.backward()
    g = oracle.matryoshka_grad([l.detach().numpy() for l in ls], y.numpy(), 0.3)
    for m in range(3):
        np.testing.assert_allclose(g[m], ls[m].grad.numpy(), atol=1e-14)


# --------------------------------------------------------- junction backward
def _torch_junction(h, g):
    a = torch.linalg.norm(h, dim=1, keepdim=True)
    b = torch.linalg.norm(g, dim=1, keepdim=True)
    return torch.cat([h * (b / a), g], dim=1)


@pytest.mark.parametrize("stop_grad", [False, True])
def test_junction_backward_matches_torch_autograd(stop_grad):
    """Autograd through the junction (norms, rescale, concat, embedding lookup
    with repeated ids) equals the oracle's chain-rule gradients."""
    r = rng(17)
    n, d_in, de, V = 9, 5, 4, 6
    ids = np.array([0, 3, 3, 1, 0, 3, 5, 2, 3])
    h = torch.tensor(r.standard_normal((n, d_in)) * 4, requires_grad=True)
    emb = torch.tensor(r.standard_normal((V, de)) * 0.02, requires_grad=True)
    dout = r.standard_normal((n, d_in + de))
    hin = h.detach() if stop_grad else h
    out = _torch_junction(hin, emb[torch.from_numpy(ids)])
    (out * torch.from_numpy(dout)).sum().backward()
    dh, demb = oracle.junction_backward(h.detach().numpy(), ids, emb.detach().numpy(), dout,
                                        stop_grad=stop_grad)
    np.testing.assert_allclose(demb, emb.grad.numpy(), atol=1e-12)
    if stop_grad:
        assert h.grad is None and np.all(dh == 0)
    else:
        np.testing.assert_allclose(dh, h.grad.numpy(), atol=1e-12)


def _torch_junction_mode(h, g, mode):
    """The three junction modes written directly in torch."""
    if mode == oracle.JUNCTION_NO_RESCALE:
        return torch.cat([h, g], dim=1)
    a = torch.linalg.norm(h, dim=1, keepdim=True)
    b = torch.linalg.norm(g, dim=1, keepdim=True)
    tail = torch.zeros_like(g) if mode == oracle.JUNCTION_ZERO_FILL else g
    return torch.cat([h * (b / a), tail], dim=1)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("stop_grad", [False, True])
def test_junction_mode_backward_matches_torch_autograd(mode, stop_grad):
    """The ablation modes: autograd through the torch forward of each mode."""
    r = rng(24)
    n, d_in, de, V = 8, 5, 3, 4
    ids = np.array([0, 2, 2, 1, 0, 2, 3, 2])
    h = torch.tensor(r.standard_normal((n, d_in)) * 4, requires_grad=True)
    emb = torch.tensor(r.standard_normal((V, de)) * 0.02, requires_grad=True)
    dout = r.standard_normal((n, d_in + de))
    hin = h.detach() if stop_grad else h
    out = _torch_junction_mode(hin, emb[torch.from_numpy(ids)], mode)
    (out * torch.from_numpy(dout)).sum().backward()
    dh, demb = oracle.junction_backward(h.detach().numpy(), ids, emb.detach().numpy(), dout,
                                        stop_grad=stop_grad, mode=mode)
    np.testing.assert_allclose(demb, emb.grad.numpy(), atol=1e-12)
    if stop_grad:
        assert np.all(dh == 0)
    else:
        np.testing.assert_allclose(dh, h.grad.numpy(), atol=1e-12)


def test_junction_modes_forward():
    """No rescale is a plain concatenation (torch.cat of h and the embedding
    lookup); zero fill keeps the rescaled half (norm = ||e[x]||) and zeros the
    rest; at block 1 they are the lookup and all zeros."""
    r = rng(25)
    n, d_in, de, V = 6, 4, 3, 5
    h = r.standard_normal((n, d_in)) * 4
    emb = r.standard_normal((V, de)) * 0.02
    ids = r.integers(0, V, n)
    g = torch.nn.functional.embedding(torch.from_numpy(ids), torch.from_numpy(emb)).numpy()
    np.testing.assert_array_equal(oracle.junction(h, ids, emb, oracle.JUNCTION_NO_RESCALE),
                                  torch.cat([torch.from_numpy(h), torch.from_numpy(g)], 1).numpy())
    z = oracle.junction(h, ids, emb, oracle.JUNCTION_ZERO_FILL)
    assert np.all(z[:, d_in:] == 0)
    np.testing.assert_allclose(np.linalg.norm(z[:, :d_in], axis=1), np.linalg.norm(g, axis=1),
                               rtol=1e-14)
    cos = np.sum(z[:, :d_in] * h, 1) / np.linalg.norm(z[:, :d_in], axis=1) / np.linalg.norm(h, axis=1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)
    np.testing.assert_array_equal(oracle.junction(None, ids, emb, oracle.JUNCTION_NO_RESCALE), g)
    assert np.all(oracle.junction(None, ids, emb, oracle.JUNCTION_ZERO_FILL) == 0)


def test_junction_backward_block_one_is_scatter_add():
    """d_in = 0: out = e[x], so demb is the scatter-add of dout by id."""
    r = rng(18)
    ids = np.array([2, 2, 0, 4, 2])
    emb = r.standard_normal((6, 3))
    dout = r.standard_normal((5, 3))
    dh, demb = oracle.junction_backward(None, ids, emb, dout)
    want = np.zeros((6, 3))
    for t, v in enumerate(ids):
        want[v] += dout[t]
    assert dh is None
    np.testing.assert_array_equal(demb, want)


def test_junction_backward_gradient_is_orthogonal_to_h():
    """The rescaled half keeps its norm fixed at ||g||, so dL/dh has no
    component along h: h . dL/dh = 0."""
    r = rng(19)
    h = r.standard_normal((7, 6))
    emb = r.standard_normal((3, 2))
    ids = r.integers(0, 3, 7)
    dh, _ = oracle.junction_backward(h, ids, emb, r.standard_normal((7, 8)))
    np.testing.assert_allclose(np.sum(h * dh, axis=1), 0, atol=1e-12)


# ------------------------------------------------------------- head backward
def test_head_backward_matches_torch_autograd_through_the_heads():
    """dL/dh_m and dL/dW^m of the whole forward (heads + loss, teacher detached)
    by torch autograd equal head_backward(matryoshka_grad, h_m, W^m)."""
    r = rng(14)
    D, V, N = (3, 5, 7), 11, 6
    hs = [torch.tensor(r.standard_normal((N, d)), requires_grad=True) for d in D]
    ws = [torch.tensor(r.standard_normal((V, d)) * 0.5, requires_grad=True) for d in D]
    y = torch.tensor(r.integers(0, V, N))
    ls = [h @ w.T for h, w in zip(hs, ws)]
    p = torch.softmax(ls[-1], dim=1).detach()
    tot = F.cross_entropy(ls[-1], y, reduction="sum")
    for m in range(2):
        tot = tot + 0.7 * F.cross_entropy(ls[m], y, reduction="sum") \
            - 0.3 * (p * torch.log_softmax(ls[m], dim=1)).sum()
    tot.backward()
    g = oracle.matryoshka_grad([l.detach().numpy() for l in ls], y.numpy(), 0.3)
    for m in range(3):
        dh, dw = oracle.head_backward(g[m], hs[m].detach().numpy(), ws[m].detach().numpy())
        np.testing.assert_allclose(dh, hs[m].grad.numpy(), atol=1e-13)
        np.testing.assert_allclose(dw, ws[m].grad.numpy(), atol=1e-13)


def test_head_backward_finite_differences_student_exit():
    """Central differences of the total loss in a student's h and W."""
    r = rng(15)
    D, V, N = (2, 4), 5, 3
    hs = [r.standard_normal((N, d)) for d in D]
    ws = [r.standard_normal((V, d)) * 0.7 for d in D]
    y = r.integers(0, V, N)

    def total(hs_, ws_):
        return oracle.matryoshka_loss(oracle.heads(hs_, ws_), y, 0.3)["total"].sum()

    g = oracle.matryoshka_grad(oracle.heads(hs, ws), y, 0.3)
    dh, dw = oracle.head_backward(g[0], hs[0], ws[0])
    eps = 1e-6
    for (arr, grad) in ((hs[0], dh), (ws[0], dw)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            fp = total(hs, ws)
            arr[idx] = old - eps
            fm = total(hs, ws)
            arr[idx] = old
            assert grad[idx] == pytest.approx((fp - fm) / (2 * eps), abs=1e-8)


def test_head_backward_weight_gradient_columns_sum_to_zero():
    """Rows of G sum to zero, so sum_v dW[v] = sum_t (sum_v G[t, v]) h[t] = 0."""
    r = rng(16)
    ls = [r.standard_normal((9, 40)) for _ in range(2)]
    g = oracle.matryoshka_grad(ls, r.integers(0, 40, 9), 0.3)
    h = r.standard_normal((9, 8))
    w = r.standard_normal((40, 8))
    for gm in g:
        _, dw = oracle.head_backward(gm, h, w)
        np.testing.assert_allclose(dw.sum(axis=0), 0, atol=1e-12)


def test_loss_backward_matches_torch_autograd_with_weights_and_scale():
    """The chunked loss + head backward equals torch autograd of
    grad_scale * sum_t sum_m lambda_m L_m through the heads, the teacher's
    softmax detached inside the smaller exits' distillation terms; chunks of
    3 tokens over 7 split the tokens unevenly."""
    r = rng(17)
    D, V, N, a, gs = (3, 5, 8), 13, 7, 0.3, 0.37
    lam = (0.5, 2.0, 1.25)
    hs = [torch.tensor(r.standard_normal((N, d)), requires_grad=True) for d in D]
    ws = [torch.tensor(r.standard_normal((V, d)) * 0.4, requires_grad=True) for d in D]
    y = torch.tensor(r.integers(0, V, N))
    ls = [h @ w.T for h, w in zip(hs, ws)]
    logp = torch.log_softmax(ls[-1], dim=1).detach()
    tot = lam[2] * F.cross_entropy(ls[-1], y, reduction="sum")
    for m in range(2):
        dist = F.kl_div(torch.log_softmax(ls[m], dim=1), logp, log_target=True,
                        reduction="sum") + (-(logp.exp() * logp).sum())
        tot = tot + lam[m] * ((1 - a) * F.cross_entropy(ls[m], y, reduction="sum") + a * dist)
    (gs * tot).backward()
    res, dhs, dws = oracle.loss_backward([h.detach().numpy() for h in hs],
                                         [w.detach().numpy() for w in ws], y.numpy(), a,
                                         grad_scale=gs, exit_weights=lam, chunk=3)
    assert res["total"].sum() == pytest.approx(tot.item(), rel=1e-12)
    for m in range(3):
        np.testing.assert_allclose(dhs[m], hs[m].grad.numpy(), atol=1e-12)
        np.testing.assert_allclose(dws[m], ws[m].grad.numpy(), atol=1e-12)


def test_loss_backward_invariant_to_a_common_head_row():
    """Adding one vector c to every row of W^m shifts each token's logits by
    h_t . c, which leaves every softmax and so G unchanged; dW = G^T h is then
    unchanged and dh = G (W + 1 c^T) = G W because each row of G sums to 0
    (1 - (1 - a) - a for a smaller exit, 1 - 1 for the teacher)."""
    r = rng(18)
    D, V, N = (4, 6), 17, 9
    hs = [r.standard_normal((N, d)) for d in D]
    ws = [r.standard_normal((V, d)) * 0.5 for d in D]
    y = r.integers(0, V, N)
    _, dh0, dw0 = oracle.loss_backward(hs, ws, y, 0.3)
    ws2 = [w + r.standard_normal((1, w.shape[1])) for w in ws]
    _, dh1, dw1 = oracle.loss_backward(hs, ws2, y, 0.3)
    for m in range(2):
        np.testing.assert_allclose(dh1[m], dh0[m], atol=1e-12)
        np.testing.assert_allclose(dw1[m], dw0[m], atol=1e-12)
        assert np.abs(dh0[m]).max() > 1e-3


def test_loss_backward_single_exit_is_plain_cross_entropy_backward():
    """One exit (alpha irrelevant): dh and dW are those of the summed
    library cross-entropy through a linear head."""
    r = rng(19)
    h = torch.tensor(r.standard_normal((6, 5)), requires_grad=True)
    w = torch.tensor(r.standard_normal((11, 5)), requires_grad=True)
    y = torch.tensor(r.integers(0, 11, 6))
    F.cross_entropy(h @ w.T, y, reduction="sum").backward()
    _, dhs, dws = oracle.loss_backward([h.detach().numpy()], [w.detach().numpy()], y.numpy(), 0.9)
    np.testing.assert_allclose(dhs[0], h.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dws[0], w.grad.numpy(), atol=1e-12)


# --------------------------------------------------------------------- heads
def test_heads_against_exactly_rounded_dot_products():
    r = rng(13)
    N, V = 5, 7
    hs = [r.standard_normal((N, d)) * 4 for d in (3, 8, 13)]
    ws = [r.standard_normal((V, d)) * 0.02 for d in (3, 8, 13)]
    ls = oracle.heads(hs, ws)
    for h, w, l in zip(hs, ws, ls):
        assert l.shape == (N, V)
        for t in range(N):
            for v in range(V):
                want = math.fsum(float(a) * float(b) for a, b in zip(h[t], w[v]))
                assert l[t, v] == pytest.approx(want, rel=1e-13, abs=1e-16)


# --------------------------------------------------------------------- junction
def test_junction_invariants():
    r = rng(14)
    N, Din, Dout, V = 40, 24, 40, 50
    h = r.standard_normal((N, Din)) * 4
    h[3] = 0.0
    emb = r.standard_normal((V, Dout - Din)) * 0.02
    ids = r.integers(0, V, N)
    out = oracle.junction(h, ids, emb)
    assert out.shape == (N, Dout)
    np.testing.assert_array_equal(out[:, Din:], emb[ids])                    # exact copy
    b = np.linalg.norm(emb[ids], axis=1)
    nz = np.arange(N) != 3
    np.testing.assert_allclose(np.linalg.norm(out[nz, :Din], axis=1), b[nz], rtol=1e-14)
    cos = np.sum(out[nz, :Din] * h[nz], axis=1) / (
        np.linalg.norm(out[nz, :Din], axis=1) * np.linalg.norm(h[nz], axis=1))
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)                           # positive multiple
    assert np.all(out[3, :Din] == 0)
    np.testing.assert_array_equal(oracle.junction(8.0 * h, ids, emb), out)   # scale invariance
    np.testing.assert_allclose(oracle.junction(0.37 * h, ids, emb), out, rtol=1e-14)


def test_junction_block_one_is_embedding_lookup():
    r = rng(15)
    emb = r.standard_normal((30, 9))
    ids = r.integers(0, 30, 17)
    want = F.embedding(torch.from_numpy(ids), torch.from_numpy(emb)).numpy()
    np.testing.assert_array_equal(oracle.junction(None, ids, emb), want)
    np.testing.assert_array_equal(oracle.junction(np.zeros((17, 0)), ids, emb), want)


# --------------------------------------------------------------------- argmax / accept
def test_argmax_ties_lowest_index_brute_force():
    r = rng(16)
    l = np.round(r.standard_normal((50, 12)), 1)
    l[:, 7] = l.max(axis=1)          # plant ties with the max
    got = oracle.argmax_lowest(l)
    for t in range(50):
        best = 0
        for v in range(12):
            if l[t, v] > l[t, best]:
                best = v
        assert got[t] == best
    assert np.all(got <= 7)


def test_accept_prefix_brute_force():
    r = rng(17)
    B, P = 200, 7
    d = r.integers(0, 3, (B, P))
    v = np.where(r.random((B, P)) < 0.7, d, r.integers(0, 3, (B, P)))
    got = oracle.accept_prefix(d, v, 6)
    for b in range(B):
        k = 0
        for i in range(6):
            if d[b, i] != v[b, i]:
                break
            k += 1
        assert got[b] == k
    assert set(got.tolist()) >= {0, 6}


# --------------------------------------------------------------------- covariance
def test_vocab_and_token_permutation_covariance():
    r = rng(18)
    M, N, V = 3, 12, 31
    ls = [r.standard_normal((N, V)) * 3 for _ in range(M)]
    y = r.integers(0, V, N)
    base = oracle.matryoshka_loss(ls, y, 0.3)
    gb = oracle.matryoshka_grad(ls, y, 0.3)
    pv = r.permutation(V)
    inv = np.argsort(pv)
    lsp = [l[:, pv] for l in ls]
    o = oracle.matryoshka_loss(lsp, inv[y], 0.3)
    np.testing.assert_allclose(o["loss"], base["loss"], rtol=1e-12)
    for g, g0 in zip(oracle.matryoshka_grad(lsp, inv[y], 0.3), gb):
        np.testing.assert_allclose(g, g0[:, pv], atol=1e-15)
    pt = r.permutation(N)
    o = oracle.matryoshka_loss([l[pt] for l in ls], y[pt], 0.3)
    np.testing.assert_allclose(o["loss"], base["loss"][:, pt], rtol=1e-14)


def test_forward_tokens_chunked_equals_whole():
    s = synth.make_suite((16, 32, 48), 97, 2, 19, dtype="bf16", seed=3)
    res, g = oracle.forward_tokens(s.h, s.w, s.labels, 0.3, 0.25, chunk=5)
    lg = oracle.heads(s.h, s.w)
    whole = oracle.matryoshka_loss(lg, s.labels, 0.3)
    gw = oracle.matryoshka_grad(lg, s.labels, 0.3, 0.25)
    np.testing.assert_allclose(res["loss"], whole["loss"], rtol=1e-13)
    for a, b in zip(g, gw):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-16)
    rows = np.array([5, 0, 37])
    r2, g2 = oracle.forward_tokens(s.h, s.w, s.labels, 0.3, 0.25, rows=rows, exits=(0, 2))
    np.testing.assert_allclose(r2["ce"][1], oracle.matryoshka_loss([lg[0][rows], lg[2][rows]],
                                                                   s.labels[rows], 0.3)["ce"][1])


# ------------------------------------------------------ sampled verification
def test_beta_is_one_minus_total_variation():
    """beta = sum_v min(p_v, q_v) = 1 - TV(p, q) for any two distributions."""
    r = rng(20)
    B, V = 5, 50
    dl = r.standard_normal((B, 2, V)) * 2
    vl = r.standard_normal((B, 2, V)) * 2
    beta, _, _ = oracle.speculative_verify(dl, vl, np.zeros((B, 2), int), np.zeros((B, 2)),
                                           np.zeros(B), 1, temperature=0.8, top_p=0.9)
    p = oracle.nucleus(dl[:, 0], 0.8, 0.9)
    q = oracle.nucleus(vl[:, 0], 0.8, 0.9)
    np.testing.assert_allclose(beta[:, 0], 1.0 - 0.5 * np.abs(p - q).sum(axis=1), atol=1e-12)


def test_nucleus_limits():
    r = rng(21)
    l = r.standard_normal((4, 30)) * 3
    np.testing.assert_allclose(oracle.nucleus(l, 1.0, 1.0), scipy.special.softmax(l, axis=1), atol=1e-15)
    tiny = oracle.nucleus(l, 1.0, 1e-9)
    np.testing.assert_array_equal(np.argmax(tiny, axis=1), np.argmax(l, axis=1))
    assert np.all(np.isclose(tiny.max(axis=1), 1.0))
    # the kept set is a set of top entries reaching the mass, ties at the edge kept
    lt = np.array([3.0, 1.0, 1.0, 0.0, -1.0])
    p = scipy.special.softmax(lt)
    keep = oracle.nucleus(lt, 1.0, p[0] + 1e-9) > 0
    np.testing.assert_array_equal(keep, [True, True, True, False, False])
    for tp in (0.3, 0.6, 0.95):
        n = oracle.nucleus(l, 1.0, tp)
        full = scipy.special.softmax(l, axis=1)
        for i in range(4):
            kept = n[i] > 0
            assert full[i][kept].sum() >= tp - 1e-12
            assert full[i][kept].min() >= full[i][~kept].max(initial=0.0)


def test_speculative_sampling_emits_the_verifier_distribution():
    """Integrated over the drafted token (drawn from p) and over both uniforms,
    the first emitted token is distributed exactly as q: the accept / residual
    rule of speculative sampling.  Midpoint grids of 200 points per uniform."""
    r = rng(22)
    V = 3
    dl = r.standard_normal((1, 2, V)) * 1.5
    vl = r.standard_normal((1, 2, V)) * 1.5
    p = oracle.nucleus(dl[0, 0])
    q = oracle.nucleus(vl[0, 0])
    grid = (np.arange(200) + 0.5) / 200
    dist = np.zeros(V)
    for x in range(V):
        for ua in grid:
            for un in grid:
                _, acc, nxt = oracle.speculative_verify(dl, vl, np.array([[x, 0]]),
                                                        np.array([[ua, 0.0]]), np.array([un]), 1)
                emitted = x if acc[0] == 1 else nxt[0]
                dist[emitted] += p[x] / len(grid) ** 2
    np.testing.assert_allclose(dist, q, atol=1e-2)


def test_greedy_limit_is_greedy_acceptance():
    """As the temperature goes to 0 with drafted tokens the draft exit's argmax,
    acceptance is the greedy prefix match and the next token the verifier's argmax
    at the first mismatch."""
    r = rng(23)
    B, P, V = 20, 7, 40
    dl = r.standard_normal((B, P, V)) * 2
    vl = dl + r.standard_normal((B, P, V)) * 0.8
    dtok = oracle.argmax_lowest(dl)
    _, acc, nxt = oracle.speculative_verify(dl, vl, dtok, r.random((B, P)), r.random(B), 6,
                                            temperature=1e-4)
    vtok = oracle.argmax_lowest(vl)
    np.testing.assert_array_equal(acc, oracle.accept_prefix(dtok, vtok, 6))
    np.testing.assert_array_equal(nxt, vtok[np.arange(B), acc])


# ------------------------------------------------ divergences and exit weights
def test_divergence_values_against_scipy():
    """Reverse KL is scipy's relative entropy of q to p; Jensen-Shannon is the
    square of scipy's Jensen-Shannon distance (natural log); total variation is
    half the L1 distance and 1 - beta of the speculative rule."""
    import scipy.spatial.distance
    import scipy.stats
    r = rng(30)
    lp = r.standard_normal((6, 40)) * 2
    lq = r.standard_normal((6, 40)) * 2
    p, q = scipy.special.softmax(lp, axis=1), scipy.special.softmax(lq, axis=1)
    np.testing.assert_allclose(oracle.divergence(p, q, oracle.DIV_REVERSE_KL),
                               scipy.stats.entropy(q, p, axis=1), rtol=1e-12)
    np.testing.assert_allclose(oracle.divergence(p, q, oracle.DIV_FORWARD),
                               scipy.stats.entropy(p, axis=1) + scipy.stats.entropy(p, q, axis=1),
                               rtol=1e-12)
    js = np.array([scipy.spatial.distance.jensenshannon(p[i], q[i]) ** 2 for i in range(6)])
    np.testing.assert_allclose(oracle.divergence(p, q, oracle.DIV_JS), js, rtol=1e-10)
    beta, _, _ = oracle.speculative_verify(lq[:, None, :].repeat(2, 1), lp[:, None, :].repeat(2, 1),
                                           np.zeros((6, 2), int), np.zeros((6, 2)), np.zeros(6), 1)
    np.testing.assert_allclose(oracle.divergence(p, q, oracle.DIV_TV), 1.0 - beta[:, 0], rtol=1e-12)
    np.testing.assert_allclose(oracle.divergence(p, q, oracle.DIV_TV),
                               0.5 * np.abs(p - q).sum(axis=1), rtol=1e-12)
    for k in (oracle.DIV_REVERSE_KL, oracle.DIV_JS, oracle.DIV_TV):
        np.testing.assert_allclose(oracle.divergence(p, p, k), 0.0, atol=1e-15)


@pytest.mark.parametrize("div", [1, 2, 3])
def test_divergence_loss_gradient_central_differences(div):
    """The whole loss (three exits, alpha, exit weights) with each divergence:
    the oracle gradient of every student exit against central differences of
    the oracle total, the teacher held fixed inside D (stop-gradient)."""
    r = rng(31 + div)
    V, n, M, alpha = 7, 3, 3, 0.4
    lam = np.array([0.5, 2.0, 1.5])
    ls = [r.standard_normal((n, V)) * 1.5 for _ in range(M)]
    y = r.integers(0, V, n)
    g = oracle.matryoshka_grad(ls, y, alpha, exit_weights=lam, div=div)
    p = scipy.special.softmax(ls[-1], axis=1)
    eps = 1e-6
    for m in range(M - 1):
        num = np.zeros((n, V))
        for t in range(n):
            for v in range(V):
                def total(delta):
                    lm = ls[m].copy()
                    lm[t, v] += delta
                    q = scipy.special.softmax(lm, axis=1)
                    ce = -np.log(q[np.arange(n), y])
                    return np.sum(lam[m] * ((1 - alpha) * ce + alpha * oracle.divergence(p, q, div)))
                num[t, v] = (total(eps) - total(-eps)) / (2 * eps)
        np.testing.assert_allclose(g[m], num, atol=1e-7)
    # the teacher's gradient ignores the divergence, scaled by its weight
    q = p.copy()
    q[np.arange(n), y] -= 1.0
    np.testing.assert_allclose(g[-1], lam[-1] * q, atol=1e-15)


def test_reverse_kl_gradient_matches_torch_kl_div():
    """torch.nn.functional.kl_div with log targets computes KL(target || input):
    target = log_softmax of the student, input = the detached teacher's."""
    r = rng(35)
    n, V = 5, 11
    ls = torch.tensor(r.standard_normal((n, V)) * 2, requires_grad=True)
    lt = torch.tensor(r.standard_normal((n, V)) * 2)
    kl = torch.nn.functional.kl_div(torch.log_softmax(lt, 1), torch.log_softmax(ls, 1),
                                    reduction="none", log_target=True).sum(1)
    kl.sum().backward()
    p = scipy.special.softmax(lt.numpy(), axis=1)
    q = scipy.special.softmax(ls.detach().numpy(), axis=1)
    np.testing.assert_allclose(oracle.divergence(p, q, oracle.DIV_REVERSE_KL), kl.detach().numpy(),
                               rtol=1e-12)
    np.testing.assert_allclose(oracle.divergence_grad(p, q, oracle.DIV_REVERSE_KL), ls.grad.numpy(),
                               atol=1e-13)


def test_exit_weights_scale_total_and_gradients():
    """total = sum_m lambda_m L_m; equal weights of 1 are the default."""
    r = rng(36)
    ls = [r.standard_normal((4, 9)) for _ in range(3)]
    y = r.integers(0, 9, 4)
    lam = np.array([0.25, 3.0, 0.5])
    a = oracle.matryoshka_loss(ls, y, 0.3)
    b = oracle.matryoshka_loss(ls, y, 0.3, exit_weights=lam)
    np.testing.assert_array_equal(a["loss"], b["loss"])
    np.testing.assert_allclose(b["total"], (lam[:, None] * a["loss"]).sum(0), rtol=1e-15)
    ones = oracle.matryoshka_loss(ls, y, 0.3, exit_weights=np.ones(3))
    np.testing.assert_array_equal(ones["total"], a["total"])
