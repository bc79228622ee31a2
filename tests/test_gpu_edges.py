"""Edge cases of the HIP path: tiny and ragged vocabularies and widths,
empty batches, many exits, out-of-range labels, the invariants the method
fixes, and run-to-run determinism."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth
from gpu_util import DevSuite, assert_grad_close, assert_loss_close, log, to_np

pytestmark = pytest.mark.gpu


def full_compare(nel, s, alpha=0.3, tol_loss=1e-3, tol_grad=2e-2):
    ds = DevSuite(s)
    mean, tok, dl = nel.matryoshka_loss(ds.h, ds.w, ds.labels, alpha_d=alpha)
    tok = to_np(tok)
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, alpha, 1.0)
    assert_loss_close(tok[:, 0], ref["ce"], tol_loss, "CE")
    assert_loss_close(tok[:, 1], ref["dist"], tol_loss, "Dist")
    assert_loss_close(tok[:, 2], ref["loss"], tol_loss, "L")
    for m in range(s.n_exits):
        assert_grad_close(to_np(dl[m]), grads[m], tol_grad, f"dlogits {m}")
    return ds, to_np(mean), tok, dl


@pytest.mark.parametrize("V", [1, 2, 7, 16, 129, 257])
@pytest.mark.parametrize("widths", [(8, 16, 24), (5, 11, 17)])
def test_tiny_and_ragged_vocab(nel, V, widths):
    s = synth.make_suite(widths, V, 1, 33, seed=V)
    log(f"[edge] V={V} widths={widths}")
    full_compare(nel, s)


@pytest.mark.parametrize("N", [1, 2, 127, 128, 129])
def test_ragged_token_counts(nel, N):
    s = synth.make_suite((64, 128), 300, 1, N, seed=N)
    full_compare(nel, s)


def test_eight_exits(nel):
    s = synth.make_suite(tuple(16 * (i + 1) for i in range(8)), 640, 1, 96, seed=51)
    full_compare(nel, s)


def test_empty_batch(nel):
    import torch
    s = synth.make_suite((8, 16), 10, 1, 1, seed=52)
    ds = DevSuite(s)
    h = [x[:0] for x in ds.h]
    mean, tok, dl = nel.matryoshka_loss(h, ds.w, ds.labels[:0])
    torch.cuda.synchronize()
    assert tok.shape == (2, 3, 0) and dl[0].shape == (0, 10)
    assert np.all(to_np(mean) == 0)
    out = nel.junction(h[0], ds.ids[:0], ds.emb[1])
    assert out.shape == (0, 16)


def test_bad_labels_give_nan_and_flag(nel):
    import torch
    s = synth.make_suite((32, 64), 200, 1, 40, seed=53)
    ds = DevSuite(s)
    labels = ds.labels.clone()
    labels[3] = 200
    labels[7] = -5
    ws = nel.loss_workspace(ds.h[0].device, 2, 40, 200)
    nel.clear_flags(ws)
    mean, tok, dl = nel.matryoshka_loss(ds.h, ds.w, labels, workspace=ws)
    tok = to_np(tok)
    assert nel.read_flags(ws) == nel.FLAG_BAD_LABEL
    assert np.all(np.isnan(tok[:, :, [3, 7]]))
    assert np.all(np.isnan(to_np(dl[0])[[3, 7]]))
    ok = np.setdiff1d(np.arange(40), [3, 7])
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, 0.3, rows=ok)
    assert_loss_close(tok[:, 0, ok], ref["ce"], 1e-3, "CE")
    assert_grad_close(to_np(dl[1])[ok], grads[1], 2e-2, "dlogits")
    assert np.isnan(to_np(mean)).all()
    nel.clear_flags(ws)
    assert nel.read_flags(ws) == 0


def _loss_either(nel, ds, packed, hs=None, ws=None, alpha=0.3):
    """(tok, dlogits) of the row-major or the packed (benchmarked) path."""
    hs = ds.h if hs is None else hs
    ws = ds.w if ws is None else ws
    if packed:
        _, tok, dl = nel.matryoshka_loss_packed(hs, [nel.pack_weights(w) for w in ws], ds.labels,
                                                alpha_d=alpha)
    else:
        _, tok, dl = nel.matryoshka_loss(hs, ws, ds.labels, alpha_d=alpha)
    return to_np(tok), dl


# The packed path runs one of two GEMMs by the mean exit width (below 512:
# two workgroups per CU; from 512, as at every benchmark width: one wavefront
# per SIMD); "packed-wide" takes the second.
PATHS = [("row-major", False, (128, 256)), ("packed", True, (128, 256)),
         ("packed-wide", True, (1536, 1664))]


@pytest.mark.parametrize("name,packed,widths", PATHS, ids=[p[0] for p in PATHS])
def test_student_equal_to_teacher_gives_teacher_entropy(nel, name, packed, widths):
    """l_1 = l_2 exactly: W^2 = [W^1, 0] and h_2 = [h_1, noise].  On the packed
    path Dist is formed from the fp16 teacher weights and fp16 l - m."""
    V = 3008 if packed else 3000
    d1 = widths[0]
    s = synth.make_suite(widths, V, 2, 96, seed=54)
    s.w[1][:, :d1] = s.w[0]
    s.w[1][:, d1:] = 0
    s.h[1][:, :d1] = s.h[0]
    ds = DevSuite(s)
    tok, _ = _loss_either(nel, ds, packed)
    l = oracle.heads([s.h[1]], [s.w[1]])[0]
    H = scipy.stats.entropy(scipy.special.softmax(l, axis=1), axis=1)
    assert_loss_close(tok[0, 1], H, 1e-3, "Dist vs entropy")
    np.testing.assert_allclose(tok[0, 0], tok[1, 0], rtol=1e-5)   # same CE


M1_PATHS = [("row-major", False, (64, 96, 160), 1100), ("packed", True, (64, 128, 192), 1120),
            ("packed-wide", True, (1536, 1600, 1664), 1120)]


@pytest.mark.parametrize("name,packed,widths,V", M1_PATHS, ids=[p[0] for p in M1_PATHS])
def test_single_exit_and_alpha_zero_reduce_to_cross_entropy(nel, name, packed, widths, V):
    import torch.nn.functional as F
    import torch
    s = synth.make_suite(widths, V, 1, 130, seed=55)
    ds = DevSuite(s)
    for m in range(3):
        tok, dl = _loss_either(nel, ds, packed, hs=[ds.h[m]], ws=[ds.w[m]])
        l = torch.from_numpy(oracle.heads([s.h[m]], [s.w[m]])[0])
        ce = F.cross_entropy(l, torch.from_numpy(s.labels).long(), reduction="none").numpy()
        assert_loss_close(tok[0, 0], ce, 1e-3, "M=1 CE")
        assert_loss_close(tok[0, 2], ce, 1e-3, "M=1 L")
        # the single exit's gradient is softmax - onehot (the teacher's, unmixed)
        g = scipy.special.softmax(l.numpy(), axis=1)
        g[np.arange(len(s.labels)), s.labels] -= 1.0
        assert_grad_close(to_np(dl[0]), g, 2e-2, "M=1 dlogits")
    tok, _ = _loss_either(nel, ds, packed, alpha=0.0)
    np.testing.assert_array_equal(tok[:, 2], tok[:, 0])


def test_determinism(nel):
    import torch
    s = synth.make_suite((256, 512, 768), 4096, 2, 300, seed=56)
    ds = DevSuite(s)
    a = nel.matryoshka_loss(ds.h, ds.w, ds.labels)
    a = (a[0].clone(), a[1].clone(), [x.clone() for x in a[2]])
    b = nel.matryoshka_loss(ds.h, ds.w, ds.labels)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for x, y in zip(a[2], b[2]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    _, am1 = nel.exit_heads(ds.h, ds.w)
    _, am2 = nel.exit_heads(ds.h, ds.w)
    assert torch.equal(am1, am2)


def test_vocab_permutation_covariance(nel):
    s = synth.make_suite((64, 128), 900, 1, 100, seed=57)
    ds = DevSuite(s)
    _, tok, dl = nel.matryoshka_loss(ds.h, ds.w, ds.labels)
    tok = to_np(tok)
    perm = np.random.default_rng(58).permutation(900)
    inv = np.argsort(perm)
    s2 = synth.make_suite((64, 128), 900, 1, 100, seed=57)
    s2.w = [w[perm] for w in s2.w]
    s2.labels = inv[s2.labels].astype(np.int32)
    ds2 = DevSuite(s2)
    _, tok2, dl2 = nel.matryoshka_loss(ds2.h, ds2.w, ds2.labels)
    assert_loss_close(to_np(tok2), tok, 1e-4, "permuted losses")
    for m in range(2):
        assert_grad_close(to_np(dl2[m]), to_np(dl[m])[:, perm], 1e-2, "permuted dlogits")


def test_junction_backward_without_tokens(nel):
    """No tokens: dL/dh is empty and every embedding row's gradient is 0, in
    every junction mode and at block 1."""
    import torch
    s = synth.make_suite((8, 16), 10, 1, 3, seed=53)
    ds = DevSuite(s)
    dout = torch.zeros(0, 16, dtype=torch.bfloat16, device="cuda:0")
    for mode in (0, 1, 2):
        dh, demb = nel.junction_backward(ds.h[0][:0], ds.ids[:0], ds.emb[1], dout, mode=mode)
        torch.cuda.synchronize()
        assert dh.shape == (0, 8) and demb.shape == (10, 8)
        assert float(demb.abs().max()) == 0.0
        assert nel.junction(ds.h[0][:0], ds.ids[:0], ds.emb[1], mode=mode).shape == (0, 16)
    _, demb = nel.junction_backward(None, ds.ids[:0], ds.emb[0],
                                    torch.zeros(0, 8, dtype=torch.bfloat16, device="cuda:0"))
    torch.cuda.synchronize()
    assert float(demb.abs().max()) == 0.0


@pytest.mark.parametrize("div", [1, 2, 3])
def test_divergence_degenerate(nel, div):
    """V = 1: every softmax is [1], so CE, every divergence and every gradient
    are 0.  One token at V = 7 (fp32): the oracle, entry by entry."""
    import torch
    s = synth.make_suite((8, 16, 24), 1, 1, 5, dtype="f32", seed=54)
    ds = DevSuite(s)
    mean, tok, dl = nel.matryoshka_loss(ds.h, ds.w, ds.labels, divergence=div)
    torch.cuda.synchronize()
    assert np.all(np.abs(to_np(tok)) <= 1e-6) and np.all(np.abs(to_np(mean)) <= 1e-6)
    for g in dl:
        assert float(g.abs().max()) <= 1e-6
    s = synth.make_suite((8, 16, 24), 7, 1, 1, dtype="f32", seed=55)
    ds = DevSuite(s)
    mean, tok, dl = nel.matryoshka_loss(ds.h, ds.w, ds.labels, divergence=div,
                                        exit_weights=[0.5, 1.5, 1.0])
    torch.cuda.synchronize()
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, s.alpha, exit_weights=[0.5, 1.5, 1.0],
                                       div=div)
    np.testing.assert_allclose(to_np(tok)[:, 1], ref["dist"], atol=1e-5, rtol=1e-4)
    np.testing.assert_allclose(to_np(tok)[:, 2], ref["loss"], atol=1e-5, rtol=1e-4)
    for m in range(3):
        np.testing.assert_allclose(to_np(dl[m]), grads[m], atol=1e-4)


def test_speculative_empty_batch(nel):
    import torch
    z = torch.zeros(0, 7, 50, dtype=torch.float32, device="cuda:0")
    beta, acc, nxt = nel.speculative_verify(z, z, torch.zeros(0, 7, dtype=torch.int32, device="cuda:0"),
                                            torch.zeros(0, 7, device="cuda:0"),
                                            torch.zeros(0, device="cuda:0"), 6)
    torch.cuda.synchronize()
    assert beta.shape == (0, 6) and acc.shape == (0,) and nxt.shape == (0,)
