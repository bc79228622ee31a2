"""The packed-weight path (nel_pack_weights + nel_matryoshka_loss_packed /
nel_exit_heads_packed) against the CPU oracle, at the same bars as the
row-major path: losses rel 1e-3 per token (scaled by max(1,|ref|)), bf16
logit gradients 2e-2 max-abs, argmax exact wherever the exact top-2 margin
exceeds the fp32 accumulation bound.  The full-size cases run the launch
configuration the benchmark times."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DevSuite, assert_grad_close, assert_loss_close, check_full, head_error_bound,
                      log, run_loss, sample_rows, to_np)
from test_gpu_verify import check_argmax

pytestmark = pytest.mark.gpu


def vperm(q):
    """A-row q of a 32-row operand block holds vocabulary entry vperm(q) (nel.h)."""
    return ((q >> 2) & 1) * 16 + (q >> 3) * 4 + (q & 3)


def packed_reference(w: np.ndarray) -> np.ndarray:
    """The tiled layout written out from its definition in nel.h:
    P[((rb * D/16 + kp) * 64 + l) * 8 + j] = W[32 rb + vperm(l % 32), 16 kp + 8 (l / 32) + j]."""
    V, D = w.shape
    rb, kp, l, j = np.meshgrid(np.arange(V // 32), np.arange(D // 16), np.arange(64), np.arange(8),
                               indexing="ij")
    rows = 32 * rb + vperm(l % 32)
    cols = 16 * kp + 8 * (l // 32) + j
    return w[rows, cols].reshape(-1)


@pytest.mark.parametrize("V,D", [(32, 64), (96, 192), (544, 320)])
def test_pack_layout(nel, V, D):
    import torch
    r = np.random.default_rng(V + D)
    w = synth.round_to_bf16(r.standard_normal((V, D)).astype(np.float32))
    from gpu_util import dev_tensor
    wd = dev_tensor(w, "bf16")
    p = nel.pack_weights(wd)
    torch.cuda.synchronize()
    got = to_np(p).reshape(-1)
    np.testing.assert_array_equal(got, packed_reference(w.astype(np.float64)))


PACKED_SMALL = [
    # (name, widths, V, batch, seq, seed): ragged token counts, partial last
    # vocabulary tile (V % 256 != 0), V below one tile, odd K-step counts
    ("3exit-ragged-n", (64, 128, 256), 1024, 3, 100, 51),
    ("2exit-partial-vtile", (128, 192), 544, 2, 70, 52),
    ("4exit-tiny-vocab", (64, 128, 192, 256), 96, 1, 129, 53),
    ("1exit", (64,), 256, 1, 1, 54),
    ("3exit-odd-steps", (64, 192, 320), 800, 1, 257, 55),
]


@pytest.mark.parametrize("name,widths,V,B,S,seed", PACKED_SMALL, ids=[c[0] for c in PACKED_SMALL])
def test_packed_loss_small_full_compare(nel, name, widths, V, B, S, seed):
    s = synth.make_suite(widths, V, B, S, seed=seed)
    log(f"[packed] {name}: widths={s.widths} V={s.vocab} N={s.n_tokens}")
    check_full(nel, s, s.alpha, packed=True)


@pytest.mark.parametrize("alpha", [0.0, 1.0])
def test_packed_loss_alpha_edges(nel, alpha):
    s = synth.make_suite((128, 192, 256), 1536, 2, 160, seed=56)
    log(f"[packed] alpha={alpha}")
    check_full(nel, s, alpha, packed=True)


def test_packed_loss_grad_scale(nel):
    s = synth.make_suite((64, 128, 192), 640, 2, 64, seed=57)
    check_full(nel, s, 0.3, grad_scale=1.0 / 128, packed=True)


def test_packed_matches_row_major_losses(nel):
    """Both GEMMs compute the same losses (different tilings and teacher-weight
    precision: equal to well within the oracle bar)."""
    s = synth.make_suite((128, 256, 384), 2048, 2, 300, seed=58)
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    m1, t1, d1 = run_loss(nel, ds, 0.3)
    m2, t2, d2 = run_loss(nel, ds, 0.3, packed=pw)
    assert_loss_close(t2, t1, 2e-4, "token losses")
    assert_loss_close(m2, m1, 2e-4, "means")
    for m in range(s.n_exits):
        assert_grad_close(to_np(d2[m]), to_np(d1[m]), 2e-2, f"dlogits exit {m}")


@pytest.mark.parametrize("k,alpha", [(1, 0.3), (2, 0.0), (2, 0.3), (2, 1.0), (3, 0.3)])
def test_packed_loss_full_size_sampled(nel, k, alpha):
    import torch
    s = synth.make_workload(k)
    log(f"[packed] workload {k} ({s.name}) alpha={alpha}: N={s.n_tokens} widths={s.widths}")
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    mean, tok, dl = run_loss(nel, ds, alpha, packed=pw)
    rows = sample_rows(s.n_tokens, 28, 200 + k)
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, alpha, 1.0, rows=rows)
    assert_loss_close(tok[:, 0, rows], ref["ce"], 1e-3, "CE")
    assert_loss_close(tok[:, 1, rows], ref["dist"], 1e-3, "Dist")
    assert_loss_close(tok[:, 2, rows], ref["loss"], 1e-3, "L")
    idx = torch.from_numpy(rows).cuda()
    for m in range(s.n_exits):
        err = assert_grad_close(to_np(dl[m].index_select(0, idx)), grads[m], 2e-2,
                                f"dlogits exit {m}")
        log(f"  exit {m}: max |dlogits err| {err:.2e}")
    want = np.concatenate([tok[:, 0].mean(1), tok[:, 1].mean(1), tok[:, 2].mean(1),
                           [tok[:, 2].sum(0).mean()]])
    np.testing.assert_allclose(mean, want, rtol=2e-6, atol=1e-6)
    for m in range(s.n_exits):
        assert float(dl[m].float().sum(dim=1).abs().max()) < 5e-2


def test_packed_heads_verify_workload(nel):
    """Greedy verification shape (102 sequences x 7 positions, exits 1 and 3)."""
    import torch
    s = synth.make_workload(4)
    ds = DevSuite(s, exits=s.exits)
    pw = [nel.pack_weights(w) for w in ds.w]
    _, am = nel.exit_heads_packed(ds.h, pw, want_logits=False, want_argmax=True)
    _, am_rm = nel.exit_heads(ds.h, ds.w, want_logits=False, want_argmax=True)
    am = am.cpu().numpy()
    amb = sum(check_argmax(am[i], s.h[m], s.w[m]) for i, m in enumerate(s.exits))
    log(f"[packed] verify workload: ambiguous argmax rows {amb}")
    if amb == 0:
        np.testing.assert_array_equal(am, am_rm.cpu().numpy())
    B, P = s.batch, s.seq
    acc = nel.accept_prefix(torch.from_numpy(am[0].reshape(B, P)).cuda(),
                            torch.from_numpy(am[1].reshape(B, P)).cuda(), 6).cpu().numpy()
    np.testing.assert_array_equal(acc, oracle.accept_prefix(am[0].reshape(B, P),
                                                            am[1].reshape(B, P), 6))


def test_packed_heads_logits_partial_tile(nel):
    s = synth.make_suite((64, 128), 544, 1, 131, seed=59)
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    logits, am = nel.exit_heads_packed(ds.h, pw, want_logits=True, want_argmax=True)
    am = am.cpu().numpy()
    for m in range(2):
        l = oracle.heads([s.h[m]], [s.w[m]])[0]
        bound = head_error_bound(s.h[m], s.w[m])
        assert np.all(np.abs(to_np(logits[m]) - l) <= bound + 1e-30)
        check_argmax(am[m], s.h[m], s.w[m])
