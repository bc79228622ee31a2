"""The packed-weight path (nel_pack_weights + nel_matryoshka_loss_packed /
nel_exit_heads_packed) against the CPU oracle, at the same bars as the
row-major path: losses rel 1e-3 per token (scaled by max(1,|ref|)), bf16
logit gradients 2e-2 max-abs, argmax by the rule of test_gpu_verify (the
verify shape itself is covered there, on both paths).  The full-size cases
run the launch configuration the benchmark times."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DevSuite, assert_grad_close, assert_loss_close, check_full, head_error_bound,
                      log, run_loss, sample_rows, to_np)
from test_gpu_verify import check_argmax

pytestmark = pytest.mark.gpu


def packed_reference(w: np.ndarray) -> np.ndarray:
    """The tiled layout written out from its definition in nel.h:
    P[((rb * D/32 + kb) * 64 + l) * 8 + j] = W[16 rb + l % 16, 32 kb + 8 (l / 16) + j]."""
    V, D = w.shape
    rb, kb, l, j = np.meshgrid(np.arange(V // 16), np.arange(D // 32), np.arange(64), np.arange(8),
                               indexing="ij")
    rows = 16 * rb + l % 16
    cols = 32 * kb + 8 * (l // 16) + j
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
    # mean width >= 512: the one-wavefront-per-SIMD kernel (512-entry tiles,
    # statistics per 128 entries).  Partial last tile with wavefronts wholly
    # beyond V, V below one wavefront's 128 entries, odd step counts, exits of
    # fewer K steps than the main loop's unrolling (1 and 5)
    ("3exit-wide-ragged", (1536, 1600, 1664), 1056, 1, 300, 58),
    ("2exit-wide-tiny-vocab", (1536, 1600), 96, 1, 129, 59),
    ("1exit-wide", (1600,), 544, 2, 70, 60),
    ("2exit-wide-short-exits", (64, 3008), 512, 1, 140, 61),
    ("2exit-wide-five-steps", (320, 2752), 640, 1, 131, 62),
    # V = 32 (two of a wavefront's eight 16-entry blocks exist), a single
    # token, and a mean width of exactly 512 (the rule's threshold)
    ("2exit-wide-vocab-32", (512, 576), 32, 1, 70, 63),
    ("2exit-wide-one-token", (1536, 1600), 1056, 1, 1, 64),
    ("2exit-mean-512", (448, 576), 800, 2, 67, 65),
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


@pytest.mark.parametrize("V,S", [(544, 131), (1056, 11264)], ids=["few-tokens", "many-tokens"])
def test_packed_heads_logits_partial_tile(nel, V, S):
    """Logits and argmax against the oracle with a partial last vocabulary
    tile.  Few tokens run the two-workgroups-per-CU argmax GEMM; 11,264 tokens
    give the one-wavefront-per-SIMD one at least two workgroups per CU (its
    512-entry tiles: the last has wavefronts wholly beyond V)."""
    s = synth.make_suite((64, 128), V, 1, S, seed=59)
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    logits, am = nel.exit_heads_packed(ds.h, pw, want_logits=True, want_argmax=True)
    am = am.cpu().numpy()
    for m in range(2):
        l = oracle.heads([s.h[m]], [s.w[m]])[0]
        bound = head_error_bound(s.h[m], s.w[m])
        assert np.all(np.abs(to_np(logits[m]) - l) <= bound + 1e-30)
        check_argmax(am[m], s.h[m], s.w[m], to_np(logits[m]))


@pytest.mark.parametrize("k", [2, 1, 3], ids=["500M-1.5B-3B-3exit", "200M-proxy-3exit", "4exit"])
def test_packed_every_token(nel, k):
    """Each bf16 training workload (k = 2 is the benchmark's: 500M/1.5B/3B
    widths, 16,384 tokens, V = 32,768, alpha 0.3) in the benchmark's launch
    configuration, every token against the oracle: CE, Dist and L per token
    and exit, every logit gradient, and the reported means (rel 1e-3 of the
    oracle's float64 means)."""
    import torch
    s = synth.make_workload(k)
    log(f"[packed] workload {k} ({s.name}) every token: N={s.n_tokens} widths={s.widths}")
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    mean, tok, dl = run_loss(nel, ds, s.alpha, packed=pw)
    M, N = s.n_exits, s.n_tokens
    ce, dist, loss = [], [], []
    worst_g = 0.0
    chunk = 2048
    for c0 in range(0, N, chunk):
        rows = np.arange(c0, min(c0 + chunk, N))
        ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, s.alpha, 1.0, rows=rows, chunk=chunk)
        assert_loss_close(tok[:, 0, rows], ref["ce"], 1e-3, f"CE rows {c0}..")
        assert_loss_close(tok[:, 1, rows], ref["dist"], 1e-3, f"Dist rows {c0}..")
        assert_loss_close(tok[:, 2, rows], ref["loss"], 1e-3, f"L rows {c0}..")
        for m in range(M):
            g = to_np(dl[m][c0:c0 + len(rows)])
            worst_g = max(worst_g, assert_grad_close(g, grads[m], 2e-2, f"dlogits exit {m} rows {c0}.."))
        ce.append(ref["ce"])
        dist.append(ref["dist"])
        loss.append(ref["loss"])
        log(f"  [every token] rows {c0}..{c0 + len(rows) - 1} ok")
    ce, dist, loss = (np.concatenate(x, axis=1) for x in (ce, dist, loss))
    want = np.concatenate([ce.mean(1), dist.mean(1), loss.mean(1), [loss.sum(0).mean()]])
    assert_loss_close(mean, want, 1e-3, "means")
    log(f"[packed] workload {k}, every token: worst |dlogits err| {worst_g:.2e}, "
        f"worst mean scaled err {np.max(np.abs(mean - want) / np.maximum(1.0, np.abs(want))):.2e}")


@pytest.mark.parametrize("widths", [(64, 960), (64, 128)], ids=["one-wave-per-simd", "two-wg-per-cu"])
def test_packed_loss_large_scratch_partial_vocab(nel, widths):
    """V = 32,800 (not a multiple of 128: the last vocabulary tile's first
    wavefront holds 32 valid entries, the rest are dropped stores) and 34,816
    tokens, so that the scratch beyond a tile's first row spans more than
    2^31 bytes: a dropped store's lane offset (2^31) would land inside the
    buffer about 32,737 rows later if a store resource spanned to token n.
    The rows that such stores would hit are checked against the oracle (a
    student entry overwritten with -inf makes its Dist infinite), plus a few
    others; every sampled gradient row is finite and within the bar."""
    import torch
    V = 32800
    s = synth.make_suite(widths, V, 17, 2048, seed=91)
    n = s.n_tokens
    assert n * V * 2 > 2 ** 31 + 2 * 32768   # from row 0, column 32,768: past 2^31 bytes
    log(f"[packed] large scratch: n={n} V={V} widths={widths}")
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    mean, tok, dl = run_loss(nel, ds, 0.3, packed=pw)
    r = np.random.default_rng(92)
    danger = np.arange(32736, n)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, n - 1],
                                     r.choice(danger, size=120, replace=False),
                                     r.choice(32736, size=20, replace=False)]))
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, 0.3, 1.0, rows=rows)
    assert np.all(np.isfinite(tok[:, :, rows]))
    assert_loss_close(tok[:, 0, rows], ref["ce"], 1e-3, "CE")
    assert_loss_close(tok[:, 1, rows], ref["dist"], 1e-3, "Dist")
    assert_loss_close(tok[:, 2, rows], ref["loss"], 1e-3, "L")
    idx = torch.from_numpy(rows).cuda()
    for m in range(s.n_exits):
        got = to_np(dl[m].index_select(0, idx))
        assert np.all(np.isfinite(got))
        assert_grad_close(got, grads[m], 2e-2, f"dlogits exit {m}")
    assert np.all(np.isfinite(mean))
    del dl, ds, pw
    torch.cuda.empty_cache()
