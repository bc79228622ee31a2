"""Backward of one exit head (nel_head_backward) against the oracle:
dH = G W (bf16 output) and dW = G^T h (fp32 output), G = the logit gradients.

Bars: fp32 accumulation in any order is within gamma_K * (|A| |B|) of the
exact product (products of bf16 values are exact in fp32), with
gamma_K = 2 K 2^-24; the bf16 output adds half an ulp (2^-8 relative)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev_tensor, log, to_np

pytestmark = pytest.mark.gpu


def bound(a, b, K):
    return 2.0 * K * 2.0 ** -24 * (np.abs(a) @ np.abs(b))


def check(nel, g, h, w, want_dh=True, want_dw=True):
    import torch
    G, H, W = dev_tensor(g, "bf16"), dev_tensor(h, "bf16"), dev_tensor(w, "bf16")
    dh, dw = nel.head_backward(G, H, W, want_dh=want_dh, want_dw=want_dw)
    torch.cuda.synchronize()
    ref_dh, ref_dw = oracle.head_backward(g, h, w)
    n, V = g.shape
    if want_dh:
        got = to_np(dh)
        b = bound(g, w, V)
        tol = 2.0 ** -8 * (np.abs(ref_dh) + b) + b + 1e-30
        assert np.all(np.abs(got - ref_dh) <= tol), f"dh: worst {np.max(np.abs(got - ref_dh) / tol):.3g} x bound"
    else:
        assert dh is None
    if want_dw:
        got = to_np(dw)
        tol = bound(g.T, h, n) + 1e-30
        assert np.all(np.abs(got - ref_dw) <= tol), f"dw: worst {np.max(np.abs(got - ref_dw) / tol):.3g} x bound"
    else:
        assert dw is None


def oracle_gradients(widths, V, B, S, seed):
    """A suite and the oracle's bf16-rounded logit gradients of every exit."""
    s = synth.make_suite(widths, V, B, S, seed=seed)
    g = oracle.matryoshka_grad(oracle.heads(s.h, s.w), s.labels, 0.3)
    return s, [synth.round_to_bf16(gm.astype(np.float32)) for gm in g]


CASES = [
    # widths (all multiples of 64), V, batch, seq: ragged token counts, d below and
    # above one 256-row tile, a vocabulary of one K step
    ("3exit-ragged", (64, 128, 192), 1024, 3, 100, 61),
    ("partial-A-tile", (320,), 512, 1, 129, 62),
    ("tiny-vocab", (64, 128), 64, 1, 65, 63),
    ("one-token", (128,), 256, 1, 1, 64),
    # V % 128 == 64: dW's last 128-entry B tile half outside the vocabulary
    ("partial-B-tile", (192, 256), 576, 2, 77, 65),
]


@pytest.mark.parametrize("name,widths,V,B,S,seed", CASES, ids=[c[0] for c in CASES])
def test_head_backward_small(nel, name, widths, V, B, S, seed):
    s, g = oracle_gradients(widths, V, B, S, seed)
    log(f"[bwd] {name}: n={s.n_tokens} V={V} widths={widths}")
    for m in range(s.n_exits):
        check(nel, g[m], s.h[m], s.w[m])


def test_head_backward_single_outputs(nel):
    s, g = oracle_gradients((128, 256), 512, 2, 70, 65)
    check(nel, g[1], s.h[1], s.w[1], want_dh=True, want_dw=False)
    check(nel, g[0], s.h[0], s.w[0], want_dh=False, want_dw=True)


def test_head_backward_no_tokens_zeroes_dw(nel):
    import torch
    V, d = 128, 64
    G = torch.empty(0, V, dtype=torch.bfloat16, device="cuda:0")
    H = torch.empty(0, d, dtype=torch.bfloat16, device="cuda:0")
    W = torch.ones(V, d, dtype=torch.bfloat16, device="cuda:0")
    dw = torch.full((V, d), 7.0, dtype=torch.float32, device="cuda:0")
    _, out = nel.head_backward(G, H, W, want_dh=False, dw=dw)
    assert float(out.abs().max()) == 0.0


def test_head_backward_full_size_sampled(nel):
    """The benchmark's largest exit (n = 16384, V = 32768, d = 4352) on seeded
    synthetic inputs; sampled rows of dH and of dW against the oracle."""
    import torch
    n, V, d = 16384, 32768, 4352
    r = np.random.default_rng(66)
    h = synth.round_to_bf16((r.standard_normal((n, d), dtype=np.float32) * 4.0))
    w = synth.round_to_bf16((r.standard_normal((V, d), dtype=np.float32) * 0.02))
    g = np.empty((n, V), dtype=np.float32)
    for i in range(0, n, 2048):
        g[i:i + 2048] = synth.round_to_bf16(r.standard_normal((min(2048, n - i), V), dtype=np.float32) * 1e-3)
    log(f"[bwd] full size n={n} V={V} d={d}")
    G, H, W = dev_tensor(g, "bf16"), dev_tensor(h, "bf16"), dev_tensor(w, "bf16")
    dh, dw = nel.head_backward(G, H, W)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, n - 1], r.choice(n, 13, replace=False)]))
    cols = np.unique(np.concatenate([[0, V - 1], r.choice(V, 14, replace=False)]))
    got_dh = to_np(dh[torch.from_numpy(rows).cuda()])
    ref_dh = g[rows].astype(np.float64) @ w.astype(np.float64)
    b = bound(g[rows], w, V)
    tol = 2.0 ** -8 * (np.abs(ref_dh) + b) + b
    assert np.all(np.abs(got_dh - ref_dh) <= tol)
    got_dw = to_np(dw[torch.from_numpy(cols).cuda()])
    ref_dw = g[:, cols].T.astype(np.float64) @ h.astype(np.float64)
    assert np.all(np.abs(got_dw - ref_dw) <= bound(g[:, cols].T, h, n))


# ------------------------------------------------ every exit in one grouped call
def grouped_vs_per_exit(nel, g, hs, ws, want_dh=True, want_dw=True):
    """nel_heads_backward and nel_head_backward per exit on the same device
    operands: every output bit-identical (the same tiles and K order)."""
    import torch
    G = [dev_tensor(x, "bf16") for x in g]
    H = [dev_tensor(x, "bf16") for x in hs]
    W = [dev_tensor(x, "bf16") for x in ws]
    dhs, dws = nel.heads_backward(G, H, W, want_dh=want_dh, want_dw=want_dw)
    for m in range(len(H)):
        dh1, dw1 = nel.head_backward(G[m], H[m], W[m], want_dh=want_dh, want_dw=want_dw)
        torch.cuda.synchronize()
        if want_dh:
            assert torch.equal(dhs[m].view(torch.int16), dh1.view(torch.int16)), f"dh[{m}]"
        else:
            assert dhs is None
        if want_dw:
            assert torch.equal(dws[m].view(torch.int32), dw1.view(torch.int32)), f"dw[{m}]"
        else:
            assert dws is None
    return dhs, dws


@pytest.mark.parametrize("name,widths,V,B,S,seed", CASES, ids=[c[0] for c in CASES])
def test_heads_backward_grouped_small(nel, name, widths, V, B, S, seed):
    s, g = oracle_gradients(widths, V, B, S, seed)
    log(f"[bwd-group] {name}: n={s.n_tokens} V={V} widths={widths}")
    dhs, dws = grouped_vs_per_exit(nel, g, s.h, s.w)
    n = s.n_tokens
    for m in range(s.n_exits):
        ref_dh, ref_dw = oracle.head_backward(g[m], s.h[m], s.w[m])
        b = bound(g[m], s.w[m], V)
        tol = 2.0 ** -8 * (np.abs(ref_dh) + b) + b + 1e-30
        assert np.all(np.abs(to_np(dhs[m]) - ref_dh) <= tol)
        assert np.all(np.abs(to_np(dws[m]) - ref_dw) <= bound(g[m].T, s.h[m], n) + 1e-30)


def test_heads_backward_grouped_single_outputs(nel):
    s, g = oracle_gradients((128, 256, 320), 512, 2, 70, 67)
    grouped_vs_per_exit(nel, g, s.h, s.w, want_dh=True, want_dw=False)
    grouped_vs_per_exit(nel, g, s.h, s.w, want_dh=False, want_dw=True)


def test_heads_backward_grouped_no_tokens_zeroes_dw(nel):
    import torch
    V = 128
    G = [torch.empty(0, V, dtype=torch.bfloat16, device="cuda:0") for _ in range(2)]
    H = [torch.empty(0, d, dtype=torch.bfloat16, device="cuda:0") for d in (64, 192)]
    W = [torch.ones(V, d, dtype=torch.bfloat16, device="cuda:0") for d in (64, 192)]
    dws = [torch.full((V, d), 7.0, dtype=torch.float32, device="cuda:0") for d in (64, 192)]
    _, out = nel.heads_backward(G, H, W, want_dh=False, dws=dws)
    assert all(float(x.abs().max()) == 0.0 for x in out)


def test_heads_backward_grouped_full_size(nel):
    """The benchmark's three exits (n = 16384, V = 32768, widths 1024 / 2304 /
    4352) on seeded synthetic operands: the grouped call against the per-exit
    call, bit for bit, and sampled rows of the widest exit against the oracle."""
    import torch
    n, V, D = 16384, 32768, (1024, 2304, 4352)
    log(f"[bwd-group] full size n={n} V={V} widths={D}")
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(68)
    G = [(torch.randn(n, V, generator=gen, device="cuda:0") * 1e-3).bfloat16() for _ in D]
    H = [(torch.randn(n, d, generator=gen, device="cuda:0") * 4.0).bfloat16() for d in D]
    W = [(torch.randn(V, d, generator=gen, device="cuda:0") * 0.02).bfloat16() for d in D]
    dhs, dws = nel.heads_backward(G, H, W)
    for m in range(3):
        dh1, dw1 = nel.head_backward(G[m], H[m], W[m])
        torch.cuda.synchronize()
        assert torch.equal(dhs[m].view(torch.int16), dh1.view(torch.int16)), f"dh[{m}]"
        assert torch.equal(dws[m].view(torch.int32), dw1.view(torch.int32)), f"dw[{m}]"
        del dh1, dw1
    r = np.random.default_rng(69)
    rows = np.unique(np.concatenate([[0, n - 1], r.choice(n, 6, replace=False)]))
    cols = np.unique(np.concatenate([[0, V - 1], r.choice(V, 6, replace=False)]))
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    g_rows = to_np(G[2][ri])                      # [rows, V]
    g_cols = to_np(G[2][:, ci].contiguous())      # [n, cols]
    h, w = to_np(H[2]), to_np(W[2])
    ref_dh = oracle.head_backward(g_rows, h[:len(rows)], w)[0]
    b = bound(g_rows, w, V)
    assert np.all(np.abs(to_np(dhs[2][ri]) - ref_dh) <= 2.0 ** -8 * (np.abs(ref_dh) + b) + b)
    ref_dw = g_cols.T @ h
    assert np.all(np.abs(to_np(dws[2][ci]) - ref_dw) <= bound(g_cols.T, h, n))
