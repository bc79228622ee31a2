"""Largest-size case: 131,072 tokens (8x the benchmark batch) at the
500M/1.5B/3B suite's widths, so each exit's 16-bit logit-gradient buffer is
8 GiB and byte offsets into it pass 2^32.  Seeded synthetic operands drawn on
the device (same distributions as the benchmark: h ~ N(0, 4^2), heads ~
N(0, 0.02^2), uniform labels).

Checked against the oracle on sampled rows (the first, the last, the middle
and random ones): per-token losses (rel 1e-3), logit gradients (2e-2), the
means against the per-token values; then the grouped head backward on those
gradients: sampled rows of dh and sampled vocabulary rows of dW (a sum over
all 131,072 tokens, read K-major) against float64 products within the fp32
accumulation bound."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_grad_close, assert_loss_close, log, sample_rows, to_np

pytestmark = pytest.mark.gpu

N, V, WIDTHS = 131072, 32768, (1024, 2304, 4352)


def bound(a, b, K):
    return 2.0 * K * 2.0 ** -24 * (np.abs(a) @ np.abs(b))


def test_packed_loss_and_backward_131072_tokens(nel):
    import torch
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(71)
    log(f"[max] N={N} V={V} widths={WIDTHS}")
    hs = [(torch.randn(N, d, generator=gen, device=dev) * 4.0).bfloat16() for d in WIDTHS]
    ws = [(torch.randn(V, d, generator=gen, device=dev) * 0.02).bfloat16() for d in WIDTHS]
    labels = torch.randint(0, V, (N,), generator=gen, device=dev, dtype=torch.int32)
    pw = [nel.pack_weights(w) for w in ws]
    mean, tok, dl = nel.matryoshka_loss_packed(hs, pw, labels, alpha_d=0.3)
    torch.cuda.synchronize()
    log("[max] loss done")

    rows = sample_rows(N, 12, 72)
    ri = torch.from_numpy(rows).to(dev)
    w_np = [to_np(w) for w in ws]
    ref, grads = oracle.forward_tokens([to_np(h.index_select(0, ri)) for h in hs], w_np,
                                       labels.index_select(0, ri).cpu().numpy(), 0.3, 1.0)
    tok_np = to_np(tok)
    assert_loss_close(tok_np[:, 0, rows], ref["ce"], 1e-3, "CE")
    assert_loss_close(tok_np[:, 1, rows], ref["dist"], 1e-3, "Dist")
    assert_loss_close(tok_np[:, 2, rows], ref["loss"], 1e-3, "L")
    for m in range(len(WIDTHS)):
        err = assert_grad_close(to_np(dl[m].index_select(0, ri)), grads[m], 2e-2, f"dlogits {m}")
        log(f"  exit {m}: max |dlogits err| {err:.2e}")
    want = np.concatenate([tok_np[:, 0].mean(1), tok_np[:, 1].mean(1), tok_np[:, 2].mean(1),
                           [tok_np[:, 2].sum(0).mean()]])
    np.testing.assert_allclose(to_np(mean), want, rtol=2e-6, atol=1e-6)

    dhs, dws = nel.heads_backward(dl, hs, ws)
    torch.cuda.synchronize()
    log("[max] backward done")
    m = len(WIDTHS) - 1
    g_rows = to_np(dl[m].index_select(0, ri))
    ref_dh = g_rows @ w_np[m]
    b = bound(g_rows, w_np[m], V)
    got_dh = to_np(dhs[m].index_select(0, ri))
    assert np.all(np.abs(got_dh - ref_dh) <= 2.0 ** -8 * (np.abs(ref_dh) + b) + b), "dh"
    cols = sample_rows(V, 6, 73)
    ci = torch.from_numpy(cols).to(dev)
    g_cols = to_np(dl[m].index_select(1, ci))          # [N, cols]
    h = to_np(hs[m])
    ref_dw = g_cols.T @ h
    got_dw = to_np(dws[m].index_select(0, ci))
    assert np.all(np.abs(got_dw - ref_dw) <= bound(g_cols.T, h, N)), "dW"
