"""The sampled-verification validity check of test_gpu_speculative (used on
the GPU's outcomes) is itself tested here, on the CPU: per-row statistics are
produced the kernel's way in NumPy float32 (exp of the fp32 difference, the
nucleus threshold as the smallest kept value), the oracle's own outcome must
pass, and planting a mistake in it -- the next token moved by one entry, one
accept more or one fewer -- must fail."""
import numpy as np
import pytest

import oracle
import test_gpu_speculative as spec


def emulated_stats(l, T, tp):
    """[B, P, 4] row statistics as the kernel defines them (nel.h)."""
    B, P, V = l.shape
    st = np.zeros((B, P, 4))
    inv_t = np.float32(1) / np.float32(T)
    for b in range(B):
        for i in range(P):
            sc = l[b, i].astype(np.float32) * inv_t
            mx = sc.max()
            e = np.exp((sc - mx).astype(np.float32).astype(np.float64)).astype(np.float32)
            S = e.astype(np.float64).sum()
            if tp >= 1:
                thr, kept = 0.0, e
            else:
                srt = np.sort(e)[::-1].astype(np.float64)
                k = min(int(np.searchsorted(np.cumsum(srt), tp * S)), V - 1)
                thr = float(srt[k])
                kept = e[e >= thr]
            st[b, i] = (mx, kept.astype(np.float64).sum(), thr, S)
    return st


@pytest.mark.parametrize("T,tp", [(1.0, 0.9), (0.7, 1.0), (1.3, 0.5)])
def test_validity_check_accepts_the_definition_and_rejects_mistakes(T, tp):
    r = np.random.default_rng(91)
    B, P, V, L = 16, 7, 600, 6
    dl = (r.standard_normal((B, P, V)) * 2.0).astype(np.float32)
    vl = (dl + r.standard_normal((B, P, V)) * 1.0).astype(np.float32)
    tok = spec.draft_tokens(dl, T, tp, r)
    ua = r.random((B, P)).astype(np.float32)
    un = r.random(B).astype(np.float32)
    _, acc, nxt = oracle.speculative_verify(dl, vl, tok, ua, un, L, T, tp)
    stats = np.stack([emulated_stats(dl, T, tp), emulated_stats(vl, T, tp)])
    spec.check_valid(dl, vl, tok, ua, un, L, T, tp, acc, nxt, stats)
    planted = caught = 0
    for b in range(B):
        for kind in ("next", "more", "fewer"):
            a2, n2 = acc.copy(), nxt.copy()
            if kind == "next":
                n2[b] = (nxt[b] + 1) % V
            elif kind == "more" and acc[b] < L:
                a2[b] += 1
            elif kind == "fewer" and acc[b] > 0:
                a2[b] -= 1
            else:
                continue
            planted += 1
            try:
                spec.check_valid(dl, vl, tok, ua, un, L, T, tp, a2, n2, stats)
            except AssertionError:
                caught += 1
    assert caught == planted, f"{planted - caught} of {planted} planted mistakes passed"
