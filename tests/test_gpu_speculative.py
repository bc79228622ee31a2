"""Sampled speculative verification (nel_speculative_verify) against the oracle.

Both sides read the same fp32 logits (written by the test).  The kernel takes
its decisions in fp32, the oracle in fp64.  A decision on a sequence's path
whose fp64 margin is below what the kernel's rounding can move (2e-6 of the
mass for where the nucleus ends, 1e-5 relative for a tie at its edge or an
accept comparison, 1e-6 of the total for a draw boundary; the kernel sums the
masses from per-thread fp32 partials of 32 terms combined in fp64, and the
draw in fp64)
is "borderline": either outcome is accepted there, and the sequence is checked
for validity instead of equality.  beta is compared to 2e-5."""
import numpy as np
import pytest

import oracle
from gpu_util import log

pytestmark = pytest.mark.gpu

EDGE = 1e-5     # relative: a tie at the nucleus edge, the accept comparison
MASS = 2e-6     # of the mass: where the nucleus ends
DRAW = 1e-6     # of the total weight: a draw boundary


def draft_tokens(dl, T, tp, r):
    """Tokens drawn from the draft exit's own distributions (as a drafter would)."""
    B, P, V = dl.shape
    p = oracle.nucleus(dl, T, tp)
    tok = np.zeros((B, P), dtype=np.int32)
    for b in range(B):
        for i in range(P):
            tok[b, i] = oracle.sample_inverse_cdf(p[b, i], r.random())
    return tok


def nucleus_edge_is_close(row, T, tp):
    if tp >= 1.0:
        return False
    pr = oracle.softmax(row.astype(np.float64) / T)
    srt = np.sort(pr)[::-1]
    c = np.cumsum(srt)
    k = min(int(np.searchsorted(c, tp)), srt.size - 1)
    near_mass = abs(c[k] - tp) < MASS or (k > 0 and abs(c[k - 1] - tp) < MASS)
    near_tie = k + 1 < srt.size and srt[k + 1] > srt[k] * (1 - EDGE) and srt[k + 1] < srt[k]
    return near_mass or near_tie


def borderline(dl, vl, tok, ua, un, L, T, tp):
    """Per sequence: does any decision on its (oracle) path sit within rounding of flipping?"""
    B, P, V = dl.shape
    out = np.zeros(B, bool)
    for b in range(B):
        p = oracle.nucleus(dl[b, :L + 1], T, tp)
        q = oracle.nucleus(vl[b, :L + 1], T, tp)
        k = 0
        while True:
            out[b] |= nucleus_edge_is_close(dl[b, k], T, tp) or nucleus_edge_is_close(vl[b, k], T, tp)
            if k >= L:
                break
            x = tok[b, k]
            lhs, rhs = ua[b, k] * p[k, x], q[k, x]
            if abs(lhs - rhs) <= EDGE * max(lhs, rhs, 1e-30):
                out[b] = True
            if not lhs < rhs:
                break
            k += 1
        w = np.maximum(q[k] - p[k], 0.0) if k < L else q[L]
        if k < L and w.sum() <= 0:
            w = q[k]
        c = np.cumsum(w)
        t = un[b] * c[-1]
        j = int(np.searchsorted(c, t, side="right"))
        if (j < V and abs(c[j] - t) < DRAW * c[-1]) or (j > 0 and abs(c[j - 1] - t) < DRAW * c[-1]):
            out[b] = True
    return out


def run(nel, dl, vl, tok, ua, un, L, T, tp):
    import torch
    dev = "cuda:0"
    beta, acc, nxt = nel.speculative_verify(torch.from_numpy(dl).to(dev), torch.from_numpy(vl).to(dev),
                                            torch.from_numpy(tok).to(dev), torch.from_numpy(ua).to(dev),
                                            torch.from_numpy(un).to(dev), L, temperature=T, top_p=tp)
    torch.cuda.synchronize()
    return beta.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()


def check(nel, dl, vl, tok, ua, un, L, T, tp):
    beta, acc, nxt = run(nel, dl, vl, tok, ua, un, L, T, tp)
    rb, ra, rn = oracle.speculative_verify(dl, vl, tok, ua, un, L, T, tp)
    amb = borderline(dl, vl, tok, ua, un, L, T, tp)
    if L > 0:
        # positions with a borderline nucleus edge may keep one more or one
        # fewer entry on either side: there beta may move by that entry's mass
        close = np.array([[nucleus_edge_is_close(dl[b, i], T, tp) or
                           nucleus_edge_is_close(vl[b, i], T, tp) for i in range(L)]
                          for b in range(dl.shape[0])])
        tol = np.where(close, 1e-3, 2e-5)
        assert np.all(np.abs(beta - rb) <= tol), f"beta: worst {np.max(np.abs(beta - rb) / tol):.3g} x tol"
    assert np.array_equal(acc[~amb], ra[~amb])
    assert np.array_equal(nxt[~amb], rn[~amb])
    # borderline sequences: a valid outcome (accepted length in range, a
    # next token of positive weight under the GPU's own accepted length)
    for b in np.nonzero(amb)[0]:
        assert 0 <= acc[b] <= L
        k = acc[b]
        p = oracle.nucleus(dl[b, k], T, tp)
        q = oracle.nucleus(vl[b, k], T, tp)
        w = np.maximum(q - p, 0.0) if k < L else q
        assert w[nxt[b]] > 0 or q[nxt[b]] > 0
    return int(amb.sum()), acc


@pytest.mark.parametrize("T,tp", [(1.0, 0.9), (0.7, 1.0), (1.3, 0.5)])
def test_speculative_small(nel, T, tp):
    r = np.random.default_rng(81)
    B, P, V, L = 48, 7, 1000, 6
    dl = (r.standard_normal((B, P, V)) * 2.0).astype(np.float32)
    vl = (dl + r.standard_normal((B, P, V)) * 1.0).astype(np.float32)
    tok = draft_tokens(dl, T, tp, r)
    ua = r.random((B, P)).astype(np.float32)
    un = r.random(B).astype(np.float32)
    amb, acc = check(nel, dl, vl, tok, ua, un, L, T, tp)
    log(f"[spec] T={T} top_p={tp}: accepted mean {acc.mean():.2f}, borderline sequences {amb}/{B}")
    assert amb <= B // 4


def test_speculative_verify_workload_shape(nel):
    """102 sequences x 7 positions, V = 32768, draft length 6: logits of exits 1
    and 3 of the verify workload computed by the oracle (fp64, rounded to fp32).
    Random heads are unrelated, so the verifier's logits are mixed with the
    draft's (as in a trained suite, where the exits agree) to exercise acceptance."""
    import synth
    s = synth.make_workload(4)
    l1, l3 = oracle.heads([s.h[0], s.h[2]], [s.w[0], s.w[2]])
    B, P, V, L = s.batch, s.seq, s.vocab, 6
    dl = l1.astype(np.float32).reshape(B, P, V)
    vl = (l1 + 0.25 * l3).astype(np.float32).reshape(B, P, V)
    r = np.random.default_rng(82)
    tok = draft_tokens(dl, 1.0, 0.9, r)
    ua = r.random((B, P)).astype(np.float32)
    un = r.random(B).astype(np.float32)
    amb, acc = check(nel, dl, vl, tok, ua, un, L, 1.0, 0.9)
    log(f"[spec] verify workload: accepted mean {acc.mean():.2f}, borderline {amb}/{B}")
    # ~3300-entry nuclei of ~3e-5 each: where top_p falls within 2e-6 of a
    # step is common over up to 14 rows per path; at least half must compare exactly
    assert amb <= B // 2


def test_speculative_greedy_limit(nel):
    r = np.random.default_rng(83)
    B, P, V, L = 40, 7, 500, 6
    dl = (r.standard_normal((B, P, V)) * 3).astype(np.float32)
    vl = (dl + r.standard_normal((B, P, V)) * 0.5).astype(np.float32)
    tok = oracle.argmax_lowest(dl).astype(np.int32)
    _, acc, nxt = run(nel, dl, vl, tok, r.random((B, P)).astype(np.float32),
                      r.random(B).astype(np.float32), L, 1e-4, 1.0)
    vt = oracle.argmax_lowest(vl)
    np.testing.assert_array_equal(acc, oracle.accept_prefix(tok, vt, L))
    np.testing.assert_array_equal(nxt, vt[np.arange(B), acc])


def test_speculative_edges(nel):
    import torch
    r = np.random.default_rng(84)
    B, P, V = 8, 3, 77
    dl = (r.standard_normal((B, P, V))).astype(np.float32)
    vl = (r.standard_normal((B, P, V))).astype(np.float32)
    ua = r.random((B, P)).astype(np.float32)
    un = r.random(B).astype(np.float32)
    # draft length 0: nothing to accept, the next token is drawn from q at position 0
    tok = np.zeros((B, P), np.int32)
    check(nel, dl, vl, tok, ua, un, 0, 1.0, 1.0)
    # a drafted token outside the vocabulary is rejected and flagged
    tok = draft_tokens(dl, 1.0, 1.0, r)
    tok[2, 0] = V
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    dev = "cuda:0"
    _, acc, _ = nel.speculative_verify(torch.from_numpy(dl).to(dev), torch.from_numpy(vl).to(dev),
                                       torch.from_numpy(tok).to(dev), torch.from_numpy(ua).to(dev),
                                       torch.from_numpy(un).to(dev), 2, flags=flags)
    assert int(acc[2]) == 0
    assert nel.read_flags(flags) == nel.FLAG_BAD_ID
