"""Sampled speculative verification (nel_speculative_verify) against the oracle.

Both sides read the same fp32 logits (written by the test).  The kernel takes
its decisions in fp32, the oracle in fp64.  A decision on a sequence's path
whose fp64 margin is below what the kernel's rounding can move (2e-6 of the
mass for where the nucleus ends, 1e-5 relative for a tie at its edge or an
accept comparison, 1e-6 of the total for a draw boundary; the kernel sums the
masses from per-thread fp32 partials of 32 terms combined in fp64, and the
draw in fp64)
is "borderline": either outcome is accepted there.  Every sequence, borderline
or not, is then checked for validity step by step from the GPU's own per-row
statistics (check_valid below): the nucleus threshold reaches top_p and is the
largest that does, every accept and the first reject agree with the float64
comparison u p(x) < q(x) up to the kernel's rounding, and the next token sits
where the running sum of the draw's weights crosses u times their total.
beta is compared to 2e-5."""
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


def run(nel, dl, vl, tok, ua, un, L, T, tp, want_stats=False):
    import torch
    dev = "cuda:0"
    B = tok.shape[0]
    ws = torch.zeros(max(int(nel.load().nel_speculative_workspace(B, L)), 256), dtype=torch.uint8,
                     device=dev)
    beta, acc, nxt = nel.speculative_verify(torch.from_numpy(dl).to(dev), torch.from_numpy(vl).to(dev),
                                            torch.from_numpy(tok).to(dev), torch.from_numpy(ua).to(dev),
                                            torch.from_numpy(un).to(dev), L, temperature=T, top_p=tp,
                                            workspace=ws)
    torch.cuda.synchronize()
    out = (beta.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy())
    if want_stats:
        out += (nel.speculative_row_stats(ws, B, L).cpu().numpy().astype(np.float64),)
    return out


# ---------------------------------------------------------------- validity
# The GPU's outcome on a sequence is valid if it is what the definition gives
# for some admissible rounding of the kernel's fp32 arithmetic.  The check
# replays the kernel's steps in float64 from the GPU's own per-row statistics
# (row max, nucleus mass, threshold), carrying an interval for every value the
# kernel rounds:
#   e_v = exp(fl(l_v / T) - max): the scaled logit and the difference are
#     exact fp32 operations (replayed exactly); exp is the base-2 hardware
#     exponential of an fp32 product, relative error <= (|d| + 4) 2^-23;
#   membership e_v >= threshold is decided unless e_v is within that error of it;
#   p_v = e_v / mass, with one more rounding.

def _row(l_row, T, st, tp):
    """float64 model of one row: (e, err, status, mass, threshold); status is
    +1 kept, -1 dropped, 0 undecided.  Also checks the row statistics."""
    inv_t = np.float32(1.0) / np.float32(T)
    sc = np.asarray(l_row, np.float32) * inv_t                  # fl(l / T)
    mx = np.float32(st[0])
    assert mx == sc.max(), "row max"
    d = (sc - mx).astype(np.float32).astype(np.float64)         # fl(sc - mx), as the kernel
    e = np.exp(d)
    rel = (np.abs(d) + 4.0) * 2.0 ** -23
    thr = float(st[2])
    total = e.sum()
    assert abs(st[3] - total) <= 1e-5 * total, "softmax mass"
    if tp >= 1.0:
        assert thr == 0.0, "top_p = 1 keeps every entry"
        status = np.ones(e.size, np.int8)
    else:
        status = np.where(e * (1 - rel) >= thr, 1, np.where(e * (1 + rel) < thr, -1, 0)).astype(np.int8)
        need = tp * total
        tol = MASS * total + float(np.max(rel[status >= 0] * e[status >= 0], initial=0.0)) * 4
        # the GPU set reaches top_p, and no strictly smaller set above the threshold does
        upper = e[status >= 0].sum()
        assert upper >= need - tol, f"nucleus below top_p: {upper / total:.7f} < {tp}"
        above = e[e * (1 - rel) > thr].sum()
        assert above < need + tol, f"threshold not the largest: {above / total:.7f} >= {tp}"
    mass = float(st[1])
    status = _resolve_by_mass(d, e, rel, status, mass, total)
    kept = e[status > 0].sum()
    und = e[status == 0].sum()
    assert abs(mass - kept) <= und + 1e-5 * total, "nucleus mass"
    return e, rel, status, mass


def _resolve_by_mass(d, e, rel, status, mass, total):
    """Decide the entries within rounding of the threshold from the GPU's own
    nucleus mass.  The kernel's e_v grows with the exactly replayed d_v, so the
    entries it kept among the undecided ones are those with the largest d (equal
    d, equal decision): the prefix whose mass matches the reported one.  Left
    undecided unless exactly one prefix matches."""
    und = np.nonzero(status == 0)[0]
    if und.size == 0:
        return status
    order = und[np.argsort(-d[und], kind="stable")]
    # prefix sizes that do not split entries of equal d
    cuts = [0] + [j for j in range(1, order.size + 1)
                  if j == order.size or d[order[j]] != d[order[j - 1]]]
    base = e[status > 0].sum()
    csum = np.concatenate([[0.0], np.cumsum(e[order])])
    tol = 4e-6 * total + float(np.sum((e * rel)[status >= 0]))
    fits = [j for j in cuts if abs(base + csum[j] - mass) <= tol]
    if len(fits) != 1:
        return status
    out = status.copy()
    out[order[:fits[0]]] = 1
    out[order[fits[0]:]] = -1
    return out


def _prob_interval(e, rel, status, mass):
    """Bounds of the GPU's fp32 probability of every entry."""
    r = rel + 2.0 ** -22
    hi = np.where(status >= 0, e / mass * (1 + r), 0.0)
    lo = np.where(status > 0, e / mass * (1 - r), 0.0)
    return lo, hi


def check_valid(dl, vl, tok, ua, un, L, T, tp, acc, nxt, stats):
    """Every sequence's accepted length and next token are reachable by the
    definition under the kernel's rounding (see above).  Returns nothing; fails
    with the sequence and step that is not."""
    B = dl.shape[0]
    for b in range(B):
        k = int(acc[b])
        assert 0 <= k <= L, f"seq {b}: accepted {k}"
        rows_p = [_row(dl[b, i], T, stats[0, b, i], tp) for i in range(k + 1)]
        rows_q = [_row(vl[b, i], T, stats[1, b, i], tp) for i in range(k + 1)]
        # the acceptance chain: accepted at i < k, rejected at k (if k < L)
        for i in range(min(k + 1, L)):
            x = int(tok[b, i])
            pl, ph = _prob_interval(*rows_p[i])
            ql, qh = _prob_interval(*rows_q[i])
            u = float(ua[b, i])
            can_accept = u * pl[x] * (1 - 2.0 ** -23) < qh[x]
            can_reject = not (u * ph[x] * (1 + 2.0 ** -23) < ql[x])
            if i < k:
                assert can_accept, f"seq {b}: position {i} accepted, but u p(x) >= q(x)"
            else:
                assert can_reject, f"seq {b}: position {i} rejected, but u p(x) < q(x)"
        # the draw at k from the residual (k < L; q if the residual is 0) or from q
        ql, qh = _prob_interval(*rows_q[k])
        cands = []
        if k < L:
            pl, ph = _prob_interval(*rows_p[k])
            wl = np.maximum(ql - ph, 0.0)
            wh = np.maximum(qh - pl, 0.0)
            if wh.sum() > 0:
                cands.append((wl, wh))
            if wl.sum() == 0:
                cands.append((ql, qh))
        else:
            cands.append((ql, qh))
        n = int(nxt[b])
        ok = False
        for wl, wh in cands:
            u = float(un[b])
            before_lo = wl[:n].sum()
            through_hi = wh[:n + 1].sum()
            tot_lo, tot_hi = wl.sum(), wh.sum()
            slack = DRAW * tot_hi
            ok |= bool(wh[n] > 0 and before_lo <= u * tot_hi + slack and through_hi > u * tot_lo - slack)
        assert ok, f"seq {b}: next token {n} is not where the running sum crosses u times the total"


def check(nel, dl, vl, tok, ua, un, L, T, tp):
    beta, acc, nxt, stats = run(nel, dl, vl, tok, ua, un, L, T, tp, want_stats=True)
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
    # sequences with no decision near a rounding boundary: equal to the oracle
    assert np.array_equal(acc[~amb], ra[~amb])
    assert np.array_equal(nxt[~amb], rn[~amb])
    # every sequence (borderline or not): each step of the GPU's own path is valid
    check_valid(dl, vl, tok, ua, un, L, T, tp, acc, nxt, stats)
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
    log(f"[spec] T={T} top_p={tp}: accepted mean {acc.mean():.2f}, borderline sequences {amb}/{B} "
        f"(compared for validity step by step)")


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
    # ~3300-entry nuclei of ~3e-5 each: where top_p falls within 2e-6 of a
    # step is common over up to 14 rows per path; every sequence is checked
    # for validity step by step, the others are also equal to the oracle
    log(f"[spec] verify workload: accepted mean {acc.mean():.2f}, borderline {amb}/{B} "
        f"(compared for validity step by step)")


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
