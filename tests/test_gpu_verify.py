"""Greedy speculative verification on the GPU: exit heads + argmax and the
accepted prefix length, against the oracle.

How argmax parity is decided.  The heads kernel can return its own fp32
logits from the same launch that computes the argmax.  Then:
  1. the GPU argmax equals the argmax (lowest index on ties) of the GPU's own
     fp32 logits on every row -- bit-exact, whatever the rounding;
  2. those logits are within the order-aware accumulation bound of the exact
     (float64) logits on every entry;
  3. on every row whose exact top-2 margin exceeds twice the row's largest
     measured logit error, the GPU argmax equals the oracle's argmax: there no
     rounding the GPU actually did can change the order.  Only the rows left
     (exact near-ties, "exempt") may differ from the oracle, and for them 1
     and 2 already pin the result.
Acceptance is compared with the oracle's (computed from the oracle's own
argmax) on every sequence whose decisive positions are all non-exempt."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DevSuite, bf16_ulp, head_error_bound, head_error_bound_ordered, log,
                      to_np)

pytestmark = pytest.mark.gpu


def top2_margin(l: np.ndarray) -> np.ndarray:
    if l.shape[1] < 2:
        return np.full(l.shape[0], np.inf)
    srt = np.sort(l, axis=1)
    return srt[:, -1] - srt[:, -2]


def check_argmax(gpu_am, h, w, gpu_logits=None):
    """Returns the boolean exempt-row mask (see the module docstring).  Without
    the GPU's logits the order-aware bound stands in for the measured error."""
    h = np.asarray(h, np.float64)
    w = np.asarray(w, np.float64)
    l = oracle.heads([h], [w])[0]
    ref = oracle.argmax_lowest(l)
    bound = head_error_bound_ordered(h, w)
    if gpu_logits is not None:
        g = np.asarray(gpu_logits, np.float64)
        np.testing.assert_array_equal(gpu_am, oracle.argmax_lowest(g))
        err = np.abs(g - l)
        assert np.all(err <= bound + 1e-30), \
            f"logit error above the ordered bound: worst {np.max(err / (bound + 1e-30)):.3g} x"
        row_err = err.max(axis=1)
    else:
        row_err = bound.max(axis=1)
    amb = top2_margin(l) <= 2.0 * row_err
    assert np.array_equal(gpu_am[~amb], ref[~amb])
    if amb.any() and gpu_logits is None:
        rows = np.arange(l.shape[0])
        assert np.all(l[rows, ref][amb] - l[rows, gpu_am][amb] <= 2.0 * row_err[amb])
    return amb


def decisive_exempt(amb_d, amb_v, acc_ref, L):
    """Per sequence: is any position that decides the accepted length exempt?
    Positions 0 .. min(acc_ref, L - 1) decide it (the first mismatch ends it)."""
    B, P = amb_d.shape
    out = np.zeros(B, bool)
    for b in range(B):
        last = min(int(acc_ref[b]), L - 1)
        out[b] = bool(np.any(amb_d[b, :last + 1]) or np.any(amb_v[b, :last + 1]))
    return out


def check_acceptance(acc_gpu, am_gpu, l_draft, l_verify, amb, B, P, L=6):
    """acc_gpu against the oracle's acceptance from the oracle's own argmax on
    every sequence with no exempt decisive position; on every sequence against
    accept_prefix of the GPU argmax.  Returns the number of sequences compared
    with the oracle's argmax."""
    np.testing.assert_array_equal(
        acc_gpu, oracle.accept_prefix(am_gpu[0].reshape(B, P), am_gpu[1].reshape(B, P), L))
    want = oracle.accept_prefix(oracle.argmax_lowest(l_draft).reshape(B, P),
                                oracle.argmax_lowest(l_verify).reshape(B, P), L)
    skip = decisive_exempt(amb[0].reshape(B, P), amb[1].reshape(B, P), want, L)
    np.testing.assert_array_equal(acc_gpu[~skip], want[~skip])
    return int((~skip).sum())


def run_verify(nel, ds, s, packed):
    import torch
    if packed:
        pw = [nel.pack_weights(w) for w in ds.w]
        logits, am = nel.exit_heads_packed(ds.h, pw, want_logits=True, want_argmax=True)
        _, am_only = nel.exit_heads_packed(ds.h, pw, want_logits=False, want_argmax=True)
    else:
        logits, am = nel.exit_heads(ds.h, ds.w, want_logits=True, want_argmax=True)
        _, am_only = nel.exit_heads(ds.h, ds.w, want_logits=False, want_argmax=True)
    torch.cuda.synchronize()
    # the argmax does not depend on whether the logits are also written
    assert torch.equal(am, am_only)
    return [to_np(x) for x in logits], am.cpu().numpy()


@pytest.mark.parametrize("packed", [False, True], ids=["row-major", "packed"])
def test_verify_workload_102x7(nel, packed):
    import torch
    s = synth.make_workload(4)
    log(f"[verify] workload 4 ({'packed' if packed else 'row-major'}): B={s.batch} P={s.seq} "
        f"widths={s.widths} exits={s.exits}")
    ds = DevSuite(s, exits=s.exits)
    # junction 1 -> 2 on the draft's hidden state
    j = to_np(nel.junction(ds.h[0], ds.ids, ds.emb[1]))
    ref = oracle.junction(s.h[0], s.ids, s.emb[1])
    assert np.all(np.abs(j - ref) <= bf16_ulp(ref) + 1e-30)
    logits, am = run_verify(nel, ds, s, packed)
    amb = [check_argmax(am[i], s.h[m], s.w[m], logits[i]) for i, m in enumerate(s.exits)]
    B, P = s.batch, s.seq
    acc = nel.accept_prefix(torch.from_numpy(am[0].reshape(B, P)).cuda(),
                            torch.from_numpy(am[1].reshape(B, P)).cuda(), 6).cpu().numpy()
    l1, l3 = oracle.heads([s.h[0], s.h[2]], [s.w[0], s.w[2]])
    compared = check_acceptance(acc, am, l1, l3, amb, B, P)
    ordered = sum(int((top2_margin(l) <= 2.0 * head_error_bound_ordered(s.h[m], s.w[m]).max(axis=1)).sum())
                  for l, m in zip((l1, l3), s.exits))
    log(f"  exempt rows (measured error): exit 1 {int(amb[0].sum())}, exit 3 {int(amb[1].sum())} "
        f"of {B * P} each; under the ordered bound alone {ordered}; acceptance compared with the "
        f"oracle's argmax on {compared}/{B} sequences")
    assert compared >= B - 2


def test_packed_and_row_major_argmax_agree(nel):
    """Both GEMM paths at the verify shape: equal on every row that is exempt
    under neither path's measured error (both then equal the exact argmax)."""
    s = synth.make_workload(4)
    ds = DevSuite(s, exits=s.exits)
    lr, ar = run_verify(nel, ds, s, packed=False)
    lp, ap = run_verify(nel, ds, s, packed=True)
    n_cmp = 0
    for i, m in enumerate(s.exits):
        amb_r = check_argmax(ar[i], s.h[m], s.w[m], lr[i])
        amb_p = check_argmax(ap[i], s.h[m], s.w[m], lp[i])
        ok = ~(amb_r | amb_p)
        np.testing.assert_array_equal(ar[i][ok], ap[i][ok])
        n_cmp += int(ok.sum())
    log(f"[verify] packed vs row-major argmax equal on {n_cmp}/{2 * s.n_tokens} rows")
    assert n_cmp >= 2 * s.n_tokens - 4


def test_planted_agreement_all_lengths(nel):
    """Exit 3 computes exit 1's logits at planted positions, so greedy tokens agree
    there; accepted lengths 0..6 are drawn per sequence."""
    import torch
    r = np.random.default_rng(41)
    B, P, V = 64, 7, 4096
    s = synth.make_suite((256, 512, 768), V, B, P, seed=42)
    w3 = np.zeros_like(s.w[2])
    w3[:, :256] = s.w[0]
    s.w[2] = w3
    want_len = r.integers(0, 7, B)
    want_len[:7] = np.arange(7)
    h3 = s.h[2].reshape(B, P, 768).copy()
    h1 = s.h[0].reshape(B, P, 256)
    for b in range(B):
        h3[b, :want_len[b], :256] = h1[b, :want_len[b]]
    s.h[2] = h3.reshape(B * P, 768)
    ds = DevSuite(s, exits=(0, 2))
    logits, am = nel.exit_heads(ds.h, ds.w, want_logits=True, want_argmax=True)
    am = am.cpu().numpy()
    check_argmax(am[0], s.h[0], s.w[0], to_np(logits[0]))
    check_argmax(am[1], s.h[2], s.w[2], to_np(logits[1]))
    acc = nel.accept_prefix(torch.from_numpy(am[0].reshape(B, P)).cuda(),
                            torch.from_numpy(am[1].reshape(B, P)).cuda(), 6).cpu().numpy()
    np.testing.assert_array_equal(acc, np.minimum(want_len, 6))
    # fp32 logits output is within the accumulation bound of the exact logits
    for i, m in enumerate((0, 2)):
        l = oracle.heads([s.h[m]], [s.w[m]])[0]
        bound = head_error_bound(s.h[m], s.w[m])
        assert np.all(np.abs(to_np(logits[i]) - l) <= bound + 1e-30)


def test_argmax_exact_ties_take_lowest_index(nel):
    s = synth.make_suite((64, 128), 700, 1, 150, seed=43)
    for m in range(2):
        w = s.w[m]
        w[517] = w[3]          # exact ties between rows 3 and 517, and 130 / 640
        w[640] = w[130]
        w[200] = w[199]
    # make those rows win for some tokens: add a large common direction
    for m in range(2):
        for v in (3, 517, 130, 640, 199, 200):
            s.w[m][v] = synth.round_to_bf16(s.w[m][v] * 0 + s.h[m][:8].mean(0) * 0.05)
    ds = DevSuite(s)
    logits, am = nel.exit_heads(ds.h, ds.w, want_logits=True, want_argmax=True)
    am = am.cpu().numpy()
    for m in range(2):
        l = oracle.heads([s.h[m]], [s.w[m]])[0]
        ref = oracle.argmax_lowest(l)
        tied = np.isin(ref, [3, 130, 199])
        assert np.array_equal(am[m][tied], ref[tied])
        check_argmax(am[m], s.h[m], s.w[m], to_np(logits[m]))
