"""Greedy speculative verification on the GPU: exit heads + argmax and the
accepted prefix length, against the oracle (bit-exact where the argmax is
unique in exact arithmetic)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DevSuite, bf16_ulp, head_error_bound, log, to_np

pytestmark = pytest.mark.gpu


def check_argmax(gpu_am, h, w):
    """GPU argmax equals the exact argmax wherever the exact top-2 margin exceeds
    the fp32 accumulation bound; elsewhere the GPU's pick must be within the
    bound of the maximum.  Returns the number of such ambiguous rows."""
    l = oracle.heads([h], [w])[0]
    ref = oracle.argmax_lowest(l)
    bound = head_error_bound(np.asarray(h, np.float64), np.asarray(w, np.float64))
    srt = np.sort(l, axis=1)
    margin = srt[:, -1] - srt[:, -2] if l.shape[1] > 1 else np.full(l.shape[0], np.inf)
    rows = np.arange(l.shape[0])
    amb = margin <= 2 * bound[rows, ref]
    assert np.array_equal(gpu_am[~amb], ref[~amb])
    if amb.any():
        mx = l[rows, ref]
        pick = l[rows, gpu_am]
        assert np.all(mx[amb] - pick[amb] <= 2 * bound[rows, ref][amb])
    return int(amb.sum())


def test_verify_workload_102x7(nel):
    import torch
    s = synth.make_workload(4)
    log(f"[verify] workload 4: B={s.batch} P={s.seq} widths={s.widths} exits={s.exits}")
    ds = DevSuite(s, exits=s.exits)
    # junction 1 -> 2 on the draft's hidden state
    j = to_np(nel.junction(ds.h[0], ds.ids, ds.emb[1]))
    ref = oracle.junction(s.h[0], s.ids, s.emb[1])
    assert np.all(np.abs(j - ref) <= bf16_ulp(ref) + 1e-30)
    _, am = nel.exit_heads(ds.h, ds.w, want_logits=False, want_argmax=True)
    am = am.cpu().numpy()
    amb = 0
    for i, m in enumerate(s.exits):
        amb += check_argmax(am[i], s.h[m], s.w[m])
    log(f"  ambiguous argmax rows: {amb}")
    B, P = s.batch, s.seq
    acc = nel.accept_prefix(torch.from_numpy(am[0].reshape(B, P)).cuda(),
                            torch.from_numpy(am[1].reshape(B, P)).cuda(), 6).cpu().numpy()
    np.testing.assert_array_equal(acc, oracle.accept_prefix(am[0].reshape(B, P), am[1].reshape(B, P), 6))
    if amb == 0:
        l1, l3 = oracle.heads([s.h[0], s.h[2]], [s.w[0], s.w[2]])
        want = oracle.accept_prefix(oracle.argmax_lowest(l1).reshape(B, P),
                                    oracle.argmax_lowest(l3).reshape(B, P), 6)
        np.testing.assert_array_equal(acc, want)


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
    check_argmax(am[0], s.h[0], s.w[0])
    check_argmax(am[1], s.h[2], s.w[2])
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
    _, am = nel.exit_heads(ds.h, ds.w, want_argmax=True)
    am = am.cpu().numpy()
    for m in range(2):
        l = oracle.heads([s.h[m]], [s.w[m]])[0]
        ref = oracle.argmax_lowest(l)
        tied = np.isin(ref, [3, 130, 199])
        assert np.array_equal(am[m][tied], ref[tied])
        check_argmax(am[m], s.h[m], s.w[m])
