"""Backward of the junction (nel_junction_backward) against the oracle.

Bars: dL/dh is computed in fp32 and rounded once to its type, so for bf16 it
is within half an ulp (2^-8 relative) plus the fp32 error of the norms; the
embedding gradient is an fp32 sum, within 1e-5 of the sum of the magnitudes
of its terms."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DevSuite, dev_tensor, log, to_np

pytestmark = pytest.mark.gpu


def upstream(n, d_out, dtype, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((n, d_out)).astype(np.float32) * 1e-2
    return synth.round_to_bf16(x) if dtype == "bf16" else x


def term_magnitude(h, ids, emb, dout):
    """sum over the tokens of |each term| of demb (the scale of its rounding error)."""
    _, m = oracle.junction_backward(None if h is None else np.abs(h), ids, np.abs(emb),
                                    np.abs(dout))
    return m


def check(nel, s, m, dtype, stop_grad=False, seed=0):
    """Junction m -> m+1 of suite s (m = 0 is block 1: no h)."""
    import torch
    ds = DevSuite(s)
    h = None if m == 0 else s.h[m - 1]
    d_in = 0 if m == 0 else s.widths[m - 1]
    dout = upstream(s.n_tokens, s.widths[m], dtype, seed)
    dh, demb = nel.junction_backward(None if m == 0 else ds.h[m - 1], ds.ids, ds.emb[m],
                                     dev_tensor(dout, dtype), stop_grad=stop_grad)
    torch.cuda.synchronize()
    ref_dh, ref_demb = oracle.junction_backward(h, s.ids, s.emb[m], dout, stop_grad=stop_grad)
    got = to_np(demb)
    tol = 1e-5 * term_magnitude(h, s.ids, s.emb[m], dout) + 1e-30
    assert np.all(np.abs(got - ref_demb) <= tol), "demb"
    if m > 0:
        g = to_np(dh)
        scale = float(np.max(np.abs(ref_dh))) if ref_dh.size else 0.0
        rel = 2.0 ** -8 if dtype == "bf16" else 1e-6
        assert np.all(np.abs(g - ref_dh) <= rel * np.abs(ref_dh) + 1e-5 * scale + 1e-30), "dh"
    else:
        assert dh is None
    return dh, demb


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_junction_backward_small(nel, dtype):
    s = synth.make_suite((64, 136, 200), 300, 2, 150, dtype=dtype, seed=71)
    log(f"[jbwd] small {dtype}: n={s.n_tokens} widths={s.widths}")
    for m in range(3):
        check(nel, s, m, dtype, seed=m)


def test_junction_backward_stop_gradient(nel):
    import torch
    s = synth.make_suite((64, 128), 200, 1, 90, seed=72)
    _, e1 = check(nel, s, 1, "bf16", stop_grad=False, seed=5)
    dh, e2 = check(nel, s, 1, "bf16", stop_grad=True, seed=5)
    assert float(dh.float().abs().max()) == 0.0
    assert torch.equal(e1, e2)   # the embedding gradient does not depend on the option


def test_junction_backward_deterministic(nel):
    import torch
    s = synth.make_suite((128, 256), 64, 4, 256, seed=73)   # few ids: long repeated rows
    ds = DevSuite(s)
    dout = dev_tensor(upstream(s.n_tokens, 256, "bf16", 9), "bf16")
    a = nel.junction_backward(ds.h[0], ds.ids, ds.emb[1], dout)
    b = nel.junction_backward(ds.h[0], ds.ids, ds.emb[1], dout)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_junction_backward_bad_ids(nel):
    import torch
    s = synth.make_suite((64, 128), 100, 1, 40, seed=74)
    ds = DevSuite(s)
    ids = ds.ids.clone()
    ids[3] = 100
    ids[7] = -2
    dout = upstream(s.n_tokens, 128, "bf16", 11)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    dh, demb = nel.junction_backward(ds.h[0], ids, ds.emb[1], dev_tensor(dout, "bf16"),
                                     flags=flags)
    assert nel.read_flags(flags) == nel.FLAG_BAD_ID
    g = to_np(dh)
    assert np.all(np.isnan(g[[3, 7]]))
    ok = np.ones(s.n_tokens, bool)
    ok[[3, 7]] = False
    ref_dh, ref_demb = oracle.junction_backward(s.h[0][ok], s.ids[ok], s.emb[1], dout[ok])
    np.testing.assert_allclose(g[ok], ref_dh, rtol=2 ** -8, atol=1e-6)
    np.testing.assert_allclose(to_np(demb), ref_demb, rtol=1e-5, atol=1e-7)


def test_junction_backward_full_size(nel):
    """Junction 2 -> 3 of the benchmark workload (16384 tokens, 2304 -> 4352,
    Zipf ids over 32768), every element compared."""
    s = synth.make_workload(2)
    log(f"[jbwd] full size n={s.n_tokens} {s.widths[1]} -> {s.widths[2]}")
    check(nel, s, 2, "bf16", seed=12)
