"""Junction ablation modes (no rescale, zero fill) against the oracle, forward
and backward, on both kernel paths (16-byte chunks and element-wise widths).

Bars as for the method's junction: copies and zeros bit-exact, a rescaled
element within one bf16 ulp (fp32: 1e-6 relative); dL/dh within half a bf16
ulp plus the fp32 error of the norms; the fp32 embedding gradient within 1e-5
of the sum of its terms' magnitudes."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DevSuite, bf16_ulp, dev_tensor, log, to_np

pytestmark = pytest.mark.gpu

MODES = [oracle.JUNCTION_NO_RESCALE, oracle.JUNCTION_ZERO_FILL]


def suites():
    # chunked widths (multiples of 8) and element-wise widths, bf16 and fp32
    return [("chunked-bf16", synth.make_suite((64, 136, 200), 300, 2, 150, seed=91)),
            ("chunked-f32", synth.make_suite((64, 136, 200), 300, 2, 150, dtype="f32", seed=92)),
            ("odd-bf16", synth.make_suite((13, 40, 57), 50, 1, 37, seed=93))]


@pytest.mark.parametrize("mode", MODES)
def test_junction_mode_forward(nel, mode):
    for name, s in suites():
        ds = DevSuite(s)
        for m in range(s.n_exits):
            h = None if m == 0 else s.h[m - 1]
            d_in = 0 if m == 0 else s.widths[m - 1]
            out = to_np(nel.junction(None if m == 0 else ds.h[m - 1], ds.ids, ds.emb[m], mode=mode))
            ref = oracle.junction(h, s.ids, s.emb[m], mode)
            # copies (h unscaled, the embedding) and zeros are exact
            if mode == oracle.JUNCTION_NO_RESCALE or d_in == 0:
                np.testing.assert_array_equal(out, ref)
                continue
            np.testing.assert_array_equal(out[:, d_in:], 0.0)
            if s.dtype == "bf16":
                assert np.all(np.abs(out[:, :d_in] - ref[:, :d_in]) <= bf16_ulp(ref[:, :d_in]) + 1e-30)
            else:
                np.testing.assert_allclose(out[:, :d_in], ref[:, :d_in], rtol=1e-6, atol=1e-30)
        log(f"[jmode] forward mode {mode} {name} ok")


def term_magnitude(h, ids, emb, dout, mode):
    _, m = oracle.junction_backward(None if h is None else np.abs(h), ids, np.abs(emb),
                                    np.abs(dout), mode=mode)
    return m


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("stop_grad", [False, True])
def test_junction_mode_backward(nel, mode, stop_grad):
    for name, s in suites():
        ds = DevSuite(s)
        r = np.random.default_rng(94)
        for m in range(s.n_exits):
            h = None if m == 0 else s.h[m - 1]
            dout = (r.standard_normal((s.n_tokens, s.widths[m])) * 1e-2).astype(np.float32)
            if s.dtype == "bf16":
                dout = synth.round_to_bf16(dout)
            dh, demb = nel.junction_backward(None if m == 0 else ds.h[m - 1], ds.ids, ds.emb[m],
                                             dev_tensor(dout, s.dtype), stop_grad=stop_grad,
                                             mode=mode)
            ref_dh, ref_demb = oracle.junction_backward(h, s.ids, s.emb[m], dout,
                                                        stop_grad=stop_grad, mode=mode)
            tol = 1e-5 * term_magnitude(h, s.ids, s.emb[m], dout, mode) + 1e-30
            assert np.all(np.abs(to_np(demb) - ref_demb) <= tol), f"demb {name} m={m}"
            if m == 0:
                assert dh is None
                continue
            g = to_np(dh)
            if stop_grad or mode == oracle.JUNCTION_NO_RESCALE:
                np.testing.assert_array_equal(g, ref_dh)   # 0, or a copy of dout's first half
                continue
            scale = float(np.max(np.abs(ref_dh))) if ref_dh.size else 0.0
            rel = 2.0 ** -8 if s.dtype == "bf16" else 1e-6
            assert np.all(np.abs(g - ref_dh) <= rel * np.abs(ref_dh) + 1e-5 * scale + 1e-30), \
                f"dh {name} m={m}"
        log(f"[jmode] backward mode {mode} stop_grad={stop_grad} {name} ok")
