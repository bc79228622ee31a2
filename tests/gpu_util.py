"""Shared helpers of the GPU tests: moving a synthetic suite to the device,
reading results back, and the comparison bars."""
from __future__ import annotations

import sys

import numpy as np


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(arr: np.ndarray, dtype: str, device="cuda:0"):
    """A bf16-exact float32 array as a bf16 tensor, or a float32 tensor."""
    import torch
    import synth
    if dtype == "bf16":
        bits = synth.bf16_bits(arr)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_np(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


class DevSuite:
    def __init__(self, s, device="cuda:0", exits=None):
        import torch
        self.s = s
        sel = list(range(s.n_exits)) if exits is None else list(exits)
        self.sel = sel
        self.h = [dev_tensor(s.h[m], s.dtype, device) for m in sel]
        self.w = [dev_tensor(s.w[m], s.dtype, device) for m in sel]
        self.emb = [dev_tensor(e, s.dtype, device) for e in s.emb]
        self.hall = {m: h for m, h in zip(sel, self.h)}
        self.ids = torch.from_numpy(s.ids).to(device)
        self.labels = torch.from_numpy(s.labels).to(device)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (for normal values)."""
    ax = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_loss_close(got: np.ndarray, ref: np.ndarray, rel=1e-3, what=""):
    """Per element |got - ref| <= rel * max(1, |ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rel, f"{what}: worst scaled error {worst:.3g} > {rel}"
    return worst


def assert_grad_close(got: np.ndarray, ref: np.ndarray, atol: float, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    worst = float(np.abs(got - ref).max()) if got.size else 0.0
    assert worst <= atol, f"{what}: max abs error {worst:.3g} > {atol}"
    return worst


def head_error_bound(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Upper bound of |fp32 accumulation - exact| per logit: gamma_K sum |h_k w_k| with a
    generous gamma (any summation order, fp32 products of bf16 values are exact)."""
    K = h.shape[1]
    gamma = 2.0 * K * 2.0 ** -24
    return gamma * (np.abs(h) @ np.abs(w).T)


def head_error_bound_ordered(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """The same bound following the order the bf16 GEMMs accumulate in: every
    matrix-core instruction adds the sum of 16 (32x32x16) or 32 (16x16x32)
    exact products (bf16 x bf16 fits fp32) to the fp32 accumulator, so each
    logit is a chain of at most ceil(K / 16) accumulator roundings plus, inside
    each instruction, a sum of at most 32 terms in any order (at most 31
    roundings of any one term).  The unit roundoff is taken as 2^-23
    (truncation as well as round-to-nearest), so
        |error| <= (ceil(K / 16) + 31) 2^-23 sum_k |h_k w_k|  (first order)."""
    K = h.shape[1]
    n = -(-K // 16) + 31
    u = 2.0 ** -23
    gamma = n * u / (1.0 - n * u)
    return gamma * (np.abs(h) @ np.abs(w).T)


GRAD_TOL = {"bf16": 2e-2, "f32": 1e-4}
LOSS_TOL = {"bf16": 1e-3, "f32": 1e-4}


def run_loss(nel, ds, alpha, grad_scale=1.0, want_dlogits=True, packed=None):
    """The loss through the C ABI; `packed` is None (row-major heads) or the list of
    packed head weights."""
    import torch
    if packed is None:
        mean, tok, dl = nel.matryoshka_loss(ds.h, ds.w, ds.labels, alpha_d=alpha,
                                            grad_scale=grad_scale, want_dlogits=want_dlogits)
    else:
        mean, tok, dl = nel.matryoshka_loss_packed(ds.h, packed, ds.labels, alpha_d=alpha,
                                                   grad_scale=grad_scale)
    torch.cuda.synchronize()
    return to_np(mean), to_np(tok), dl


def check_full(nel, s, alpha, grad_scale=1.0, packed=False):
    """Every token, every exit, every vocabulary entry against the oracle."""
    import oracle
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w] if packed else None
    mean, tok, dl = run_loss(nel, ds, alpha, grad_scale, packed=pw)
    ref, grads = oracle.forward_tokens(s.h, s.w, s.labels, alpha, grad_scale)
    M = s.n_exits
    tol = LOSS_TOL[s.dtype]
    assert_loss_close(tok[:, 0], ref["ce"], tol, "CE")
    assert_loss_close(tok[:, 1], ref["dist"], tol, "Dist")
    assert_loss_close(tok[:, 2], ref["loss"], tol, "L")
    want_mean = np.concatenate([ref["mean_ce"], ref["mean_dist"], ref["mean_loss"], [ref["mean_total"]]])
    assert mean.shape == (3 * M + 1,)
    assert_loss_close(mean, want_mean, tol, "means")
    for m in range(M):
        assert_grad_close(to_np(dl[m]), grads[m], GRAD_TOL[s.dtype] * max(1.0, abs(grad_scale)),
                          f"dlogits exit {m}")


def sample_rows(n, k, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, n - 1, n // 2], r.choice(n, size=k, replace=False)]))
