"""Python binding of libnel.so, the MI355X (gfx950) Matryoshka multi-exit hot path.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in ``include/nel.h``.  PyTorch supplies device memory and the
current stream.  There is no fallback: if the library is not built, every
call raises.  A call without a ``workspace`` argument uses a cached buffer of
its own per operation, device and stream.

    junction(h, ids, emb)                      -> out
    exit_heads(hs, ws, want_logits, want_argmax) -> (logits | None, argmax | None)
    accept_prefix(draft_argmax, verify_argmax, draft_len) -> accepted
    matryoshka_loss(hs, ws, labels, alpha_d, grad_scale, want_dlogits)
                                               -> (mean_loss, token_loss, dlogits)
    pack_weights(w)                            -> w in the MFMA-tiled layout (bf16)
    matryoshka_loss_packed / exit_heads_packed -> as above, on packed weights
    head_backward(dlogits, h, w)               -> (dL/dh bf16, dL/dW fp32) of one exit head
    heads_backward(dlogits, hs, ws)            -> ([dL/dh_m], [dL/dW_m]) of every exit, grouped
    loss_backward_packed(hs, ws, ws_packed, labels, alpha_d, grad_scale)
                                               -> (mean_loss, token_loss, [dL/dh_m], [dL/dW_m]),
                                                  the logit gradients never stored
    junction_backward(h, ids, emb, dout)       -> (dL/dh, dL/demb fp32) of one junction
    speculative_verify(draft_logits, verify_logits, tokens, u_accept, u_next, draft_len)
                                               -> (beta, accepted, next_token)
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

__all__ = [
    "NelError", "load", "lib_path", "junction", "exit_heads", "accept_prefix", "matryoshka_loss",
    "workspace_size", "read_flags", "clear_flags", "status_string", "timing_enable",
    "timing_read", "timing_reset", "KERNELS", "OP_LOSS", "OP_HEADS", "FLAG_BAD_ID",
    "FLAG_BAD_LABEL", "Workspace", "pack_weights", "matryoshka_loss_packed", "exit_heads_packed", "head_backward",
    "head_backward_workspace_size", "heads_backward", "heads_backward_workspace_size", "loss_workspace",
    "junction_backward", "speculative_verify", "speculative_row_stats", "exit_heads_packed_noalloc",
    "loss_backward_packed", "loss_backward_workspace_size",
    "JUNCTION_RESCALE", "JUNCTION_NO_RESCALE", "JUNCTION_ZERO_FILL", "DIV_FORWARD",
    "DIV_REVERSE_KL", "DIV_JS", "DIV_TV",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

F32, BF16 = 0, 1
JUNCTION_RESCALE, JUNCTION_NO_RESCALE, JUNCTION_ZERO_FILL = 0, 1, 2
DIV_FORWARD, DIV_REVERSE_KL, DIV_JS, DIV_TV = 0, 1, 2, 3
OP_LOSS, OP_HEADS = 0, 1
FLAG_BAD_ID, FLAG_BAD_LABEL = 1, 2
MAX_EXITS = 8
KERNELS = ["junction", "heads_loss", "merge", "means", "finalize", "heads_argmax",
           "argmax_merge", "accept", "pack", "bwd_pack", "bwd_dh", "bwd_dw", "junction_bwd", "speculative",
           "divergence", "grad_consts"]


def lib_path() -> str:
    return os.path.join(_HERE, "libnel.so")


class NelError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status) if _LIB is not None else str(status)
        if status == -6 and _LIB is not None:
            msg += " " + _LIB.nel_last_hip_error().decode()
        super().__init__(f"{where}: {msg} ({status})")


def _hip_runtimes() -> set:
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:
        return set()


def load():
    """Load libnel.so (raises if it has not been built).

    PyTorch is imported first: it carries its own HIP runtime under the same
    soname, and loading it first makes libnel.so bind to that one.  Two HIP
    runtimes in one process would own different streams and device state, so
    that case is refused."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = lib_path()
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing; build it with `python -m nested_exit_lm_amd.build`")
    import torch  # noqa: F401  (binds the HIP runtime before libnel.so loads)
    lib = ctypes.CDLL(p)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError("two HIP runtimes are loaded (" + ", ".join(sorted(rts)) + "); "
                          "import torch before any other HIP library")
    c_int, c_i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "nel_junction": [c_int, c_i64, c_int, c_int, c_int, vp, vp, vp, vp, c_int, vp, vp],
        "nel_exit_heads": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, vp, vp, sz, vp],
        "nel_exit_heads_packed": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, vp, vp, sz, vp],
        "nel_exit_heads_packed_noalloc": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, vp, vp],
        "nel_pack_weights": [c_int, c_int, c_int, vp, vp, vp],
        "nel_accept_prefix": [c_int, c_int, c_int, vp, vp, vp, vp],
        "nel_matryoshka_loss": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, ctypes.c_float,
                                ctypes.c_float, vp, c_int, vp, vp, vp, vp, sz, vp],
        "nel_matryoshka_loss_packed": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, ctypes.c_float,
                                       ctypes.c_float, vp, c_int, vp, vp, vp, vp, sz, vp],
        "nel_workspace_size": [c_int, c_int, c_i64, c_int],
        "nel_head_backward": [c_int, c_i64, c_int, c_int, vp, vp, vp, vp, vp, vp, sz, vp],
        "nel_head_backward_workspace": [c_i64, c_int, c_int],
        "nel_heads_backward": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "nel_heads_backward_workspace": [c_int, c_i64, c_int, vp],
        "nel_matryoshka_loss_backward_packed": [c_int, c_int, c_i64, c_int, vp, vp, vp, vp, vp,
                                                ctypes.c_float, ctypes.c_float, vp, vp, vp, vp,
                                                vp, vp, vp, sz, vp],
        "nel_loss_backward_workspace": [c_int, c_i64, c_int, vp],
        "nel_junction_backward": [c_int, c_i64, c_int, c_int, c_int, vp, vp, vp, vp, c_int, c_int,
                                  vp, vp, vp, vp, sz, vp],
        "nel_junction_backward_workspace": [c_i64, c_int, c_int, c_int],
        "nel_speculative_verify": [c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp, ctypes.c_float,
                                   ctypes.c_float, vp, vp, vp, vp, vp, sz, vp],
        "nel_speculative_workspace": [c_int, c_int],
        "nel_read_device_flags": [vp, vp, vp],
        "nel_clear_device_flags": [vp, vp],
        "nel_status_string": [c_int],
        "nel_timing_enable": [c_int],
        "nel_timing_read": [c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
        "nel_timing_reset": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = c_int
    lib.nel_workspace_size.restype = sz
    lib.nel_head_backward_workspace.restype = sz
    lib.nel_heads_backward_workspace.restype = sz
    lib.nel_loss_backward_workspace.restype = sz
    lib.nel_junction_backward_workspace.restype = sz
    lib.nel_speculative_workspace.restype = sz
    lib.nel_status_string.restype = ctypes.c_char_p
    lib.nel_last_hip_error.argtypes = []
    lib.nel_last_hip_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().nel_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise NelError(status, where)


# ----------------------------------------------------------------- marshalling helpers
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16 or float32)")


def _dev(t, device, name):
    if t is None:
        return 0
    if not t.is_cuda or (device is not None and t.device != device):
        raise ValueError(f"{name} must be a CUDA tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def _ptrs(ts) -> ctypes.Array:
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t if isinstance(t, int) else (t.data_ptr() if t is not None else 0)
    return arr


def workspace_size(op: int, n_exits: int, n_tokens: int, vocab: int) -> int:
    return int(load().nel_workspace_size(op, n_exits, n_tokens, vocab))


class Workspace:
    """A growable device byte buffer; zero-filled when (re)allocated, so the
    flag word in its first 4 bytes starts clear."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_WS = {}


def _workspace(op, device, nbytes):
    """The default workspace of an operation: one per (operation, device,
    stream).  Calls on one stream run in issue order, so they can share it;
    a call on another stream gets its own and cannot overwrite it mid-use."""
    ws = _WS.setdefault((op, str(device), _stream(device)), Workspace())
    return ws.get(nbytes, device)


# ----------------------------------------------------------------- entry points
def junction(h, ids, emb, out=None, flags=None, mode: int = 0):
    """out[t] = [h[t] * ||emb[ids[t]]|| / ||h[t]||, emb[ids[t]]]; h may be None (block 1).
    mode: JUNCTION_RESCALE (the method), JUNCTION_NO_RESCALE, JUNCTION_ZERO_FILL."""
    torch = _torch()
    device = emb.device
    n = ids.shape[0]
    d_in = 0 if h is None else h.shape[1]
    de = emb.shape[1]
    if h is not None and (h.dtype != emb.dtype or h.shape[0] != n):
        raise ValueError("h must be [n, d_in] with the embedding's dtype")
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    if out is None:
        out = torch.empty(n, d_in + de, dtype=emb.dtype, device=device)
    lib = load()
    _check(lib.nel_junction(_dt(emb), n, d_in, d_in + de, emb.shape[0], _dev(h, device, "h"),
                            _dev(ids, device, "ids"), _dev(emb, device, "emb"),
                            _dev(out, device, "out"), int(mode), _dev(flags, device, "flags"),
                            _stream(device)), "nel_junction")
    return out


def exit_heads(hs: Sequence, ws: Sequence, want_logits: bool = False, want_argmax: bool = True,
               workspace=None):
    """Logits (fp32, optional) and greedy argmax [n_exits, n] (int32) of each exit's head."""
    return _exit_heads(False, hs, ws, want_logits, want_argmax, workspace)


def exit_heads_packed(hs: Sequence, ws_packed: Sequence, want_logits: bool = False,
                      want_argmax: bool = True, workspace=None):
    """exit_heads on head weights from pack_weights (bf16, V % 32 == 0, every d % 64 == 0)."""
    return _exit_heads(True, hs, ws_packed, want_logits, want_argmax, workspace)


def _exit_heads(packed, hs, ws, want_logits, want_argmax, workspace):
    torch = _torch()
    E = len(hs)
    if E != len(ws) or not 1 <= E <= MAX_EXITS:
        raise ValueError("need 1..8 exits with one head each")
    device = hs[0].device
    n, V = hs[0].shape[0], ws[0].shape[0]
    dt = _dt(hs[0])
    for h, w in zip(hs, ws):
        if _dt(h) != dt or _dt(w) != dt or h.shape[0] != n or w.shape[0] != V or h.shape[1] != w.shape[1]:
            raise ValueError("inconsistent exit shapes or dtypes")
        _dev(h, device, "h")
        _dev(w, device, "w")
    d = (ctypes.c_int32 * E)(*[h.shape[1] for h in hs])
    logits = [torch.empty(n, V, dtype=torch.float32, device=device) for _ in range(E)] if want_logits else None
    am = torch.empty(E, n, dtype=torch.int32, device=device) if want_argmax else None
    need = workspace_size(OP_HEADS, E, n, V)
    wsb = workspace if workspace is not None else _workspace(OP_HEADS, device, need)
    lib = load()
    fn, name = ((lib.nel_exit_heads_packed, "nel_exit_heads_packed") if packed
                else (lib.nel_exit_heads, "nel_exit_heads"))
    _check(fn(dt, E, n, V, d, _ptrs(hs), _ptrs(ws), _ptrs(logits) if logits is not None else None,
              _dev(am, device, "argmax"), wsb.data_ptr(), wsb.numel(), _stream(device)), name)
    return logits, am


NOALLOC_SCRATCH_BYTES = 16 << 20
ETOOLARGE = -7


def exit_heads_packed_noalloc(hs: Sequence, ws_packed: Sequence, logits: Optional[List] = None,
                              argmax=None):
    """exit_heads_packed through the allocation-free entry point: the library
    uses its fixed per-GPU scratch instead of a workspace, and every output is
    the caller's (`logits`: None or a list of fp32 [n, V] tensors; `argmax`:
    None or int32 [n_exits, n]).  Calls that overlap on one GPU race.
    Returns (logits, argmax) as given."""
    E = len(hs)
    if E != len(ws_packed) or not 1 <= E <= MAX_EXITS:
        raise ValueError("need 1..8 exits with one head each")
    device = hs[0].device
    n, V = hs[0].shape[0], ws_packed[0].shape[0]
    for h, w in zip(hs, ws_packed):
        if _dt(h) != BF16 or _dt(w) != BF16 or h.shape[0] != n or w.shape[0] != V or h.shape[1] != w.shape[1]:
            raise ValueError("inconsistent exit shapes or dtypes (bf16 packed heads)")
        _dev(h, device, "h")
        _dev(w, device, "w")
    if logits is not None:
        if len(logits) != E:
            raise ValueError("one logits tensor per exit")
        for t in logits:
            if tuple(t.shape) != (n, V) or t.dtype != _torch().float32:
                raise ValueError("logits must be fp32 [n, V]")
            _dev(t, device, "logits")
    if argmax is not None and (tuple(argmax.shape) != (E, n) or argmax.dtype != _torch().int32):
        raise ValueError("argmax must be int32 [n_exits, n]")
    d = (ctypes.c_int32 * E)(*[h.shape[1] for h in hs])
    _check(load().nel_exit_heads_packed_noalloc(
        BF16, E, n, V, d, _ptrs(hs), _ptrs(ws_packed), _ptrs(logits) if logits is not None else None,
        _dev(argmax, device, "argmax"), _stream(device)), "nel_exit_heads_packed_noalloc")
    return logits, argmax


def accept_prefix(draft_argmax, verify_argmax, draft_len: int):
    """Leading matches among the first draft_len positions, per sequence ([B, P] int32 inputs)."""
    torch = _torch()
    device = draft_argmax.device
    if draft_argmax.shape != verify_argmax.shape or draft_argmax.dim() != 2:
        raise ValueError("draft and verify argmax must both be [batch, positions]")
    for t in (draft_argmax, verify_argmax):
        if t.dtype != torch.int32:
            raise TypeError("argmax arrays must be int32")
    B, P = draft_argmax.shape
    acc = torch.empty(B, dtype=torch.int32, device=device)
    _check(load().nel_accept_prefix(B, P, draft_len, _dev(draft_argmax, device, "draft"),
                                    _dev(verify_argmax, device, "verify"),
                                    _dev(acc, device, "accepted"), _stream(device)),
           "nel_accept_prefix")
    return acc


def matryoshka_loss(hs: Sequence, ws: Sequence, labels, alpha_d: float = 0.3,
                    grad_scale: float = 1.0, want_dlogits: bool = True,
                    want_token_loss: bool = True, dlogits: Optional[List] = None, workspace=None,
                    mean_loss=None, token_loss=None, exit_weights: Optional[Sequence[float]] = None,
                    divergence: int = 0):
    """Losses of every exit and, optionally, dL/dlogits (in hs' dtype).

    exit_weights: per-exit weights of the total (None: all 1); divergence: DIV_FORWARD
    (the cross-entropy to the teacher), DIV_REVERSE_KL, DIV_JS or DIV_TV (these need
    the logit gradients).
    Returns (mean_loss [3M+1] fp32, token_loss [M, 3, n] fp32 | None, dlogits list | None);
    mean_loss = (CE_1..CE_M, Dist_1..Dist_M, L_1..L_M, total)."""
    return _loss(False, hs, ws, labels, alpha_d, grad_scale, want_dlogits, want_token_loss,
                 dlogits, workspace, mean_loss, token_loss, exit_weights, divergence)


def matryoshka_loss_packed(hs: Sequence, ws_packed: Sequence, labels, alpha_d: float = 0.3,
                           grad_scale: float = 1.0, want_token_loss: bool = True,
                           dlogits: Optional[List] = None, workspace=None, mean_loss=None,
                           token_loss=None, exit_weights: Optional[Sequence[float]] = None,
                           divergence: int = 0):
    """matryoshka_loss on head weights from pack_weights (bf16, V % 32 == 0, every
    d % 64 == 0); the logit gradients are always produced."""
    return _loss(True, hs, ws_packed, labels, alpha_d, grad_scale, True, want_token_loss,
                 dlogits, workspace, mean_loss, token_loss, exit_weights, divergence)


def _loss(packed, hs, ws, labels, alpha_d, grad_scale, want_dlogits, want_token_loss, dlogits,
          workspace, mean_loss, token_loss, exit_weights=None, divergence=0):
    torch = _torch()
    E = len(hs)
    if E != len(ws) or not 1 <= E <= MAX_EXITS:
        raise ValueError("need 1..8 exits with one head each")
    device = hs[0].device
    n, V = hs[0].shape[0], ws[0].shape[0]
    dt = _dt(hs[0])
    for h, w in zip(hs, ws):
        if _dt(h) != dt or _dt(w) != dt or h.shape[0] != n or w.shape[0] != V or h.shape[1] != w.shape[1]:
            raise ValueError("inconsistent exit shapes or dtypes")
        _dev(h, device, "h")
        _dev(w, device, "w")
    if labels.dtype != torch.int32 or labels.shape != (n,):
        raise ValueError("labels must be int32 [n]")
    d = (ctypes.c_int32 * E)(*[h.shape[1] for h in hs])
    if want_dlogits and dlogits is None:
        dlogits = [torch.empty(n, V, dtype=hs[0].dtype, device=device) for _ in range(E)]
    if not want_dlogits:
        dlogits = None
    if mean_loss is None:
        mean_loss = torch.empty(3 * E + 1, dtype=torch.float32, device=device)
    if want_token_loss and token_loss is None:
        token_loss = torch.empty(E, 3, n, dtype=torch.float32, device=device)
    if not want_token_loss:
        token_loss = None
    need = workspace_size(OP_LOSS, E, n, V)
    wsb = workspace if workspace is not None else _workspace(OP_LOSS, device, need)
    lib = load()
    fn, name = ((lib.nel_matryoshka_loss_packed, "nel_matryoshka_loss_packed") if packed
                else (lib.nel_matryoshka_loss, "nel_matryoshka_loss"))
    lam = None
    if exit_weights is not None:
        if len(exit_weights) != E:
            raise ValueError("exit_weights needs one weight per exit")
        lam = (ctypes.c_float * E)(*[float(x) for x in exit_weights])
    _check(fn(dt, E, n, V, d, _ptrs(hs), _ptrs(ws), _dev(labels, device, "labels"),
              float(alpha_d), float(grad_scale), lam, int(divergence),
              _dev(token_loss, device, "token_loss"),
              _dev(mean_loss, device, "mean_loss"),
              _ptrs(dlogits) if dlogits is not None else None, wsb.data_ptr(), wsb.numel(),
              _stream(device)), name)
    return mean_loss, token_loss, dlogits


def pack_weights(w, out=None):
    """Rewrite a bf16 head weight [V, d] (V % 32 == 0, d % 64 == 0) into the MFMA-tiled layout
    the *_packed entry points read.  The result has w's shape and dtype; its element order is
    the tiled one, so it is only meaningful to those entry points."""
    torch = _torch()
    if w.dim() != 2 or w.dtype != torch.bfloat16:
        raise ValueError("w must be a 2-D bfloat16 tensor")
    device = w.device
    if out is None:
        out = torch.empty_like(w)
    elif out.shape != w.shape or out.dtype != w.dtype:
        raise ValueError("out must match w's shape and dtype")
    _check(load().nel_pack_weights(BF16, w.shape[0], w.shape[1], _dev(w, device, "w"),
                                   _dev(out, device, "out"), _stream(device)), "nel_pack_weights")
    return out


def loss_workspace(device, n_exits: int, n_tokens: int, vocab: int):
    """The workspace matryoshka_loss uses by default (its first int32 is the flag word)."""
    return _workspace(OP_LOSS, device, workspace_size(OP_LOSS, n_exits, n_tokens, vocab))


def read_flags(flags_tensor) -> int:
    """Read a device flag word (an int32 tensor or a workspace byte tensor)."""
    out = ctypes.c_int32(0)
    dev = flags_tensor.device
    _check(load().nel_read_device_flags(flags_tensor.data_ptr(), ctypes.addressof(out),
                                        _stream(dev)), "nel_read_device_flags")
    return out.value


def clear_flags(flags_tensor):
    _check(load().nel_clear_device_flags(flags_tensor.data_ptr(), _stream(flags_tensor.device)),
           "nel_clear_device_flags")


def timing_enable(on: bool = True):
    _check(load().nel_timing_enable(1 if on else 0), "nel_timing_enable")


def timing_reset():
    _check(load().nel_timing_reset(), "nel_timing_reset")


def timing_read(kernel) -> tuple:
    """(total milliseconds, launches) of one kernel since the last reset; synchronises."""
    k = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    ms, cnt = ctypes.c_double(0), ctypes.c_int64(0)
    _check(load().nel_timing_read(k, ctypes.byref(ms), ctypes.byref(cnt)), "nel_timing_read")
    return ms.value, cnt.value


def head_backward_workspace_size(n_tokens: int, vocab: int, d: int) -> int:
    return int(load().nel_head_backward_workspace(n_tokens, vocab, d))



def head_backward(dlogits, h, w, want_dh: bool = True, want_dw: bool = True, dh=None, dw=None,
                  workspace=None):
    """Backward of one exit head l = h W^T: (dL/dh = G W in bf16, dL/dW = G^T h in fp32),
    with G = dlogits (bf16 [n, V]); either output may be skipped (None returned)."""
    torch = _torch()
    device = dlogits.device
    n, V = dlogits.shape
    d = h.shape[1]
    for t, name in ((dlogits, "dlogits"), (h, "h"), (w, "w")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    if h.shape[0] != n or w.shape != (V, d):
        raise ValueError("need dlogits [n, V], h [n, d], w [V, d]")
    if want_dh and dh is None:
        dh = torch.empty(n, d, dtype=torch.bfloat16, device=device)
    if want_dw and dw is None:
        dw = torch.empty(V, d, dtype=torch.float32, device=device)
    if not want_dh:
        dh = None
    if not want_dw:
        dw = None
    need = head_backward_workspace_size(n, V, d)
    wsb = workspace if workspace is not None else _workspace("head_backward", device, need)
    _check(load().nel_head_backward(BF16, n, V, d, _dev(dlogits, device, "dlogits"),
                                    _dev(h, device, "h"), _dev(w, device, "w"),
                                    _dev(dh, device, "dh"), _dev(dw, device, "dw"),
                                    wsb.data_ptr(), wsb.numel(), _stream(device)),
           "nel_head_backward")
    return dh, dw


def heads_backward_workspace_size(n_tokens: int, vocab: int, widths) -> int:
    ds = (ctypes.c_int32 * len(widths))(*widths)
    return int(load().nel_heads_backward_workspace(len(widths), n_tokens, vocab, ds))


def heads_backward(dlogits, hs, ws, want_dh: bool = True, want_dw: bool = True, dhs=None,
                   dws=None, workspace=None):
    """head_backward for every exit in two launches (one grouped dh GEMM, one grouped
    dW GEMM): lists (dh_m bf16 [n, d_m] or None, dW_m fp32 [V, d_m] or None), with the
    same bits as the per-exit call."""
    torch = _torch()
    M = len(hs)
    if not (len(dlogits) == M == len(ws)) or M == 0:
        raise ValueError("need one dlogits, h and w per exit")
    device = dlogits[0].device
    n, V = dlogits[0].shape
    widths = [h.shape[1] for h in hs]
    for m in range(M):
        for t, name in ((dlogits[m], "dlogits"), (hs[m], "h"), (ws[m], "w")):
            if t.dtype != torch.bfloat16:
                raise TypeError(f"{name}[{m}] must be bfloat16")
        if dlogits[m].shape != (n, V) or hs[m].shape[0] != n or ws[m].shape != (V, widths[m]):
            raise ValueError("need dlogits[m] [n, V], h[m] [n, d_m], w[m] [V, d_m]")
    if want_dh:
        dhs = dhs if dhs is not None else [
            torch.empty(n, d, dtype=torch.bfloat16, device=device) for d in widths]
    if want_dw:
        dws = dws if dws is not None else [
            torch.empty(V, d, dtype=torch.float32, device=device) for d in widths]
    if not want_dh:
        dhs = None
    if not want_dw:
        dws = None
    for lst, name in ((dhs, "dhs"), (dws, "dws")):
        if lst is not None and len(lst) != M:
            raise ValueError(f"{name} needs one tensor per exit")
    need = heads_backward_workspace_size(n, V, widths)
    wsb = workspace if workspace is not None else _workspace("head_backward", device, need)
    ds = (ctypes.c_int32 * M)(*widths)
    g = _ptrs([_dev(t, device, "dlogits") for t in dlogits])
    hp = _ptrs([_dev(t, device, "h") for t in hs])
    wp = _ptrs([_dev(t, device, "w") for t in ws])
    dhp = _ptrs([_dev(t, device, "dh") for t in dhs]) if dhs is not None else None
    dwp = _ptrs([_dev(t, device, "dw") for t in dws]) if dws is not None else None
    _check(load().nel_heads_backward(BF16, M, n, V, ds, g, hp, wp, dhp, dwp, wsb.data_ptr(),
                                     wsb.numel(), _stream(device)), "nel_heads_backward")
    return dhs, dws



def loss_backward_workspace_size(n_tokens: int, vocab: int, widths) -> int:
    ds = (ctypes.c_int32 * len(widths))(*widths)
    return int(load().nel_loss_backward_workspace(len(widths), n_tokens, vocab, ds))


def loss_backward_packed(hs: Sequence, ws: Sequence, ws_packed: Sequence, labels,
                         alpha_d: float = 0.3, grad_scale: float = 1.0,
                         want_dh: bool = True, want_dw: bool = True,
                         exit_weights: Optional[Sequence[float]] = None,
                         want_token_loss: bool = True, scratch: Optional[List] = None,
                         dhs=None, dws=None, mean_loss=None, token_loss=None, workspace=None):
    """The losses (as matryoshka_loss_packed) and every exit head's backward, the logit
    gradients formed inside the dh and dW GEMMs and never stored.  ws: the heads row-major
    (bf16 [V, d_m]); ws_packed: the same heads from pack_weights; scratch: n x V 16-bit
    buffers, one per exit (allocated when None).  The workspace's first int32 is the
    device flag word.  Returns (mean_loss, token_loss | None, [dh_m bf16] | None,
    [dW_m fp32] | None): dh bit-identical to matryoshka_loss_packed followed by
    heads_backward, dW the same products summed in another fp32 order."""
    torch = _torch()
    M = len(hs)
    if not (len(ws) == M == len(ws_packed)) or not 1 <= M <= MAX_EXITS:
        raise ValueError("need 1..8 exits with one head (row-major and packed) each")
    device = hs[0].device
    n, V = hs[0].shape[0], ws[0].shape[0]
    widths = [h.shape[1] for h in hs]
    for m in range(M):
        for t, name in ((hs[m], "h"), (ws[m], "w"), (ws_packed[m], "w_packed")):
            if t.dtype != torch.bfloat16:
                raise TypeError(f"{name}[{m}] must be bfloat16")
            _dev(t, device, name)
        if hs[m].shape[0] != n or ws[m].shape != (V, widths[m]) or ws_packed[m].shape != ws[m].shape:
            raise ValueError("need h[m] [n, d_m], w[m] and w_packed[m] [V, d_m]")
    if labels.dtype != torch.int32 or labels.shape != (n,):
        raise ValueError("labels must be int32 [n]")
    if scratch is None:
        scratch = [torch.empty(n, V, dtype=torch.bfloat16, device=device) for _ in range(M)]
    if len(scratch) != M or any(t.numel() != n * V or t.element_size() != 2 for t in scratch):
        raise ValueError("scratch needs one n x V 16-bit buffer per exit")
    dhs = (dhs if dhs is not None else [torch.empty(n, d, dtype=torch.bfloat16, device=device)
                                        for d in widths]) if want_dh else None
    dws = (dws if dws is not None else [torch.empty(V, d, dtype=torch.float32, device=device)
                                        for d in widths]) if want_dw else None
    for lst, name in ((dhs, "dhs"), (dws, "dws")):
        if lst is not None and len(lst) != M:
            raise ValueError(f"{name} needs one tensor per exit")
    if mean_loss is None:
        mean_loss = torch.empty(3 * M + 1, dtype=torch.float32, device=device)
    if want_token_loss and token_loss is None:
        token_loss = torch.empty(M, 3, n, dtype=torch.float32, device=device)
    if not want_token_loss:
        token_loss = None
    lam = None
    if exit_weights is not None:
        if len(exit_weights) != M:
            raise ValueError("exit_weights needs one weight per exit")
        lam = (ctypes.c_float * M)(*[float(x) for x in exit_weights])
    need = loss_backward_workspace_size(n, V, widths)
    if need == 0:
        raise ValueError("shape not supported (V and every d_m must be multiples of 64)")
    wsb = workspace if workspace is not None else _workspace("loss_backward", device, need)
    ds = (ctypes.c_int32 * M)(*widths)
    _check(load().nel_matryoshka_loss_backward_packed(
        BF16, M, n, V, ds, _ptrs(hs), _ptrs(ws), _ptrs(ws_packed),
        _dev(labels, device, "labels"), float(alpha_d), float(grad_scale), lam,
        _dev(token_loss, device, "token_loss"), _dev(mean_loss, device, "mean_loss"),
        _ptrs([_dev(t, device, "scratch") for t in scratch]),
        _ptrs([_dev(t, device, "dh") for t in dhs]) if dhs is not None else None,
        _ptrs([_dev(t, device, "dw") for t in dws]) if dws is not None else None,
        wsb.data_ptr(), wsb.numel(), _stream(device)), "nel_matryoshka_loss_backward_packed")
    return mean_loss, token_loss, dhs, dws


def junction_backward(h, ids, emb, dout, stop_grad: bool = False, want_dh: bool = True,
                      want_demb: bool = True, dh=None, demb=None, flags=None, workspace=None,
                      mode: int = 0):
    """Gradients of junction(h, ids, emb) given dout = dL/dout: (dL/dh in h's dtype or None,
    dL/demb fp32 [V, d_out - d_in] or None).  h may be None (block 1)."""
    torch = _torch()
    device = emb.device
    n = ids.shape[0]
    d_in = 0 if h is None else h.shape[1]
    de = emb.shape[1]
    if dout.shape != (n, d_in + de) or dout.dtype != emb.dtype:
        raise ValueError("dout must be [n, d_in + d_emb] in the embedding's dtype")
    if h is not None and (h.dtype != emb.dtype or h.shape[0] != n):
        raise ValueError("h must be [n, d_in] in the embedding's dtype")
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    if want_dh and d_in > 0 and dh is None:
        dh = torch.empty(n, d_in, dtype=emb.dtype, device=device)
    if not want_dh or d_in == 0:
        dh = None
    if want_demb and demb is None:
        demb = torch.empty(emb.shape[0], de, dtype=torch.float32, device=device)
    if not want_demb:
        demb = None
    lib = load()
    need = int(lib.nel_junction_backward_workspace(n, d_in, d_in + de, emb.shape[0]))
    wsb = workspace if workspace is not None else _workspace("junction_backward", device, need)
    _check(lib.nel_junction_backward(_dt(emb), n, d_in, d_in + de, emb.shape[0],
                                     _dev(h, device, "h"), _dev(ids, device, "ids"),
                                     _dev(emb, device, "emb"), _dev(dout, device, "dout"),
                                     1 if stop_grad else 0, int(mode), _dev(dh, device, "dh"),
                                     _dev(demb, device, "demb"), _dev(flags, device, "flags"),
                                     wsb.data_ptr(), wsb.numel(), _stream(device)),
           "nel_junction_backward")
    return dh, demb



def speculative_verify(draft_logits, verify_logits, draft_tokens, u_accept, u_next,
                       draft_len: int, temperature: float = 1.0, top_p: float = 1.0,
                       want_beta: bool = True, flags=None, workspace=None):
    """Sampled speculative verification from two exits' fp32 logits [B, P, V]
    (or [B*P, V] with draft_tokens / u_accept [B, P]).  Returns
    (beta [B, draft_len] | None, accepted [B], next_token [B])."""
    torch = _torch()
    device = draft_logits.device
    B, P = draft_tokens.shape
    V = draft_logits.shape[-1]
    for t, name in ((draft_logits, "draft_logits"), (verify_logits, "verify_logits"),
                    (u_accept, "u_accept"), (u_next, "u_next")):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if draft_tokens.dtype != torch.int32:
        raise TypeError("draft_tokens must be int32")
    if draft_logits.numel() != B * P * V or verify_logits.numel() != B * P * V:
        raise ValueError("logits must hold [B, P, V]")
    beta = torch.empty(B, max(draft_len, 0), dtype=torch.float32, device=device) if want_beta else None
    acc = torch.empty(B, dtype=torch.int32, device=device)
    nxt = torch.empty(B, dtype=torch.int32, device=device)
    lib = load()
    need = int(lib.nel_speculative_workspace(B, draft_len))
    wsb = workspace if workspace is not None else _workspace("speculative", device, need)
    _check(lib.nel_speculative_verify(B, P, draft_len, V, _dev(draft_logits, device, "draft_logits"),
                                      _dev(verify_logits, device, "verify_logits"),
                                      _dev(draft_tokens, device, "draft_tokens"),
                                      _dev(u_accept, device, "u_accept"), _dev(u_next, device, "u_next"),
                                      float(temperature), float(top_p), _dev(beta, device, "beta"),
                                      _dev(acc, device, "accepted"), _dev(nxt, device, "next_token"),
                                      _dev(flags, device, "flags"), wsb.data_ptr(), wsb.numel(),
                                      _stream(device)), "nel_speculative_verify")
    return beta, acc, nxt


def speculative_row_stats(workspace, batch: int, draft_len: int):
    """The per-row statistics nel_speculative_verify leaves in its workspace
    (nel.h): fp32 [2, batch, draft_len + 1, 4] = (max of l / T, nucleus mass,
    threshold value, softmax mass) for the draft exit, then the verifying
    exit.  A view of the workspace: read it before the next call reuses it."""
    torch = _torch()
    n = 2 * batch * (draft_len + 1) * 4
    return workspace[: 4 * n].view(torch.float32).view(2, batch, draft_len + 1, 4)
