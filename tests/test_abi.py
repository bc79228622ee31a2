"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before launching."""
import ctypes
import os
import re

import pytest

import nested_exit_lm_amd as nel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "nel.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nel_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = nel.load()
    syms = declared_symbols()
    assert len(syms) == 26
    for s in syms:
        assert hasattr(lib, s), s


def test_status_strings_and_workspace_sizes():
    assert nel.status_string(0) == "ok"
    assert "workspace" in nel.status_string(-5)
    assert nel.status_string(-99) == "unknown status"
    assert nel.load().nel_last_hip_error() == b"none"
    n, V = 16384, 32768
    nvt = V // 128
    ws = nel.workspace_size(nel.OP_LOSS, 3, n, V)
    assert ws >= 4 * (3 * 3 * nvt * n + 3 * n * 5)
    assert nel.workspace_size(nel.OP_HEADS, 2, 714, V) >= 4 * 2 * 2 * nvt * 714
    assert nel.workspace_size(nel.OP_LOSS, 0, n, V) == 0
    assert nel.workspace_size(nel.OP_LOSS, 9, n, V) == 0
    assert nel.workspace_size(7, 3, n, V) == 0


def _arr(t, *v):
    return (t * len(v))(*v)


FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)
MIS = 0x10004           # 4-byte aligned only: misaligned for tensors
MIS4 = 0x10002          # misaligned for int32 arrays


def test_junction_host_validation():
    lib = nel.load()
    assert lib.nel_junction(7, 4, 8, 16, 10, FAKE, FAKE, FAKE, FAKE, 0, None, None) == -3
    assert lib.nel_junction(1, -1, 8, 16, 10, FAKE, FAKE, FAKE, FAKE, 0, None, None) == -2
    assert lib.nel_junction(1, 4, 8, 8, 10, FAKE, FAKE, FAKE, FAKE, 0, None, None) == -2
    assert lib.nel_junction(1, 4, 8, 16, 0, FAKE, FAKE, FAKE, FAKE, 0, None, None) == -2
    assert lib.nel_junction(1, 4, 8, 16, 10, None, FAKE, FAKE, FAKE, 0, None, None) == -1
    assert lib.nel_junction(1, 4, 8, 16, 10, MIS, FAKE, FAKE, FAKE, 0, None, None) == -4
    assert lib.nel_junction(1, 4, 8, 16, 10, FAKE, MIS4, FAKE, FAKE, 0, None, None) == -4
    assert lib.nel_junction(1, 0, 8, 16, 10, None, None, None, None, 0, None, None) == 0
    assert lib.nel_junction(1, 4, 8, 16, 10, FAKE, FAKE, FAKE, FAKE, 3, None, None) == -1
    assert lib.nel_junction(1, 4, 8, 16, 10, FAKE, FAKE, FAKE, FAKE, -1, None, None) == -1


def test_loss_host_validation():
    lib = nel.load()
    d = _arr(ctypes.c_int32, 8, 16, 24)
    p3 = _arr(ctypes.c_void_p, FAKE, FAKE, FAKE)
    ws_need = nel.workspace_size(nel.OP_LOSS, 3, 4, 10)

    def call(dt=1, E=3, n=4, V=10, d=d, h=p3, w=p3, labels=FAKE, alpha=0.3, gs=1.0,
             mean=FAKE, dl=None, ws=FAKE, wsb=ws_need, lam=None, div=0):
        return lib.nel_matryoshka_loss(dt, E, n, V, d, h, w, labels, alpha, gs, lam, div, None,
                                       mean, dl, ws, wsb, None)

    assert call(dt=5) == -3
    assert call(E=0) == -1
    assert call(E=9) == -1
    assert call(n=-1) == -2
    assert call(V=0) == -2
    assert call(d=_arr(ctypes.c_int32, 8, 8, 24)) == -2        # widths must increase strictly
    assert call(d=_arr(ctypes.c_int32, 0, 8, 24)) == -2
    assert call(alpha=1.5) == -1
    assert call(alpha=float("nan")) == -1
    assert call(gs=float("inf")) == -1
    assert call(mean=None) == -1
    assert call(labels=None) == -1
    assert call(h=_arr(ctypes.c_void_p, FAKE, MIS, FAKE)) == -4
    assert call(ws=None) == -5
    assert call(wsb=ws_need - 1) == -5
    assert call(dl=_arr(ctypes.c_void_p, FAKE, None, FAKE)) == -1
    assert call(div=4) == -1
    assert call(div=-1) == -1
    assert call(div=1) == -1                                 # needs the logit gradient buffers
    assert call(lam=_arr(ctypes.c_float, 1.0, -0.5, 1.0)) == -1
    assert call(lam=_arr(ctypes.c_float, 1.0, float("nan"), 1.0)) == -1
    assert call(lam=_arr(ctypes.c_float, 1.0, float("inf"), 1.0)) == -1


def test_heads_and_accept_host_validation():
    lib = nel.load()
    d = _arr(ctypes.c_int32, 8, 24)
    p2 = _arr(ctypes.c_void_p, FAKE, FAKE)
    need = nel.workspace_size(nel.OP_HEADS, 2, 4, 10)
    assert lib.nel_exit_heads(3, 2, 4, 10, d, p2, p2, None, FAKE, FAKE, need, None) == -3
    assert lib.nel_exit_heads(1, 2, 4, 10, d, p2, p2, None, FAKE, FAKE, need - 1, None) == -5
    assert lib.nel_exit_heads(1, 2, 4, 10, d, p2, p2, None, MIS4, FAKE, need, None) == -4
    assert lib.nel_exit_heads(1, 2, 4, 10, d, p2, p2, None, FAKE, MIS, need, None) == -4
    assert lib.nel_accept_prefix(4, 7, 6, MIS4, FAKE, FAKE, None) == -4
    assert lib.nel_exit_heads(1, 2, 4, 0, d, p2, p2, None, FAKE, FAKE, need, None) == -2
    assert lib.nel_accept_prefix(4, 7, 8, FAKE, FAKE, FAKE, None) == -2
    assert lib.nel_accept_prefix(4, 7, -1, FAKE, FAKE, FAKE, None) == -2
    assert lib.nel_accept_prefix(4, 7, 6, None, FAKE, FAKE, None) == -1
    assert lib.nel_accept_prefix(0, 7, 6, None, None, None, None) == 0
    assert lib.nel_read_device_flags(None, None, None) == -1
    assert lib.nel_timing_read(99, None, None) == -1


def test_packed_host_validation():
    lib = nel.load()
    # nel_pack_weights: bf16 only, V % 32 == 0, d % 64 == 0, distinct aligned buffers
    assert lib.nel_pack_weights(0, 64, 128, FAKE, FAKE + 65536, None) == -3
    assert lib.nel_pack_weights(1, 48, 128, FAKE, FAKE + 65536, None) == -2
    assert lib.nel_pack_weights(1, 64, 96, FAKE, FAKE + 65536, None) == -2
    assert lib.nel_pack_weights(1, 0, 128, FAKE, FAKE + 65536, None) == -2
    assert lib.nel_pack_weights(1, 64, 128, None, FAKE, None) == -1
    assert lib.nel_pack_weights(1, 64, 128, MIS, FAKE + 65536, None) == -4
    assert lib.nel_pack_weights(1, 64, 128, FAKE, FAKE + 1024, None) == -1   # overlapping
    d = _arr(ctypes.c_int32, 64, 128, 192)
    p3 = _arr(ctypes.c_void_p, FAKE, FAKE, FAKE)
    ws_need = nel.workspace_size(nel.OP_LOSS, 3, 4, 256)

    def loss(dt=1, V=256, d=d, dl=p3, alpha=0.3, div=0):
        return lib.nel_matryoshka_loss_packed(dt, 3, 4, V, d, p3, p3, FAKE, alpha, 1.0, None, div,
                                              None, FAKE, dl, FAKE, ws_need, None)

    assert loss(dt=0) == -3                                    # fp32 has no packed form
    assert loss(V=100) == -2
    assert loss(V=1 << 24) == -2                               # 32-bit scratch-store ranges
    assert loss(d=_arr(ctypes.c_int32, 64, 128, 200)) == -2    # a width not a multiple of 64
    assert loss(d=_arr(ctypes.c_int32, 64, 64, 192)) == -2
    assert loss(dl=None) == -1                                 # gradients are required
    assert loss(alpha=-0.1) == -1
    d2 = _arr(ctypes.c_int32, 64, 192)
    p2 = _arr(ctypes.c_void_p, FAKE, FAKE)
    need = nel.workspace_size(nel.OP_HEADS, 2, 4, 256)
    assert lib.nel_exit_heads_packed(0, 2, 4, 256, d2, p2, p2, None, FAKE, FAKE, need, None) == -3
    assert lib.nel_exit_heads_packed(1, 2, 4, 250, d2, p2, p2, None, FAKE, FAKE, need, None) == -2
    assert lib.nel_exit_heads_packed(1, 2, 4, 1 << 24, d2, p2, p2, None, FAKE, FAKE, need,
                                     None) == -2
    assert lib.nel_exit_heads_packed(1, 2, 4, 256, _arr(ctypes.c_int32, 64, 100), p2, p2, None,
                                     FAKE, FAKE, need, None) == -2
    assert lib.nel_exit_heads_packed(1, 2, 4, 256, _arr(ctypes.c_int32, 64, 1 << 24), p2, p2,
                                     None, FAKE, FAKE, need, None) == -2   # 32-bit slice offsets


def test_noalloc_host_validation():
    """The allocation-free exit heads: the same host checks as
    nel_exit_heads_packed, and a request beyond the fixed scratch is refused
    before any device call (this runs without a GPU)."""
    lib = nel.load()
    d2 = _arr(ctypes.c_int32, 64, 192)
    p2 = _arr(ctypes.c_void_p, FAKE, FAKE)
    f = lib.nel_exit_heads_packed_noalloc
    assert f(0, 2, 4, 256, d2, p2, p2, None, FAKE, None) == -3
    assert f(1, 2, 4, 250, d2, p2, p2, None, FAKE, None) == -2
    assert f(1, 2, 4, 256, _arr(ctypes.c_int32, 64, 100), p2, p2, None, FAKE, None) == -2
    assert f(1, 0, 4, 256, d2, p2, p2, None, FAKE, None) == -1
    assert f(1, 2, 4, 256, d2, p2, p2, None, MIS4, None) == -4
    # partial results need 256 + 8 n_exits n_tokens ceil(V / 128) bytes of 16 MiB
    assert f(1, 2, 4096, 32768, d2, p2, p2, None, FAKE, None) == nel.ETOOLARGE
    assert f(1, 2, 4, 256, d2, p2, p2, None, None, None) == 0      # nothing asked: nothing launched
    assert f(1, 2, 0, 256, d2, p2, p2, None, FAKE, None) == 0      # no tokens
    assert "fixed scratch" in nel.status_string(nel.ETOOLARGE)


def test_head_backward_host_validation():
    lib = nel.load()
    need = nel.head_backward_workspace_size(100, 256, 128)
    assert need > 0
    assert nel.head_backward_workspace_size(100, 250, 128) == 0
    assert nel.head_backward_workspace_size(100, 256, 96) == 0

    def call(dt=1, n=100, V=256, d=128, g=FAKE, h=FAKE, w=FAKE, dh=FAKE, dw=FAKE, ws=FAKE,
             wsb=need):
        return lib.nel_head_backward(dt, n, V, d, g, h, w, dh, dw, ws, wsb, None)

    assert call(dt=0) == -3                 # bf16 only
    assert call(V=250) == -2
    assert call(d=100) == -2
    assert call(d=1 << 22) == -2            # output row offsets stay 32-bit within a tile
    assert call(n=-1) == -2
    assert call(dh=None, dw=None) == -1     # nothing to compute
    assert call(g=None) == -1
    assert call(h=MIS) == -4
    assert call(dw=MIS) == -4
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5


def test_heads_backward_host_validation():
    lib = nel.load()
    d2 = _arr(ctypes.c_int32, 64, 128)
    need = nel.heads_backward_workspace_size(100, 256, [64, 128])
    assert need == (nel.head_backward_workspace_size(100, 256, 64)
                    + nel.head_backward_workspace_size(100, 256, 128))
    assert nel.heads_backward_workspace_size(100, 256, [64, 96]) == 0
    assert lib.nel_heads_backward_workspace(0, 100, 256, d2) == 0
    assert lib.nel_heads_backward_workspace(9, 100, 256, d2) == 0
    assert lib.nel_heads_backward_workspace(2, 100, 256, None) == 0
    p2 = _arr(ctypes.c_void_p, FAKE, FAKE)

    def call(dt=1, E=2, n=100, V=256, d=d2, g=p2, h=p2, w=p2, dh=p2, dw=p2, ws=FAKE, wsb=need):
        return lib.nel_heads_backward(dt, E, n, V, d, g, h, w, dh, dw, ws, wsb, None)

    assert call(dt=0) == -3                 # bf16 only
    assert call(E=0) == -1
    assert call(E=9) == -1
    assert call(d=None) == -1
    assert call(V=250) == -2
    assert call(d=_arr(ctypes.c_int32, 64, 100)) == -2
    assert call(n=-1) == -2
    assert call(dh=None, dw=None) == -1     # nothing to compute
    assert call(g=None) == -1
    assert call(h=_arr(ctypes.c_void_p, FAKE, None)) == -1
    assert call(dw=_arr(ctypes.c_void_p, None, FAKE)) == -1
    assert call(h=_arr(ctypes.c_void_p, FAKE, MIS)) == -4
    assert call(dh=_arr(ctypes.c_void_p, MIS, FAKE)) == -4
    assert call(ws=MIS) == -4
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5


def test_loss_backward_host_validation():
    """Every call below fails a host check before the first launch (FAKE
    pointers are never dereferenced)."""
    lib = nel.load()
    d2 = _arr(ctypes.c_int32, 64, 128)
    need = nel.loss_backward_workspace_size(100, 256, [64, 128])
    assert need > nel.heads_backward_workspace_size(100, 256, [64, 128])
    assert nel.loss_backward_workspace_size(100, 256, [64, 96]) == 0
    assert nel.loss_backward_workspace_size(100, 250, [64, 128]) == 0
    assert lib.nel_loss_backward_workspace(9, 100, 256, d2) == 0
    p2 = _arr(ctypes.c_void_p, FAKE, FAKE)

    def call(dt=1, E=2, n=100, V=256, d=d2, h=p2, w=p2, wp=p2, labels=FAKE, alpha=0.3, gs=1.0,
             lam=None, tok=FAKE, mean=FAKE, scr=p2, dh=p2, dw=p2, ws=FAKE, wsb=need):
        return lib.nel_matryoshka_loss_backward_packed(dt, E, n, V, d, h, w, wp, labels, alpha,
                                                       gs, lam, tok, mean, scr, dh, dw, ws, wsb,
                                                       None)

    assert call(dt=0) == -3                 # bf16 only
    assert call(E=0) == -1
    assert call(E=9) == -1
    assert call(d=None) == -1
    assert call(V=250) == -2                # vocabulary a multiple of 64
    assert call(d=_arr(ctypes.c_int32, 64, 96)) == -2
    assert call(n=-1) == -2
    assert call(dh=None, dw=None) == -1     # nothing to compute
    assert call(scr=None) == -1
    assert call(wp=_arr(ctypes.c_void_p, FAKE, None)) == -1
    assert call(dw=_arr(ctypes.c_void_p, None, FAKE)) == -1
    assert call(scr=_arr(ctypes.c_void_p, FAKE, MIS)) == -4
    assert call(dh=_arr(ctypes.c_void_p, MIS, FAKE)) == -4
    assert call(ws=MIS) == -4
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5
    # checked by the loss, still before anything is launched
    assert call(d=_arr(ctypes.c_int32, 128, 128),          # widths must increase strictly
                wsb=nel.loss_backward_workspace_size(100, 256, [128, 128])) == -2
    assert call(alpha=1.5) == -1
    assert call(gs=float("inf")) == -1
    assert call(lam=_arr(ctypes.c_float, 1.0, -1.0)) == -1
    assert call(mean=None) == -1
    assert call(labels=None) == -1
    assert call(labels=MIS4) == -4


def test_junction_backward_host_validation():
    lib = nel.load()
    need = int(lib.nel_junction_backward_workspace(10, 8, 16, 50))
    assert need > 0
    assert lib.nel_junction_backward_workspace(10, 8, 8, 50) == 0
    assert lib.nel_junction_backward_workspace((1 << 30) + 1, 8, 16, 50) == 0

    def call(dt=1, n=10, d_in=8, d_out=16, V=50, h=FAKE, ids=FAKE, emb=FAKE, dout=FAKE, sg=0,
             dh=FAKE, demb=FAKE, ws=FAKE, wsb=need, mode=0):
        return lib.nel_junction_backward(dt, n, d_in, d_out, V, h, ids, emb, dout, sg, mode, dh, demb,
                                         None, ws, wsb, None)

    assert call(dt=4) == -3
    assert call(d_out=8) == -2
    assert call(V=0) == -2
    assert call(n=(1 << 30) + 1) == -2
    assert call(mode=3) == -1
    assert call(dh=None, demb=None) == -1
    assert call(d_in=0, h=None) == -1          # block 1 has no dh
    assert call(h=None) == -1
    assert call(ids=MIS4) == -4
    assert call(demb=MIS) == -4
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5


def test_speculative_host_validation():
    lib = nel.load()
    need = int(lib.nel_speculative_workspace(4, 6))
    assert need >= 16 * 2 * 4 * 7

    def call(B=4, P=7, L=6, V=100, T=1.0, tp=0.9, dl=FAKE, vl=FAKE, tok=FAKE, ua=FAKE, un=FAKE,
             acc=FAKE, nxt=FAKE, ws=FAKE, wsb=need):
        return lib.nel_speculative_verify(B, P, L, V, dl, vl, tok, ua, un, T, tp, None, acc, nxt,
                                          None, ws, wsb, None)

    assert call(P=6) == -2                  # needs draft_len + 1 positions
    assert call(V=40000) == -2
    assert call(T=0.0) == -1
    assert call(T=float("nan")) == -1
    assert call(tp=0.0) == -1
    assert call(tp=1.5) == -1
    assert call(dl=None) == -1
    assert call(tok=MIS4) == -4
    assert call(wsb=need // 2) == -5
    assert call(B=0, dl=None, vl=None, tok=None, ua=None, un=None, acc=None, nxt=None) == 0


def test_one_hip_runtime_after_load():
    """libnel.so binds to the HIP runtime PyTorch carries (same soname), never a second one."""
    nel.load()
    rts = nel._hip_runtimes()
    assert len(rts) == 1, rts


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "nested_exit_lm_amd")
    for dp, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dp, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", txt, re.M), f
                assert "oracle/" not in txt, f


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(nel, "_LIB", None)
    monkeypatch.setattr(nel, "_HERE", str(tmp_path))
    with pytest.raises(ImportError):
        nel.load()
