"""Calls on two streams at once.  Each call without a workspace argument gets
the default workspace of its own stream, so two loss steps (and two grouped
head backwards) issued concurrently on different streams must give exactly
what the same calls give one after another on one stream: the kernels'
reductions run in a fixed order, so the comparison is bit-exact."""
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

N, V, WIDTHS = 2048, 4096, (256, 512)


def make_inputs(torch, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    hs = [(torch.randn(N, d, generator=g, device="cuda:0") * 4.0).bfloat16() for d in WIDTHS]
    ws = [(torch.randn(V, d, generator=g, device="cuda:0") * 0.02).bfloat16() for d in WIDTHS]
    labels = torch.randint(0, V, (N,), generator=g, device="cuda:0", dtype=torch.int32)
    return hs, ws, labels


def step(nel, hs, pw, ws, labels):
    mean, tok, dl = nel.matryoshka_loss_packed(hs, pw, labels, alpha_d=0.3)
    dhs, dws = nel.heads_backward(dl, hs, ws)
    return [mean, tok] + list(dl) + list(dhs) + list(dws)


def test_two_streams_match_one_stream(nel):
    import torch
    sets = [make_inputs(torch, s) for s in (81, 82)]
    packed = [[nel.pack_weights(w) for w in ws] for _, ws, _ in sets]
    torch.cuda.synchronize()
    want = [[t.clone() for t in step(nel, hs, pw, ws, lab)]
            for (hs, ws, lab), pw in zip(sets, packed)]
    torch.cuda.synchronize()
    log("[streams] sequential reference done")

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None, None]
    for rep in range(3):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                hs, ws, lab = sets[i]
                got[i] = step(nel, hs, packed[i], ws, lab)
    torch.cuda.synchronize()
    log("[streams] concurrent calls done")
    for i in range(2):
        for j, (a, b) in enumerate(zip(got[i], want[i])):
            assert torch.equal(a, b), f"set {i}, output {j} differs from the one-stream result"
