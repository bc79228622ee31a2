"""nel_exit_heads_packed_noalloc, the allocation-free entry point, against
nel_exit_heads_packed, the entry point with a workspace: the same argmax and
the same fp32 logits, bit for bit.  Two calls in a row, the second with fewer
tokens, so that the library's fixed scratch still holds the first call's
values when the second runs; and the largest request the scratch admits, with
the next larger one refused before anything is launched."""
import pytest

import synth
from gpu_util import DevSuite, log

pytestmark = pytest.mark.gpu


def compare(nel, hs, pw, want_logits):
    import torch
    dev = hs[0].device
    ref_l, ref_a = nel.exit_heads_packed(hs, pw, want_logits=want_logits, want_argmax=True)
    n, V = hs[0].shape[0], pw[0].shape[0]
    lg = ([torch.full((n, V), float("nan"), dtype=torch.float32, device=dev) for _ in hs]
          if want_logits else None)
    am = torch.full((len(hs), n), -1, dtype=torch.int32, device=dev)
    nel.exit_heads_packed_noalloc(hs, pw, logits=lg, argmax=am)
    torch.cuda.synchronize()
    assert torch.equal(am, ref_a), "argmax differs"
    if want_logits:
        for e, (a, b) in enumerate(zip(lg, ref_l)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"logits of exit {e} differ"


def test_noalloc_matches_workspace_entry_point(nel):
    """The verify shape (exits 1 and 3 of the 500M/1.5B/3B suite, 102 x 7
    tokens, V = 32768), then its first 100 tokens."""
    s = synth.make_workload(4)
    ds = DevSuite(s, exits=s.exits)
    pw = [nel.pack_weights(w) for w in ds.w]
    log(f"[noalloc] call 1: {s.n_tokens} tokens, widths {[h.shape[1] for h in ds.h]}")
    compare(nel, ds.h, pw, want_logits=True)
    log("[noalloc] call 2: 100 tokens")
    compare(nel, [h[:100] for h in ds.h], pw, want_logits=False)


def test_noalloc_largest_request(nel):
    """Two exits at V = 32768 need 256 + 8 x 2 x n x 256 bytes: 4095 tokens fit
    the 16 MiB scratch, 4096 do not (NEL_ETOOLARGE, nothing launched)."""
    import torch
    s = synth.make_suite((64, 128), 32768, 1, 4096, seed=61)
    ds = DevSuite(s)
    pw = [nel.pack_weights(w) for w in ds.w]
    log("[noalloc] largest request: 4095 tokens x 2 exits")
    compare(nel, [h[:4095] for h in ds.h], pw, want_logits=False)
    am = torch.empty(2, 4096, dtype=torch.int32, device=ds.h[0].device)
    with pytest.raises(nel.NelError) as err:
        nel.exit_heads_packed_noalloc(ds.h, pw, argmax=am)
    assert err.value.status == nel.ETOOLARGE
    log("[noalloc] then a small call after the refused one")
    compare(nel, [h[:37] for h in ds.h], pw, want_logits=True)
