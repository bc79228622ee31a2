"""The matrix-core rate probe (nel_probe_mfma): with all-ones operands every
MFMA 32x32x16 adds 16 to each of a lane's 16 accumulators; 8 MFMAs per
iteration over 4 chains give each accumulator 32 per iteration, so a
wavefront's sum is 64 lanes x 64 accumulators x 32 x iters = 131072 x iters
(exact in fp32 for the sizes used)."""
import pytest

pytestmark = pytest.mark.gpu


def test_probe_all_ones(nel):
    import torch
    ops = torch.ones(16, 64, 8, dtype=torch.bfloat16, device="cuda:0")
    for iters in (1, 7):
        sink = nel.probe_mfma(ops, iters, 3)
        torch.cuda.synchronize()
        assert sink.shape == (12,)
        assert torch.all(sink == 131072.0 * iters), sink
