"""The MFMA calibration kernel (qgalore_mfma_probe) computes the products it claims: on
constant operands every accumulator holds iters * 16 * v^2, so each lane's checksum over its
16 blocks x 16 accumulators is 256 times that."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_mfma_probe_constant_operands_checksum():
    from quantized_rank_gradient_amd import binding as B
    v = torch.tensor(0.01, dtype=torch.bfloat16).item()          # the bf16 value of 0.01
    ops = torch.full((4096,), 0.01, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(8 * 256, dtype=torch.float32, device="cuda")
    flops = B.mfma_probe(ops, out, 8, 10)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 10 * 16 * 32768
    want = 256 * 10 * 16 * v * v
    got = out.cpu().numpy()
    assert np.all(np.abs(got - want) <= 1e-4 * want), (got[:4], want)
