"""The matrix-core throughput probe behind bench.py's measured ceiling.

Every thread's sink value is the sum of its 16 accumulators after `iters`
rounds of one fixed bf16 product, so it is `iters` times the one-round value
(up to fp32 rounding of the running sums), and it is the same on every run."""
import pytest
import torch


@pytest.mark.gpu
def test_probe_runs_scales_and_repeats(gpu_lib):
    mv = gpu_lib
    blocks = 8
    dev = torch.device("cuda:0")
    s1 = torch.full((blocks * 256,), float("nan"), device=dev)
    s4 = torch.full_like(s1, float("nan"))
    again = torch.full_like(s1, float("nan"))
    f1 = mv.probe_mfma_bf16(blocks, 1, s1)
    f4 = mv.probe_mfma_bf16(blocks, 4, s4)
    mv.probe_mfma_bf16(blocks, 1, again)
    torch.cuda.synchronize()
    assert f1 == blocks * 4 * 16 * 2 * 32 * 32 * 16 and f4 == 4 * f1
    assert torch.isfinite(s1).all() and torch.isfinite(s4).all()
    assert s1.abs().max() > 0
    assert torch.allclose(s4, 4 * s1, rtol=1e-4, atol=1e-2)
    assert torch.equal(again, s1)
