"""The measurement probe (fa_probe_mfma) runs and reports sane values: every
workgroup writes its clock and tick counts, the implied shader clock is
between 0.5 and 3 GHz, and the achieved MFMA rate is below the spec peak."""

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_probe_runs(gpu_lib):
    print("\n[case] fa_probe_mfma 512 x 256 iterations", flush=True)
    blocks, iters = 512, 256
    sink = torch.zeros(3 * blocks, device="cuda", dtype=torch.int64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_lib.fa_probe_mfma(sink, blocks, iters)
    e0.record()
    gpu_lib.fa_probe_mfma(sink, blocks, iters)
    e1.record()
    torch.cuda.synchronize()
    v = sink.view(blocks, 3).cpu()
    assert bool((v[:, 0] > 0).all()) and bool((v[:, 1] > 0).all())
    mhz = (v[:, 0].double() / v[:, 1].double()).median().item() * 100.0
    assert 500.0 < mhz < 3000.0, mhz
    tflops = blocks * 4 * iters * 4 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 0.0 < tflops < 2516.6, tflops
