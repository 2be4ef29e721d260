"""The matrix-core throughput probe behind bench.py's mfma_ceiling: it runs through the C ABI,
writes every sink element, and its rate lies between a fifth of the published dense bf16 peak
and that peak (2.5 PFLOP/s)."""

import pytest
import torch

from attention_relation_distillation_amd import relkl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("vector_work", [False, True])
def test_probe_rate_is_within_the_published_peak(vector_work):
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.full((cus * relkl.PROBE_THREADS,), float("nan"), device=dev)
    iters = 400
    relkl.probe_mfma(vector_work, iters, cus, sink)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    relkl.probe_mfma(vector_work, iters, cus, sink)
    e1.record()
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    flops = cus * 8 * iters * relkl.PROBE_MFMA_PER_ITER * relkl.PROBE_FLOPS_PER_MFMA
    tflops = flops / (e0.elapsed_time(e1) / 1e3) / 1e12
    print(f"probe vector_work={vector_work}: {tflops:.1f} TFLOP/s on {cus} CUs")
    assert 500.0 < tflops < 2500.0
