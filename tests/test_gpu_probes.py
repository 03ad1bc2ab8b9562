"""The measurement probes on the GPU: their results are exact, so a probe that
skipped work (or ran the wrong instruction) fails here before it reports a
rate."""
import pytest
import torch

import paged_kv_cache_193_amd as pkv

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters", [1, 1000, 4096])
def test_mfma_probe_result_is_exact(iters):
    """Every operand element is 2^-4, so each of the 4 chains adds 2^-4 to
    each of its 16 accumulator elements per round: every lane folds to
    4 * iters exactly."""
    sink = torch.full((pkv.STREAM_SINK_BYTES // 4,), float("nan"), dtype=torch.float32,
                      device="cuda")
    pkv.mfma_probe(iters, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 4.0 * iters)
