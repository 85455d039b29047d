"""The MFMA-rate probe runs on the device, reports the flop count its launch
performs, and records positive core- and reference-clock tick counts."""
import pytest

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_mfma_probe_runs_and_counts(fp8):
    import torch
    from sparse_rank_attention_amd import rola
    sink = torch.zeros(2048, dtype=torch.float32, device="cuda")
    flop = rola.mfma_probe(rola.ROLA_PREC_FP8 if fp8 else rola.ROLA_PREC_BF16, 64, sink)
    torch.cuda.synchronize()
    per_mfma = 2 * 32 * 32 * (64 if fp8 else 16)
    assert flop == per_mfma * 4 * 64 * 4 * 1024   # 4 chains x iters x 4 waves x 1024 workgroups
    ticks = sink[1024:1026].cpu().tolist()
    assert ticks[0] > 0 and ticks[1] > 0
