"""GPU check of the measurement probes (include/grok_moe_probe.h) that give the bench its ceilings: the MFMA-only
kernel in each issue order and with zero A operands, and the prefill tiles' K loop fed from LDS without and with its
copies, each compute the sums the host expects from their operands (short runs; the sums are checked in float64 by
bench.py's probe wrapper, which these tests call)."""
import pytest
import torch

from tests._helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    import bench
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return bench.Probe(gm)


@pytest.mark.parametrize("order,zero_a", [(0, False), (1, False), (2, False), (0, True)])
def test_mfma_probe_sums(probe, order, zero_a):
    say(f"[case] mfma probe order={order} zero_a={zero_a}")
    r = probe.mfma(iters=2000, order=order, zero_a=zero_a)
    say(f"[result] {r['TFLOPs']:.0f} TFLOP/s at {r['clock_GHz']:.2f} GHz, max err {r['checksum_max_err']:.2e}")
    assert r["checksum_ok"]


@pytest.mark.parametrize("copies", [0, 1])
def test_feed_probe_sums(probe, copies):
    say(f"[case] feed probe copies={copies}")
    r = probe.feed(copies=copies, iters=1000, images=8)
    say(f"[result] {r['TFLOPs']:.0f} TFLOP/s at {r['clock_GHz']:.2f} GHz, max rel err {r['checksum_max_rel_err']:.2e}")
    assert r["checksum_ok"]
