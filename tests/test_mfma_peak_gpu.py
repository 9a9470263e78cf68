"""The measured bf16 MFMA rate (arl2_profile_mfma_peak) on the GPU.

The pure MFMA loop has no memory traffic, so its rate must sit below the
published dense bf16 peak of the part (2516.6 TFLOP/s: 256 CUs x 4 SIMDs x
1024 flop/clk x 2.4 GHz) and well above the rate of any kernel of the layer;
its clock runs near 1.9-2.4 GHz under this load, so a working loop lands at
roughly 0.6-1.0 of the published figure. The bound below is deliberately
wide (it checks that the figure is a rate of the right kind, not a tuning
target).
"""
import pytest

from parity_utils import device

pytestmark = pytest.mark.gpu

PEAK_BF16_DENSE = 2516.6


@pytest.fixture(scope="module")
def B():
    import torch  # noqa: F401
    device()
    from hybrid_softmax_gated_amd import binding
    return binding


def test_mfma_loop_rate_is_a_plausible_fraction_of_the_published_peak(B):
    rates = [B.arl2_profile_mfma_peak(4096) for _ in range(3)]
    print(f"\n[mfma peak] {', '.join(f'{r:.1f}' for r in rates)} TFLOP/s", flush=True)
    for r in rates:
        assert 0.3 * PEAK_BF16_DENSE < r < 1.05 * PEAK_BF16_DENSE


def test_mfma_loop_rate_scales_with_the_work(B):
    # Twice the rounds take about twice the time: the rate stays within 25 %.
    small = max(B.arl2_profile_mfma_peak(2048) for _ in range(2))
    large = max(B.arl2_profile_mfma_peak(8192) for _ in range(2))
    assert abs(large - small) < 0.25 * large
