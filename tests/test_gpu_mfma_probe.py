"""The MFMA-only probe reports a plausible bf16 rate and clock (a fact about the
part that bounds every GEMM on it; not compared with any page)."""

import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block", [16, 32])
def test_mfma_probe_rates_and_clock(block):
    say(f"case mfma probe block={block}")
    const = ptg.gemm_mfma_probe(iters=20000, random_operands=False, mfma_block=block)
    rand = ptg.gemm_mfma_probe(iters=20000, random_operands=True, mfma_block=block)
    for r in (const, rand):
        assert 0.3 < r["clock_ghz"] < 3.0, r
        # at most the dense peak at the clock it ran at (1024 flop/clk per SIMD, 1024 SIMDs), with 5% slack,
        # and at least a third of it (the MFMAs stay in place: no accumulator copies slow the stream)
        peak_at_clock = 1.048576 * r["clock_ghz"] * 1e3
        assert peak_at_clock / 3 < r["tflops"] <= 1.05 * peak_at_clock, r
    with pytest.raises(ptg.PtgError):
        ptg.gemm_mfma_probe(iters=0)
    with pytest.raises(ptg.PtgError):
        ptg.gemm_mfma_probe(iters=100, mfma_block=8)


def test_hbm_probe_reports_a_plausible_bandwidth():
    # a plain streaming read and copy over 1 GiB: well above 1 TB/s and below the 8 TB/s data-sheet peak
    read = ptg.gemm_hbm_probe(1 << 30, "read", reps=5)
    copy = ptg.gemm_hbm_probe(1 << 30, "copy", reps=5)
    say(f"hbm probe: read {read:.0f} GB/s, copy {copy:.0f} GB/s")
    assert 1000.0 < read < 8000.0 and 1000.0 < copy < 8000.0, (read, copy)
    with pytest.raises(ptg.PtgError):
        ptg.gemm_hbm_probe(1000, "read")          # not a multiple of 4096, under 1 MiB
