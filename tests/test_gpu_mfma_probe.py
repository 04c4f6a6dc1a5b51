"""The MFMA-only probe reports a plausible bf16 rate and clock (a fact about the
part that bounds every GEMM on it; not compared with any page)."""

import pytest

import persistent_tiled_gemm_amd as ptg
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_mfma_probe_rates_and_clock():
    say("case mfma probe")
    const = ptg.gemm_mfma_probe(iters=20000, random_operands=False)
    rand = ptg.gemm_mfma_probe(iters=20000, random_operands=True)
    for r in (const, rand):
        assert 0.3 < r["clock_ghz"] < 3.0, r
        # at most the dense peak at the clock it ran at (1024 flop/clk per SIMD, 1024 SIMDs), with 5% slack
        assert 0 < r["tflops"] <= 1.05 * 1.048576 * r["clock_ghz"] * 1e3, r
    with pytest.raises(ptg.PtgError):
        ptg.gemm_mfma_probe(iters=0)
