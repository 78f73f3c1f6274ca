"""GPU: the arithmetic shortcuts inside the kernels agree with the IEEE
operations they replace over every input bit pattern of their ranges
(pact_selftest_arith): the FMA-corrected reciprocal and division by 6 used
for block scales and element quotients, the sigmoid's division, the
hardware BF16 conversion and the hardware E4M3 conversions of the row
kernels' block scales.  Parity of the kernels themselves is checked
element by element against the oracle elsewhere; this pins the shortcuts
over the inputs those tests cannot enumerate."""

import pytest

pytestmark = pytest.mark.gpu


def test_arith_shortcuts_exhaustive():
    import frozen_weight_gemms_amd as fw
    counts = fw.selftest_arith()
    names = ["reciprocal", "division by 6", "sigmoid", "bf16 conversion", "e4m3 conversions"]
    assert counts == [0, 0, 0, 0, 0], dict(zip(names, counts))


def test_mfma_probe_rates():
    """The MFMA-loop probe runs both instruction kinds and reports a rate and a
    clock inside physical limits (it is a measurement aid for the GEMM
    rooflines, so only plausibility is checked)."""
    import frozen_weight_gemms_amd as fw
    for kind, peak in ((0, 2500.0), (1, 10100.0)):
        tflops, ghz = fw.mfma_probe(kind, iters=500)
        assert 0.1 * peak < tflops < 1.05 * peak, (kind, tflops)
        assert 0.5 < ghz < 3.0, (kind, ghz)
