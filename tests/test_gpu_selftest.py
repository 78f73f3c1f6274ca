"""GPU: the arithmetic shortcuts inside the kernels agree with the IEEE
operations they replace over every input bit pattern of their ranges
(pact_selftest_arith): the FMA-corrected reciprocal and division by 6 used
for block scales and element quotients, the sigmoid's division, and the
hardware BF16 conversion.  Parity of the kernels themselves is checked
element by element against the oracle elsewhere; this pins the shortcuts
over the inputs those tests cannot enumerate."""

import pytest

pytestmark = pytest.mark.gpu


def test_arith_shortcuts_exhaustive():
    import frozen_weight_gemms_amd as fw
    counts = fw.selftest_arith()
    names = ["reciprocal", "division by 6", "sigmoid", "bf16 conversion"]
    assert counts == [0, 0, 0, 0], dict(zip(names, counts))
