"""The CPU oracle against its pins (see ``oracle_pins.py``)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


def test_representable_on_workload_data():
    """Every dequantized weight of 4-bit and 8-bit workload-class data is exact in binary32,
    so the fp32 value a GPU dequantization must produce is unique."""
    import numpy as np
    from seeded_inputs import draw_quantized_weight
    for bits, k in ((4, 4096), (8, 896)):
        d = draw_quantized_weight(0, 1, 1024, k, bits)
        _, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], k, bits)
        assert bad == 0
