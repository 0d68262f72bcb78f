"""CPU pins of the fp64 oracle (each pin is described in tests/oracle_pins.py)."""

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_decode_matches_torch_widening():
    import numpy as np
    import torch
    x = (torch.randn(4096) * 1e3).to(torch.bfloat16)
    assert np.array_equal(oracle.decode_bf16(x), x.double().numpy())
