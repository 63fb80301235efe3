"""The oracle against its pins (CPU only). See tests/pins.py for what each pin fixes."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: getattr(p, "__name__", "pin"))
def test_pin(pin):
    pin(oracle)


def test_state_arithmetic_of_the_decode_workload():
    # 28 layers x 256 sequences x 8192 channels x 16 states in fp32: the state the
    # batched-decode workload keeps resident (939,524,096 values, 3.76 GB).
    assert oracle.state_bytes(28, 256 * 8192, 16, 4) == 939524096 * 4 == 3758096384


def test_bf16_widening_is_exact():
    import numpy as np
    import torch
    v = torch.tensor([1.0, -2.5, 3.140625, 65280.0, 1e-30, -0.0], dtype=torch.bfloat16)
    w = oracle.to_f64(v)
    assert w.dtype == np.float64
    assert np.array_equal(w, v.to(torch.float64).numpy())
