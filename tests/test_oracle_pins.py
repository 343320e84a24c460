"""The CPU oracle against the pages' worked examples, independent labellers,
closed forms and invariants (see tests/oracle_pins.py)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(lib, pin):
    pin(lib)


def test_oracle_rejects_bad_arguments(lib):
    import numpy as np
    img = np.zeros((2, 2), np.uint8)
    with pytest.raises(ValueError):
        oracle.label(img, 6, lib=lib)
    with pytest.raises(TypeError):
        oracle.label(img.astype(np.float32), 8, lib=lib)
