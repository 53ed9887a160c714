"""The fp64 oracle against its pins (tests/pins.py): code tables, torch's float8 conversion,
exact rational arithmetic, numpy's fp64 matmul, closed forms and identities."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, lib):
    pin(lib)


def test_bf16_products_exact():
    """Every (E2M1 code, finite E4M3 code) product is a bf16 value, so the dequantized weight the
    kernels feed to bf16 matrix cores can be exact. Checked with torch's own bf16 rounding."""
    import numpy as np
    import torch
    e2 = pins.E2M1_ARRAY
    e4 = pins.e4m3_torch(np.arange(256, dtype=np.uint8))
    e4 = e4[~np.isnan(e4)]
    assert e4.size == 254
    prod = torch.from_numpy(np.outer(e2, e4))
    assert torch.equal(prod.to(torch.bfloat16).to(torch.float64), prod)
