"""The CPU oracle against its pins (library routines, brute force, format facts,
hand-worked fixtures and invariants).  No GPU needed."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("check", P.FAST_CHECKS, ids=lambda c: c.__name__)
def test_pin(o, check):
    check(o)


def test_mx_encode_exhaustive_all_scale_codes(o):
    """Every finite bf16 pattern under every finite E8M0 code (16.6 M elements)."""
    P.check_mx_encode_exhaustive(o)


def test_mx_encode_exact_rational_sample(o):
    P.check_mx_encode_fraction_sample(o)


def test_brute_force_helper_itself():
    """The midpoint brute force agrees with torch's clamped cast on its own."""
    import numpy as np
    import torch
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(100000) * np.exp2(rng.integers(-14, 10, 100000))).astype(np.float32)
    ref = torch.from_numpy(y.copy()).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(P.nearest_even_e4m3_codes(y.astype(np.float64)), ref)
