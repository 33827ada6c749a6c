"""Pins of the oracle's number decoders (CPU only).

The fp8 table is checked against the E4M3 definition's closed-form values and against torch's
own float8 -> float64 conversion of all 256 bytes (a library routine, independent of the
oracle); bf16 against torch's bfloat16 -> float64 conversion."""
import math

import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("byte,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0x3C, 1.5), (0x7E, 448.0),
    (0xFE, -448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0xB8, -1.0), (0x80, -0.0),
])
def test_e4m3fn_closed_forms(byte, value):
    v = oracle.e4m3_value(byte, fnuz=False)
    assert v == value and math.copysign(1.0, v) == math.copysign(1.0, value)


def test_e4m3fn_nan_patterns():
    nans = [b for b in range(256) if math.isnan(oracle.e4m3_value(b, False))]
    assert nans == [0x7F, 0xFF]


@pytest.mark.parametrize("byte,value", [
    (0x00, 0.0), (0x38, 0.5), (0x40, 1.0), (0x7F, 240.0), (0xFF, -240.0), (0x01, 2.0 ** -10),
    (0x08, 2.0 ** -7),
])
def test_e4m3fnuz_closed_forms(byte, value):
    assert oracle.e4m3_value(byte, fnuz=True) == value


def test_e4m3fnuz_nan_pattern():
    nans = [b for b in range(256) if math.isnan(oracle.e4m3_value(b, True))]
    assert nans == [0x80]


@pytest.mark.parametrize("fnuz", [False, True])
def test_e4m3_table_matches_torch(fnuz):
    dt = torch.float8_e4m3fnuz if fnuz else torch.float8_e4m3fn
    ref = torch.arange(256, dtype=torch.uint8).view(dt).to(torch.float64).numpy()
    got = oracle.e4m3_table(fnuz)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_bf16_matches_torch():
    g = torch.Generator().manual_seed(7)
    bits = torch.randint(0, 1 << 16, (4096,), generator=g, dtype=torch.int32)
    bits = torch.cat([bits, torch.tensor([0, 0x8000, 0x3F80, 0x7F7F, 0x0001, 0x7F80, 0xFF80])])
    ref = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b) & 0xFFFF) for b in bits])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
