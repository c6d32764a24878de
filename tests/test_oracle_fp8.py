"""Pins of the oracle's FP8 E4M3 decoding (the index branch's lighter input
format, "How to solve the memory problem with MiniMax Sparse Attention",
'Kernel optimizations').  Values are fixed by the OCP 8-bit floating point
format: bias 7, 3 mantissa bits, subnormals at exponent field 0, no
infinities, and S.1111.111 as NaN."""

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x30, 0.5), (0xB8, -1.0), (0xC0, -2.0),
    (0x3C, 1.5), (0x7E, 448.0), (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x0F, 1.875 * 2.0 ** -6), (0x77, 1.875 * 2.0 ** 7), (0x70, 128.0), (0x78, 256.0),
])
def test_decode_values_from_the_format(code, value):
    assert O.decode_e4m3(np.array([code]))[0] == value


def test_negative_zero_and_nan_codes():
    v = O.decode_e4m3(np.array([0x80, 0x7F, 0xFF]))
    assert v[0] == 0.0 and np.signbit(v[0])
    assert np.isnan(v[1]) and np.isnan(v[2])


def test_positive_codes_increase_and_signs_mirror():
    pos = O.decode_e4m3(np.arange(0x00, 0x7F))
    assert np.all(np.diff(pos) > 0)
    neg = O.decode_e4m3(np.arange(0x80, 0xFF))
    np.testing.assert_array_equal(neg, -pos)


def test_agrees_with_torch_float8_e4m3fn_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), codes[~same]


def test_small_integers_are_exact():
    # {-2..2} are exactly representable, so FP8 index scores of such inputs
    # are exact integers as in the bf16 / fp32 branches.
    for x in (-2.0, -1.0, 0.0, 1.0, 2.0):
        code = torch.tensor([x]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert O.decode_e4m3(code)[0] == x
