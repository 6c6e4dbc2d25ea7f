"""Pins of the oracle's number formats (FP8 e4m3fn and BF16) against the format
definitions and against torch's own casts, which are independent library
implementations of the same IEEE/OCP rounding."""
import numpy as np
import pytest
import torch

import oracle as O


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x39, 1.125), (0x7E, 448.0), (0xB8, -1.0), (0xC0, -2.0), (0xFE, -448.0)])
def test_fp8_decode_spec_points(code, value):
    # OCP 8-bit floating point spec, E4M3: bias 7, max normal 448, min normal 2^-6,
    # min subnormal 2^-9.
    assert O.fp8_decode([code])[0] == value


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * rng.choice([1e-3, 1e-2, 0.1, 1, 10, 100], 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),
    ]).astype(np.float32).astype(np.float64)
    ours = O.fp8_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_encode_ties_go_to_even():
    vals = O.fp8_decode(np.arange(0, 0x7F, dtype=np.uint8))  # non-negative finite, ascending
    mids = (vals[:-1] + vals[1:]) / 2
    ours = O.fp8_encode(mids)
    lo = np.arange(0, 0x7E, dtype=np.uint8)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(ours, expect)
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # just above / below a midpoint leaves the tie
    assert O.fp8_encode([np.nextafter(mids[56], np.inf)])[0] == 57
    assert O.fp8_encode([np.nextafter(mids[57], -np.inf)])[0] == 57


def test_fp8_encode_saturates_and_keeps_sign_of_zero():
    assert list(O.fp8_encode([448.0, 460.0, 480.0, 1e6, -1e6])) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert O.fp8_encode([-1e-5])[0] == 0x80
    assert O.fp8_encode([1e-5])[0] == 0x00
    assert O.fp8_encode([2.0 ** -10])[0] == 0x00          # tie between 0 and 2^-9 -> even (0)
    assert O.fp8_encode([3 * 2.0 ** -10])[0] == 0x02      # tie between 1 and 2 (x 2^-9) -> 2


def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_encode_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(50000) * rng.choice([1e-30, 1e-3, 1, 1e3, 1e30], 50000),
        rng.uniform(-2, 2, 50000),
    ]).astype(np.float32)
    ours = O.bf16_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_rounds_from_double_directly():
    # 1 + 2^-8 is the exact midpoint between 1.0 (0x3F80) and 1+2^-7 (0x3F81).
    assert O.bf16_encode([1 + 2.0 ** -8])[0] == 0x3F80               # tie -> even
    assert O.bf16_encode([1 + 3 * 2.0 ** -8])[0] == 0x3F82           # tie -> even
    # Slightly above the midpoint: a detour through binary32 would land on the
    # tie and round down; the direct rounding must go up.
    assert O.bf16_encode([1 + 2.0 ** -8 + 2.0 ** -40])[0] == 0x3F81
    assert O.bf16_encode([-(1 + 2.0 ** -8 + 2.0 ** -40)])[0] == 0xBF81
    assert O.bf16_encode([0.0])[0] == 0x0000
    assert O.bf16_encode([-0.0])[0] == 0x8000
    assert O.bf16_encode([3.4e38])[0] == 0x7F80                       # beyond max+half ulp
    assert O.bf16_encode([2.0 ** -133])[0] == 0x0001                  # smallest subnormal
