"""Pins of the oracle's group quantizer: exact round trip of on-grid data,
nearest-grid-point codes by brute force, the error bound, degenerate groups."""
import numpy as np
import pytest

import oracle as O


def _fp8_positive_normals():
    v = O.fp8_decode(np.arange(0x08, 0x7F, dtype=np.uint8))
    return np.arange(0x08, 0x7F), v


@pytest.mark.parametrize("bits", [2, 4])
def test_on_grid_round_trip_is_exact(bits):
    rng = np.random.default_rng(10 + bits)
    Q = (1 << bits) - 1
    scodes, svals = _fp8_positive_normals()
    for trial in range(400):
        si = rng.integers(0, 60)             # keep scale moderate so s*Q+z stays exact
        sc, s = int(scodes[si]), svals[si]
        zc = int(rng.integers(0, 0x7E)) | (0x80 if rng.random() < 0.5 else 0)
        z = O.fp8_decode([zc])[0]
        c = rng.integers(0, Q + 1, 16)
        i0, i1 = rng.choice(16, 2, replace=False)
        c[i0], c[i1] = 0, Q
        x = s * c + z
        s8, z8, codes = O.quant_group(x, bits)
        assert s8 == sc
        assert O.fp8_decode([z8])[0] == z     # the byte may differ only for +-0
        assert np.array_equal(codes, c)


def _brute_codes(x, s, z, Q):
    grid = s * np.arange(Q + 1) + z
    dist = np.abs(x[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    out = []
    for i in range(len(x)):
        cand = np.nonzero(dist[i] == best[i])[0]
        even = [c for c in cand if c % 2 == 0]
        out.append(even[0] if len(cand) > 1 and even else cand[0])
    return np.array(out)


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_nearest_grid_point(bits):
    rng = np.random.default_rng(20 + bits)
    Q = (1 << bits) - 1
    for trial in range(500):
        x = rng.standard_normal(16) * rng.choice([0.01, 0.3, 1.0, 30.0])
        s8, z8, codes = O.quant_group(x, bits)
        s, z = O.fp8_decode([s8, z8])
        assert s > 0
        assert np.array_equal(codes, _brute_codes(x, s, z, Q))


@pytest.mark.parametrize("bits", [2, 4])
def test_scale_and_offset_come_from_min_and_range(bits):
    # With the scale rounding down, the max element falls past Q and is clamped;
    # with the offset rounding up, the min element falls below 0 and is clamped.
    # In all cases every reconstructed element lies within half a step of the
    # input or at the clamped end of the grid.
    rng = np.random.default_rng(30 + bits)
    Q = (1 << bits) - 1
    for trial in range(500):
        x = rng.standard_normal(16) * rng.choice([0.05, 1.0, 20.0])
        s8, z8, codes = O.quant_group(x, bits)
        s, z = O.fp8_decode([s8, z8])
        xh = s * codes + z
        lo, hi = z, s * Q + z
        inside = (x >= lo - s / 2) & (x <= hi + s / 2)
        assert np.all(np.abs(x - xh)[inside] <= s / 2 + 1e-15)
        assert np.all(xh[~inside & (x < lo)] == lo)
        assert np.all(xh[~inside & (x > hi)] == hi)
        # scale is within one fp8 rounding of range/Q, offset within one of min
        assert abs(s - (x.max() - x.min()) / Q) <= 0.0625 * (x.max() - x.min()) / Q + 2.0 ** -10
        assert abs(z - x.min()) <= 0.0625 * abs(x.min()) + 2.0 ** -10


def test_constant_group_is_degenerate():
    x = np.full(16, 0.75)
    s8, z8, codes = O.quant_group(x, 4)
    assert s8 == 0
    assert O.fp8_decode([z8])[0] == 0.75
    assert np.all(codes == 0)


def test_dequant_vector_uses_per_group_parameters():
    codes = np.arange(32, dtype=np.uint8) % 4
    s8 = O.fp8_encode([0.5, 2.0])
    z8 = O.fp8_encode([-1.0, 3.0])
    out = O.dequant_vector(codes, s8, z8, 16)
    assert np.array_equal(out[:16], 0.5 * (np.arange(16) % 4) - 1.0)
    assert np.array_equal(out[16:], 2.0 * (np.arange(16, 32) % 4) + 3.0)
