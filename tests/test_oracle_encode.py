"""Pins of the oracle's loop-group encoder and reconstruction: which loop is the
anchor, that residuals are taken against the dequantized anchor and rotated
with H while reconstruction applies H^T, least-squares optimality of alpha
(brute force and numpy lstsq), the two-read identity, and direct mode."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O


def _signs(d, seed):
    rng = np.random.default_rng(seed)
    return (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)


def _bf16_round(x):
    return O.bf16_decode(O.bf16_encode(x))


def _group_inputs(d, P, seed, sig=(0.3, 0.2, 0.1)):
    rng = np.random.default_rng(seed)
    lam = np.exp(0.5 * rng.standard_normal(d))
    anchor = rng.standard_normal(d) * lam
    x = np.empty((P, d))
    for j in range(P - 1):
        x[j] = anchor + sig[j % len(sig)] * rng.standard_normal(d)
    x[P - 1] = anchor
    return _bf16_round(x)


def _y_hat(p, codes, s8, z8, j):
    return O.dequant_vector(codes[j], s8[j], z8[j], p.g)


@pytest.mark.parametrize("d", [64, 96, 128])
def test_anchor_is_last_loop_and_unrotated(d):
    p = O.Params(d=d)
    S = _signs(d, 1)
    x = _group_inputs(d, 4, 100 + d)
    codes, s8, z8, alpha = O.encode_group(p, x, S)
    c2, s2, z2 = np.zeros(d, np.uint8), np.zeros(d // 16, np.uint8), np.zeros(d // 16, np.uint8)
    for gi in range(d // 16):
        s2[gi], z2[gi], c2[gi * 16:(gi + 1) * 16] = O.quant_group(x[3, gi * 16:(gi + 1) * 16], 4)
    assert np.array_equal(codes[3], c2) and np.array_equal(s8[3], s2) and np.array_equal(z8[3], z2)
    assert alpha[3] == 0
    assert codes[:3].max() <= 3 and codes[3].max() <= 15


@pytest.mark.parametrize("d", [64, 128])
def test_residual_is_rotated_difference_to_dequantized_anchor(d):
    """Loop l's codes quantize y = H (x_l - deq(anchor)), with H built by scipy."""
    p = O.Params(d=d)
    s = _signs(d, 2)
    Hs = scipy.linalg.hadamard(d) / np.sqrt(d) * s[None, :]
    H = O.rotation_matrix(d, s)
    n_checked = 0
    for seed in range(40):
        x = _group_inputs(d, 4, 200 + seed)
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        A = O.dequant_vector(codes[3], s8[3], z8[3], 16)
        for j in range(3):
            y = Hs @ (x[j] - A)
            for gi in range(d // 16):
                seg = y[gi * 16:(gi + 1) * 16]
                sc, zc, cc = O.quant_group(seg, 2)
                sv, zv = O.fp8_decode([sc, zc])
                t = (seg - zv) / sv
                near_tie = np.abs(t - np.floor(t) - 0.5) < 1e-9
                ok = (cc == codes[j, gi * 16:(gi + 1) * 16]) | near_tie
                assert sc == s8[j, gi] and zc == z8[j, gi]
                assert ok.all()
                n_checked += 1
    assert n_checked == 40 * 3 * (d // 16)


def test_alpha_is_least_squares_and_bf16_rounded():
    d = 128
    p = O.Params(d=d)
    s = _signs(d, 3)
    Hs = scipy.linalg.hadamard(d) / np.sqrt(d) * s[None, :]
    H = O.rotation_matrix(d, s)
    for seed in range(60):
        x = _group_inputs(d, 4, 300 + seed)
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        A = O.dequant_vector(codes[3], s8[3], z8[3], 16)
        for j in range(3):
            y = Hs @ (x[j] - A)
            yh = _y_hat(p, codes, s8, z8, j)
            a_star = np.linalg.lstsq(yh[:, None], y, rcond=None)[0][0]
            a_bf = O.bf16_decode([alpha[j]])[0]
            assert alpha[j] == O.bf16_encode([a_star])[0]
            # brute force: nothing on a fine grid around it, and no bf16 neighbour, does better
            err = lambda a: np.sum((y - a * yh) ** 2)
            grid = np.linspace(a_star - 0.05, a_star + 0.05, 2001)
            assert err(a_star) <= min(err(a) for a in grid) + 1e-12
            for nb in (alpha[j] - 1, alpha[j] + 1):
                assert err(a_bf) <= err(O.bf16_decode([nb])[0]) + 1e-15
            # alpha = 0 and alpha = 1 are bf16 values, so the rounded optimum beats both
            assert err(a_bf) <= err(1.0) + 1e-15 and err(a_bf) <= err(0.0) + 1e-15


def test_single_channel_residual_recovers_through_transpose():
    """x_l = anchor + delta e_k: y = H r is a signed Hadamard column, its 2-bit
    code is (nearly) exact, and reconstruction must apply H^T to give back x_l."""
    d = 64
    p = O.Params(d=d)
    s = _signs(d, 4)
    H = O.rotation_matrix(d, s)
    rng = np.random.default_rng(5)
    for k in range(0, d, 7):
        # on-grid anchor: deq(anchor) == anchor exactly
        s_an = O.fp8_decode(O.fp8_encode([0.25]))[0]
        z_an = O.fp8_decode(O.fp8_encode([-2.0]))[0]
        c = rng.integers(0, 16, d)
        for gi in range(d // 16):
            c[gi * 16] = 0
            c[gi * 16 + 1] = 15
        anchor = s_an * c + z_an
        x = np.tile(anchor, (4, 1))
        delta = 0.5
        x[1, k] += delta
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        assert np.array_equal(O.dequant_vector(codes[3], s8[3], z8[3], 16), anchor)
        xh = O.reconstruct_group(p, codes, s8, z8, alpha, s, 1)
        r = np.zeros(d)
        r[k] = delta
        # y = +-delta/8 in every entry: two grid levels per group, so only the fp8
        # scale rounding (a few percent) and alpha remain as error
        assert np.abs(xh - x[1]).max() < 0.05 * delta
        wrong = anchor + O.bf16_decode([alpha[1]])[0] * (H @ (H @ r))  # H instead of H^T
        assert np.abs(wrong - x[1]).max() > 0.5 * delta
        # the untouched loops reconstruct to the anchor exactly (zero residual)
        for j in (0, 2):
            assert np.array_equal(O.reconstruct_group(p, codes, s8, z8, alpha, s, j), anchor)


@pytest.mark.parametrize("d", [64, 96, 128])
def test_reconstruction_error_bound(d):
    """|x_l - xhat_l|_2 = |y - alpha yhat|_2 <= |y - yhat|_2 (H orthogonal, alpha
    is the bf16-rounded least-squares optimum and 1 is a bf16 value)."""
    p = O.Params(d=d)
    s = _signs(d, 6)
    H = O.rotation_matrix(d, s)
    for seed in range(30):
        x = _group_inputs(d, 4, 600 + seed)
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        A = O.dequant_vector(codes[3], s8[3], z8[3], 16)
        for j in range(3):
            xh = O.reconstruct_group(p, codes, s8, z8, alpha, s, j)
            y = H @ (x[j] - A)
            yh = _y_hat(p, codes, s8, z8, j)
            assert np.linalg.norm(x[j] - xh) <= np.linalg.norm(y - yh) + 1e-12
            assert np.linalg.norm(x[j] - xh) < np.linalg.norm(x[j] - A)


def test_two_read_identity():
    """Reconstructing loop l reads only the anchor and loop l's own planes."""
    d = 128
    p = O.Params(d=d)
    S = _signs(d, 7)
    x = _group_inputs(d, 4, 700)
    codes, s8, z8, alpha = O.encode_group(p, x, S)
    rng = np.random.default_rng(8)
    for j in range(4):
        ref = O.reconstruct_group(p, codes, s8, z8, alpha, S, j)
        c2, s2, z2, a2 = codes.copy(), s8.copy(), z8.copy(), alpha.copy()
        for o in range(4):
            if o in (j, 3):
                continue
            c2[o] = rng.integers(0, 4, d)
            s2[o] = rng.integers(0, 0x70, d // 16)
            z2[o] = rng.integers(0, 0xFF, d // 16)
            a2[o] = rng.integers(0, 0x7F00)
        assert np.array_equal(O.reconstruct_group(p, c2, s2, z2, a2, S, j), ref)


def test_direct_mode_quantizes_each_loop_alone():
    d = 64
    p = O.Params(d=d, mode=O.MODE_DIRECT)
    x = _group_inputs(d, 4, 900)
    codes, s8, z8, alpha = O.encode_group(p, x, None)
    for j in range(4):
        bits = 4 if j == 3 else 2
        for gi in range(d // 16):
            sc, zc, cc = O.quant_group(x[j, gi * 16:(gi + 1) * 16], bits)
            assert sc == s8[j, gi] and zc == z8[j, gi]
            assert np.array_equal(cc, codes[j, gi * 16:(gi + 1) * 16])
        xh = O.reconstruct_group(p, codes, s8, z8, alpha, None, j)
        assert np.array_equal(xh, O.dequant_vector(codes[j], s8[j], z8[j], 16))
    assert np.all(alpha == 0)


def test_alpha_variants():
    d = 64
    s = _signs(d, 9)
    H = O.rotation_matrix(d, s)
    x = _group_inputs(d, 4, 950)
    for mode in (O.ALPHA_NORM_RATIO, O.ALPHA_ONE):
        p = O.Params(d=d, alpha_mode=mode)
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        A = O.dequant_vector(codes[3], s8[3], z8[3], 16)
        for j in range(3):
            y = H @ (x[j] - A)
            yh = _y_hat(p, codes, s8, z8, j)
            want = 1.0 if mode == O.ALPHA_ONE else np.linalg.norm(y) / np.linalg.norm(yh)
            assert alpha[j] == O.bf16_encode([want])[0]


def test_rotation_off_quantizes_plain_difference():
    d = 64
    p = O.Params(d=d, rotate=0)
    x = _group_inputs(d, 4, 960)
    codes, s8, z8, alpha = O.encode_group(p, x, np.full(d, -1, np.int8))  # signs ignored
    A = O.dequant_vector(codes[3], s8[3], z8[3], 16)
    for j in range(3):
        r = x[j] - A
        for gi in range(d // 16):
            sc, zc, cc = O.quant_group(r[gi * 16:(gi + 1) * 16], 2)
            assert np.array_equal(cc, codes[j, gi * 16:(gi + 1) * 16])


def test_encode_slice_matches_groups():
    d, L, N = 64, 8, 5
    p = O.Params(d=d)
    S = _signs(d, 10)
    rng = np.random.default_rng(11)
    xs = O.bf16_encode(rng.standard_normal((L, N, d)))
    e = O.encode_slice(p, xs, S)
    for k in range(2):
        for t in range(N):
            xg = O.bf16_decode(xs[4 * k:4 * k + 4, t])
            c, s8, z8, a = O.encode_group(p, xg, S)
            assert np.array_equal(e.codes[4 * k:4 * k + 4, t], c)
            assert np.array_equal(e.s8[4 * k:4 * k + 4, t], s8)
            assert np.array_equal(e.z8[4 * k:4 * k + 4, t], z8)
            assert np.array_equal(e.alpha[4 * k:4 * k + 4, t], a)
            for j in range(4):
                assert np.array_equal(
                    O.reconstruct_slice(p, e, S, 4 * k + j, t, t + 1)[0],
                    O.reconstruct_group(p, c, s8, z8, a, S, j))
