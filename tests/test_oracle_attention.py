"""Pins of the oracle's attention: the dense form against scipy's softmax, the
fused (no-reconstruction) form against the dense form, and the zero-residual
special case that reduces to textbook attention on the raw states."""
import numpy as np
import pytest
import scipy.special

import oracle as O


def _signs(d, seed):
    rng = np.random.default_rng(seed)
    return (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)


def _textbook(q, K, V, scale):
    w = scipy.special.softmax(scale * (K @ q))
    return w @ V


@pytest.mark.parametrize("n,d", [(1, 16), (7, 64), (300, 128)])
def test_dense_matches_scipy_softmax(n, d):
    rng = np.random.default_rng(n + d)
    q, K, V = rng.standard_normal(d), rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d))
    out = O.attention_dense(q, K, V, 1 / np.sqrt(d))
    assert np.allclose(out, _textbook(q, K, V, 1 / np.sqrt(d)), rtol=1e-12, atol=1e-13)


def test_dense_empty_is_zero():
    out = O.attention_dense(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert np.all(out == 0)


def _slice_inputs(d, L, N, seed, sig=(0.3, 0.2, 0.1)):
    rng = np.random.default_rng(seed)
    lam = np.exp(0.5 * rng.standard_normal(d))
    x = np.empty((L, N, d))
    for k in range(L // 4):
        anchor = rng.standard_normal((N, d)) * lam
        for j in range(3):
            x[4 * k + j] = anchor + sig[j] * rng.standard_normal((N, d))
        x[4 * k + 3] = anchor
    return O.bf16_encode(x)


@pytest.mark.parametrize("mode,d,L", [(O.MODE_RESIDUAL, 64, 4), (O.MODE_RESIDUAL, 96, 8),
                                      (O.MODE_RESIDUAL, 128, 4), (O.MODE_DIRECT, 128, 4)])
def test_fused_equals_dense(mode, d, L):
    N = 150
    p = O.Params(d=d, mode=mode)
    SK = _signs(d, 1)
    SV = _signs(d, 2)
    xk = _slice_inputs(d, L, N, 10 + d)
    xv = _slice_inputs(d, L, N, 20 + d)
    ek, ev = O.encode_slice(p, xk, SK), O.encode_slice(p, xv, SV)
    rng = np.random.default_rng(3)
    for loop in range(L):
        q = O.bf16_encode(rng.standard_normal(d))
        for n in (N, 37, 1):
            a = O.attention_slice(p, ek, ev, SK, SV, q, loop, n, 1 / np.sqrt(d), fused=False)
            b = O.attention_slice(p, ek, ev, SK, SV, q, loop, n, 1 / np.sqrt(d), fused=True)
            assert np.allclose(a, b, rtol=1e-11, atol=1e-12), (loop, n)


def test_dense_slice_is_softmax_over_reconstruction():
    d, L, N = 64, 4, 256
    p = O.Params(d=d)
    SK = _signs(d, 5)
    SV = _signs(d, 6)
    ek = O.encode_slice(p, _slice_inputs(d, L, N, 50), SK)
    ev = O.encode_slice(p, _slice_inputs(d, L, N, 51), SV)
    q = O.bf16_encode(np.random.default_rng(4).standard_normal(d))
    for loop in range(L):
        K = O.reconstruct_slice(p, ek, SK, loop)
        V = O.reconstruct_slice(p, ev, SV, loop)
        ref = _textbook(O.bf16_decode(q), K, V, 0.125)
        out = O.attention_slice(p, ek, ev, SK, SV, q, loop, N, 0.125)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_zero_residual_reduces_to_textbook_attention_on_raw_states():
    """Every loop equal to an on-grid anchor: the anchor codes reproduce it
    exactly, the residuals are zero, so attention over the cache equals
    attention over the raw BF16 states."""
    d, N = 64, 64
    p = O.Params(d=d)
    rng = np.random.default_rng(12)
    s = O.fp8_decode(O.fp8_encode([0.125]))[0]
    z = O.fp8_decode(O.fp8_encode([-1.0]))[0]
    raw = []
    for _ in range(2):
        c = rng.integers(0, 16, (N, d))
        c[:, ::16] = 0
        c[:, 1::16] = 15
        a = s * c + z
        raw.append(a)
    xk = O.bf16_encode(np.broadcast_to(raw[0], (4, N, d)).copy())
    xv = O.bf16_encode(np.broadcast_to(raw[1], (4, N, d)).copy())
    SK = _signs(d, 13)
    SV = _signs(d, 14)
    ek, ev = O.encode_slice(p, xk, SK), O.encode_slice(p, xv, SV)
    assert np.all(ek.alpha == 0) and np.all(ek.s8[:3] == 0)
    q = O.bf16_encode(rng.standard_normal(d))
    ref = _textbook(O.bf16_decode(q), raw[0], raw[1], 0.125)
    for loop in range(4):
        for fused in (False, True):
            out = O.attention_slice(p, ek, ev, SK, SV, q, loop, N, 0.125, fused=fused)
            assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
