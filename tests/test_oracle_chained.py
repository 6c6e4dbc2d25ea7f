"""Pins of the oracle's chained ("previous-loop") mode, the ablation contrast to
the shared anchor (ai4snews summary, paragraph 3: chained reconstruction grows
with the distance from the anchor).  Loop l < a takes its residual against the
reconstruction of loop l + 1, the last-loop anchor ending the chain.

Checked against things other than the oracle's own arithmetic: the definition
recomputed with scipy's Hadamard matrix (y_l = H (x_l - xhat_{l+1})), the
recursion xhat_l = xhat_{l+1} + alpha_l H^T yhat_l, the read set (the anchor
and the residuals of loops l..a-1 only), the P = 2 case (no chain: identical to
the shared-anchor encoding), and fused == dense attention."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O


def _signs(d, seed):
    rng = np.random.default_rng(seed)
    return (1 - 2 * rng.integers(0, 2, d)).astype(np.int8)


def _group(d, P, seed):
    rng = np.random.default_rng(seed)
    lam = np.exp(0.5 * rng.standard_normal(d))
    anchor = rng.standard_normal(d) * lam
    x = np.empty((P, d))
    for j in range(P - 1):
        x[j] = anchor + (0.3 - 0.25 * j / max(P - 2, 1)) * rng.standard_normal(d)
    x[P - 1] = anchor
    return O.bf16_decode(O.bf16_encode(x))


def _deq(codes, s8, z8, j):
    return O.dequant_vector(codes[j], s8[j], z8[j], 16)


@pytest.mark.parametrize("d,P", [(64, 4), (128, 4), (96, 4), (128, 8)])
def test_chain_definition_with_scipy_hadamard(d, P):
    """Each non-anchor loop quantizes H (x_l - xhat_{l+1}) with xhat_{l+1} the
    reconstruction of the next loop (the anchor for l = a-1); H from scipy."""
    p = O.Params(d=d, P=P, mode=O.MODE_CHAINED)
    s = _signs(d, 7)
    blocks = [scipy.linalg.hadamard(n) / np.sqrt(n) for n in (64, 32)] if d == 96 else \
        [scipy.linalg.hadamard(d) / np.sqrt(d)]
    H = scipy.linalg.block_diag(*blocks) * s[None, :]
    checked = 0
    for seed in range(12):
        x = _group(d, P, 1000 + seed)
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        a = P - 1
        for l in range(a - 1, -1, -1):
            ref = O.reconstruct_group(p, codes, s8, z8, alpha, s, l + 1)
            y = H @ (x[l] - ref)
            for gi in range(d // 16):
                seg = y[gi * 16:(gi + 1) * 16]
                sc, zc, cc = O.quant_group(seg, 2)
                sv, zv = O.fp8_decode([sc, zc])
                t = (seg - zv) / sv
                near = np.abs(t - np.floor(t) - 0.5) < 1e-9
                assert sc == s8[l, gi] and zc == z8[l, gi], (seed, l, gi)
                assert ((cc == codes[l, gi * 16:(gi + 1) * 16]) | near).all(), (seed, l, gi)
                checked += 1
    assert checked == 12 * (P - 1) * (d // 16)


@pytest.mark.parametrize("d", [64, 128])
def test_chain_reconstruction_recursion(d):
    p = O.Params(d=d, mode=O.MODE_CHAINED)
    s = _signs(d, 8)
    H = O.rotation_matrix(d, s)
    for seed in range(20):
        x = _group(d, 4, 2000 + seed)
        codes, s8, z8, alpha = O.encode_group(p, x, s)
        xh = [O.reconstruct_group(p, codes, s8, z8, alpha, s, j) for j in range(4)]
        assert np.array_equal(xh[3], _deq(codes, s8, z8, 3))
        for l in range(3):
            al = O.bf16_decode([alpha[l]])[0]
            expect = xh[l + 1] + al * (H.T @ _deq(codes, s8, z8, l))
            assert np.abs(xh[l] - expect).max() < 1e-12 * max(1.0, np.abs(expect).max())


def test_chain_reads_anchor_and_residuals_up_to_the_anchor():
    """Loop j reads the anchor and the residuals of loops j..a-1: perturbing any
    of those changes it; perturbing the residuals of loops below j does not."""
    d = 128
    p = O.Params(d=d, mode=O.MODE_CHAINED)
    s = _signs(d, 9)
    x = _group(d, 4, 3000)
    codes, s8, z8, alpha = O.encode_group(p, x, s)
    base = [O.reconstruct_group(p, codes, s8, z8, alpha, s, j) for j in range(4)]
    for k in range(4):                       # perturb loop k's planes
        c2, a2 = codes.copy(), alpha.copy()
        c2[k] = (c2[k] + 1) % (4 if k < 3 else 16)
        if k < 3:
            a2[k] = O.bf16_encode([O.bf16_decode([alpha[k]])[0] * 1.5])[0]
        for j in range(4):
            got = O.reconstruct_group(p, c2, s8, z8, a2, s, j)
            reads = (k == 3) or (j <= k < 3)
            if reads:
                assert not np.array_equal(got, base[j]), (k, j)
            else:
                assert np.array_equal(got, base[j]), (k, j)


@pytest.mark.parametrize("d", [64, 96, 128])
def test_two_loop_groups_chain_equals_shared_anchor(d):
    """With P = 2 there is no chain: the encoding is bit-identical to the
    shared-anchor one and the reconstructions agree to rounding."""
    s = _signs(d, 10)
    pc = O.Params(d=d, P=2, mode=O.MODE_CHAINED)
    pr = O.Params(d=d, P=2, mode=O.MODE_RESIDUAL)
    for seed in range(10):
        x = _group(d, 2, 4000 + seed)
        ec = O.encode_group(pc, x, s)
        er = O.encode_group(pr, x, s)
        for a, b in zip(ec, er):
            assert np.array_equal(a, b)
        xc = O.reconstruct_group(pc, *ec, s, 0)
        xr = O.reconstruct_group(pr, *er, s, 0)
        assert np.abs(xc - xr).max() < 1e-12 * max(1.0, np.abs(xr).max())


@pytest.mark.parametrize("d", [64, 128])
def test_chained_fused_attention_equals_dense(d):
    p = O.Params(d=d, mode=O.MODE_CHAINED)
    rng = np.random.default_rng(11)
    L, N = 8, 50
    lam = np.exp(0.5 * rng.standard_normal(d))
    xs = []
    for kv in range(2):
        anchor = rng.standard_normal((L // 4, N, d)) * lam
        x = np.empty((L, N, d))
        for k in range(L // 4):
            for j in range(3):
                x[4 * k + j] = anchor[k] + 0.2 * rng.standard_normal((N, d))
            x[4 * k + 3] = anchor[k]
        xs.append(O.bf16_encode(x))
    sk, sv = _signs(d, 12), _signs(d, 13)
    ek, ev = O.encode_slice(p, xs[0], sk), O.encode_slice(p, xs[1], sv)
    for loop in range(L):
        q = O.bf16_encode(rng.standard_normal(d))
        for n in (1, 17, N):
            dense = O.attention_slice(p, ek, ev, sk, sv, q, loop, n, 1 / np.sqrt(d), fused=False)
            fused = O.attention_slice(p, ek, ev, sk, sv, q, loop, n, 1 / np.sqrt(d), fused=True)
            assert np.abs(dense - fused).max() < 1e-12 * max(1.0, np.abs(dense).max())
