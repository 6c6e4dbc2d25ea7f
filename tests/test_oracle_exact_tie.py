"""Regression pin: a rotated residual that is exactly zero sits on a rounding
tie of the 2-bit quantizer; the oracle must decide it on the exact value.
The fixture (tests/golden/exact_tie_group.txt) holds generator-drawn inputs
only; the expected code is derived here in exact rational arithmetic."""
import os
from fractions import Fraction

import numpy as np
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "exact_tie_group.txt")


def _load():
    signs, x = None, []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        if key == "signs":
            signs = np.array([int(v) for v in vals], np.int8)
        else:
            x.append([int(v, 16) for v in vals])
    return signs, np.array(x, np.uint16)


def test_exact_zero_residual_rounds_half_to_even():
    signs, xb = _load()
    d = 128
    x = O.bf16_decode(xb)
    p = O.Params(d=d)
    codes, s8, z8, alpha = O.encode_group(p, x, signs)

    # exact residual of loop 2 against the dequantized anchor, as fractions
    s_a = [Fraction(v) for v in O.fp8_decode(s8[3])]
    z_a = [Fraction(v) for v in O.fp8_decode(z8[3])]
    anchor = [s_a[i // 16] * int(codes[3, i]) + z_a[i // 16] for i in range(d)]
    r = [Fraction(float(x[2, i])) - anchor[i] for i in range(d)]
    S = scipy.linalg.hadamard(d)
    exact_sum = sum(int(S[80, j]) * int(signs[j]) * r[j] for j in range(d))
    assert exact_sum == 0                      # y[80] is exactly zero

    g = 80 // 16
    s, z = (Fraction(v) for v in O.fp8_decode([s8[2, g], z8[2, g]]))
    t = (0 - z) / s
    assert t == Fraction(3, 2)                 # an exact tie between codes 1 and 2
    assert codes[2, 80] == 2                   # ties go to the even code
