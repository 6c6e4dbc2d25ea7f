"""Pins of the oracle's storage accounting against the pages' printed figure."""
import os

import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accounting.txt")


def _rows():
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, r, g, d, P, al, pct = line.split()
                yield int(a), int(r), int(g), int(d), int(P), int(al), float(pct)


@pytest.mark.parametrize("row", list(_rows()))
def test_printed_storage_reduction(row):
    a, r, g, d, P, al, pct = row
    bits = O.bits_per_element(a, r, g, d, P, bool(al))
    assert round(100 * (1 - bits / 16), 1) == pct


def test_closed_form_values():
    # INT4 anchor + 3 INT2 residuals, FP8 scale+offset per 16, BF16 alpha per 128-vector
    assert O.bits_per_element(4, 2, 16, 128, 4, True) == (5 + 3 * (3 + 0.125)) / 4 == 3.59375
    # direct mode drops alpha
    assert O.bits_per_element(4, 2, 16, 128, 4, False) == (5 + 3 * 3) / 4
    # uniform precisions
    assert O.bits_per_element(4, 4, 16, 128, 4, False) == 5.0
    assert O.bits_per_element(2, 2, 16, 64, 1, False) == 3.0
