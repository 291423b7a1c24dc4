"""Readers for the text fixtures under tests/golden/."""
import os
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_pairs(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out.append((int(k, 16), v))
    return out


def exact_value(text):
    """Fraction for a decimal string; None for nan; the strings inf/-inf kept."""
    if text == "nan":
        return None
    if text in ("inf", "-inf"):
        return text
    if text == "-0":
        return "-0"
    return Fraction(text)
