"""Pins for the oracle's decoders (O1 e4m3, O2 e8m0, bf16 widening).

Each decoder is pinned to something other than itself: the printed format
facts in tests/golden/, PyTorch's own float8 / bfloat16 dtypes, and
structural invariants (monotonicity, sign symmetry, counts)."""
import math
from fractions import Fraction

import numpy as np
import torch

import oracle
from golden_io import exact_value, read_pairs


def test_e4m3_golden_values():
    for code, text in read_pairs("e4m3_ocp_values.txt"):
        want = exact_value(text)
        got = oracle.e4m3(code)
        if want is None:
            assert got is None, hex(code)
        elif want == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, hex(code)
        else:
            assert got is not None and Fraction(got) == want, (hex(code), got, want)
            if want == 0:
                assert math.copysign(1.0, got) > 0


def test_e4m3_matches_torch_float8_e4m3fn_all_codes():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = t.to(torch.float64).tolist()
    for code in range(256):
        got = oracle.e4m3(code)
        if math.isnan(ref[code]):
            assert got is None, hex(code)
        else:
            assert got == ref[code] and math.copysign(1, got) == math.copysign(1, ref[code]), hex(code)


def test_e4m3_structure():
    pos = [oracle.e4m3(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "positive codes must increase strictly"
    for b in range(0x7F):
        assert oracle.e4m3(b | 0x80) == -oracle.e4m3(b)
    finite = [b for b in range(256) if oracle.e4m3(b) is not None]
    assert len(finite) == 254
    sub = [b for b in finite if 0 < abs(oracle.e4m3(b)) < 2.0 ** -6]
    assert len(sub) == 14  # 7 positive, 7 negative subnormals


def test_e8m0_golden_values():
    for code, text in read_pairs("e8m0_ocp_values.txt"):
        got = oracle.e8m0(code)
        if text == "refused":
            assert got is None
        else:
            assert got == math.ldexp(1.0, int(text)), hex(code)


def test_e8m0_matches_torch_float8_e8m0fnu():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
    ref = t.to(torch.float64).tolist()
    for code in range(255):
        assert oracle.e8m0(code) == ref[code], hex(code)
    assert math.isnan(ref[255]) and oracle.e8m0(255) is None


def test_bf16_golden_patterns():
    for bits, text in read_pairs("bf16_patterns.txt"):
        got = oracle.bf16(bits)
        want = exact_value(text)
        if want == "inf":
            assert got == math.inf
        elif want == "-0":
            assert got == 0.0 and math.copysign(1, got) < 0
        else:
            assert Fraction(got) == want, hex(bits)


def test_bf16_matches_torch_all_patterns():
    pats = np.arange(65536, dtype=np.uint32)
    ref = torch.from_numpy(pats.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decoders_reject_nan_and_ff():
    assert oracle.e4m3(0x7F) is None and oracle.e4m3(0xFF) is None
    assert oracle.e8m0(0xFF) is None
