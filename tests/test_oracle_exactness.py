"""Pins for the oracle's bf16 exactness test (O3), load check (O4) and
dequant slab (O5).

The exhaustive pin enumerates every finite bf16 value through PyTorch's
bfloat16 dtype (exact Fractions) and checks, for all 254 finite e4m3 codes x
all 255 legal e8m0 codes, that the oracle calls an element exact iff its exact
rational value is in that set."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8_fp8blk_amd import inputs


@pytest.fixture(scope="module")
def bf16_values():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.int16)
    vals = torch.from_numpy(pats).view(torch.bfloat16).to(torch.float64).numpy()
    return {Fraction(float(v)) for v in vals if np.isfinite(v)}


def _e4m3_exact_from_torch():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return {c: Fraction(v) for c, v in enumerate(t.to(torch.float64).tolist()) if not math.isnan(v)}


def test_exhaustive_code_by_scale_exactness(bf16_values):
    e4 = _e4m3_exact_from_torch()
    assert len(e4) == 254
    n_exact = {}
    for s in range(255):
        scale = Fraction(2) ** (s - 127)
        cnt = 0
        for code, val in e4.items():
            v = val * scale
            want = v in bf16_values
            got = oracle.is_bf16_exact(float(v))  # float(v) is exact: <= 4 significant bits
            assert float(v) == v
            assert got == want, (hex(code), s)
            cnt += want
        n_exact[s] = cnt
    # Closed form: every finite code is exact for scale codes 3..246 ...
    assert all(n_exact[s] == 254 for s in range(3, 247))
    # ... and not for the extremes (underflow below 2^-133, overflow past bf16 max).
    assert all(n_exact[s] < 254 for s in list(range(0, 3)) + list(range(247, 255)))


def test_is_bf16_exact_edges():
    mx = math.ldexp(255.0, 120)
    assert oracle.is_bf16_exact(mx) and oracle.is_bf16_exact(-mx)
    assert not oracle.is_bf16_exact(mx + math.ldexp(1.0, 119))
    assert not oracle.is_bf16_exact(math.ldexp(1.0, 128))
    assert oracle.is_bf16_exact(math.ldexp(1.0, -133))
    assert not oracle.is_bf16_exact(math.ldexp(1.0, -134))
    assert not oracle.is_bf16_exact(3 * math.ldexp(1.0, -134))
    assert oracle.is_bf16_exact(127 * math.ldexp(1.0, -133))  # largest subnormal
    assert oracle.is_bf16_exact(1 + 1 / 128) and not oracle.is_bf16_exact(1 + 1 / 256)
    assert oracle.is_bf16_exact(0.0) and oracle.is_bf16_exact(-0.0)
    assert not oracle.is_bf16_exact(math.inf) and not oracle.is_bf16_exact(math.nan)


def _lin(rows, cols, seed=11):
    return inputs.host_linear(rows, cols, 1, seed, codes="uniform", scale_lo=120, scale_hi=134)


def test_load_check_ok_and_grid():
    L = _lin(200, 272)  # ragged: 2 x 3 grid with partial last blocks
    assert L.scales.shape == (2, 3)
    st, fb, grid = oracle.load_check(L.codes, L.scales)
    assert st == oracle.OK and fb == -1
    ref = torch.from_numpy(L.scales).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    assert np.array_equal(grid.view(np.uint32), ref.view(np.uint32))


def test_load_check_grid_subnormal_scale():
    codes = np.full((128, 128), 0x38, dtype=np.uint8)  # 1.0 everywhere
    scales = np.zeros((1, 1), dtype=np.uint8)  # 2^-127: an f32 subnormal, exact bf16
    st, fb, grid = oracle.load_check(codes, scales)
    assert st == oracle.OK
    assert grid[0, 0] == np.float32(math.ldexp(1.0, -127)) and grid.view(np.uint32)[0, 0] == 0x00400000


def test_load_check_refusals_and_precedence():
    L = _lin(256, 384)
    codes, scales = L.codes.copy(), L.scales.copy()
    # inexact: overflow (code 0x7E = 448 with scale 2^127) at element (130, 5)
    c1 = codes.copy(); s1 = scales.copy()
    s1[1, 0] = 254; c1[128:256, 0:128] = 0x38; c1[130, 5] = 0x7E
    st, fb, _ = oracle.load_check(c1, s1)
    assert (st, fb) == (oracle.INEXACT, 130 * 384 + 5)
    # inexact: underflow (code 0x01 = 2^-9 with scale 2^-126)
    c2 = codes.copy(); s2 = scales.copy()
    s2[0, 2] = 1; c2[0:128, 256:384] = 0x38; c2[7, 300] = 0x01; c2[9, 260] = 0x81
    st, fb, _ = oracle.load_check(c2, s2)
    assert (st, fb) == (oracle.INEXACT, 7 * 384 + 300)
    # NaN codes: the lowest index wins, and a NaN beats an earlier inexact element
    c3 = c2.copy(); c3[20, 1] = 0xFF; c3[5, 383] = 0x7F
    st, fb, _ = oracle.load_check(c3, s2)
    assert (st, fb) == (oracle.NAN_CODE, 5 * 384 + 383)
    # 0xFF scale beats everything; lowest grid index
    s4 = s2.copy(); s4[1, 2] = 0xFF; s4[1, 1] = 0xFF
    st, fb, _ = oracle.load_check(c3, s4)
    assert (st, fb) == (oracle.SCALE_FF, 1 * 3 + 1)


def test_dequant_matches_torch_path():
    L = _lin(256, 512)
    got = oracle.dequant_bf16(L.codes, L.scales)
    e = torch.from_numpy(L.codes).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(L.scales).view(torch.float8_e8m0fnu).to(torch.float64)
    s_full = s.repeat_interleave(128, 0)[:256].repeat_interleave(128, 1)[:, :512]
    ref = (e * s_full).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_dequant_refuses_inexact():
    codes = np.full((128, 128), 0x01, dtype=np.uint8)
    scales = np.full((1, 1), 1, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.dequant_bf16(codes, scales)


def test_dequant_subnormal_and_signed_zero():
    codes = np.zeros((128, 128), dtype=np.uint8)
    codes[0, :8] = [0x00, 0x80, 0x01, 0x81, 0x07, 0x08, 0x7E, 0xFE]
    scales = np.full((1, 1), 3, dtype=np.uint8)  # 2^-124: 0x01 -> 2^-133, the bf16 min subnormal
    out = oracle.dequant_bf16(codes, scales)
    assert list(out[0, :4]) == [0x0000, 0x8000, 0x0001, 0x8001]
