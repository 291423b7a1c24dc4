"""Pins of the native expert arm's oracle (oracle/fp4_expert_oracle.c) to
facts outside it: PyTorch's own FP4 / FP8 / e8m0 conversions (library
routines written independently of the oracle), exhaustive code x scale
tables, a hand-worked act_quant block, and closed forms of the GEMV.

Source passages: "Module dsv4_gpu" page, enums ExpertArm and ExpertKind
(activation codes per 128 elements in FP8 times the NVFP4 / MXFP4 slabs as
stored; unexpected recipes refused) and the rungs paragraph (routed experts
dequantize exactly to bf16).
"""
import sys
import types

import numpy as np
import pytest

import oracle
from block_scaled_fp8_fp8blk_amd import inputs as I

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def torch_fp4():
    """PyTorch's reference FP4 helpers (torch.testing._internal.common_quantized).
    That module imports its test harness, which needs the optional
    `expecttest` package; a stand-in module is enough for the helpers."""
    if "expecttest" not in sys.modules:
        try:
            import expecttest  # noqa: F401
        except ImportError:
            stub = types.ModuleType("expecttest")
            stub.TestCase = object
            sys.modules["expecttest"] = stub
    from torch.testing._internal import common_quantized as cq
    return cq


def torch_decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    import torch
    cq = torch_fp4()
    t = torch.from_numpy(np.ascontiguousarray(nibbles, dtype=np.uint8))
    return cq._floatx_unpacked_to_f32(t, 2, 1).double().numpy()


def torch_decode_e4m3(codes: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


def torch_decode_e8m0(codes: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).double().numpy()


def torch_bf16_roundtrip(v: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def unpack(codes: np.ndarray) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] nibbles, even column = low nibble
    (the layout is pinned to torch's pack_uint4 below)."""
    out = np.empty((codes.shape[0], 2 * codes.shape[1]), dtype=np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def library_weights(fmt, codes, scales) -> np.ndarray:
    """Element values from torch's decoders, scale broadcast per block."""
    B = oracle.FP4_BLOCK[fmt]
    vals = torch_decode_e2m1(unpack(codes))
    sc = torch_decode_e8m0(scales) if fmt == oracle.MXFP4 else torch_decode_e4m3(scales)
    return vals * np.repeat(sc, B, axis=1)


# --- e2m1 and the packing -----------------------------------------------------

def test_e2m1_matches_torch_for_every_code():
    ref = torch_decode_e2m1(np.arange(16, dtype=np.uint8))
    got = np.array([oracle.e2m1(c) for c in range(16)])
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))  # code 8 is -0


def test_nibble_order_matches_torch_pack_uint4():
    import torch
    cq = torch_fp4()
    rng = np.random.default_rng(11)
    nib = rng.integers(0, 16, size=(3, 64), dtype=np.int64).astype(np.uint8)
    packed = cq.pack_uint4(torch.from_numpy(nib)).numpy()
    scales = np.full((3, 2), 127, dtype=np.uint8)  # MXFP4 scale 1.0
    ref = torch_decode_e2m1(nib)
    for r in range(3):
        for c in range(64):
            assert oracle.fp4_element(oracle.MXFP4, packed, scales, r, c) == ref[r, c]


# --- exactness tables and refusals -------------------------------------------

def test_mxfp4_code_times_scale_exhaustive():
    """Every e2m1 code x every e8m0 scale: accepted iff the product is a finite
    bf16 value (decided by torch's own bf16 rounding); 0xFF refused."""
    vals = torch_decode_e2m1(np.arange(16, dtype=np.uint8))
    for s in range(256):
        for code in range(16):
            codes = np.zeros((1, 16), dtype=np.uint8)
            codes[0, 0] = code
            scales = np.array([[s]], dtype=np.uint8)
            st, fb = oracle.fp4_load_check(oracle.MXFP4, codes, scales)
            if s == 0xFF:
                assert (st, fb) == (oracle.SCALE_FF, 0)
                continue
            v = vals[code] * 2.0 ** (s - 127)
            rt = torch_bf16_roundtrip(np.array([v]))[0]
            exact = np.isfinite(rt) and rt == v
            assert (st == oracle.OK) == exact, (code, s, st)
            if not exact:
                assert (st, fb) == (oracle.INEXACT, 0)
    # the refusals are confined to the two largest scales
    bad = [(s, c) for s in range(255) for c in range(16)
           if not np.isfinite(torch_bf16_roundtrip(np.array([vals[c] * 2.0 ** (s - 127)]))[0])]
    assert bad and min(s for s, _ in bad) == 253


def test_nvfp4_code_times_scale_exhaustive():
    """Every e2m1 code x every non-negative finite e4m3 scale is exactly a
    bf16 value; negative or NaN scale codes are refused."""
    vals = torch_decode_e2m1(np.arange(16, dtype=np.uint8))
    e4 = torch_decode_e4m3(np.arange(256, dtype=np.uint8))
    for s in range(256):
        scales = np.array([[s]], dtype=np.uint8)
        codes = np.array([[0x10 * (c % 16) + c % 16 for c in range(8)]], dtype=np.uint8)
        st, fb = oracle.fp4_load_check(oracle.NVFP4, codes, scales)
        if s & 0x80 or (s & 0x7F) == 0x7F:
            assert (st, fb) == (oracle.BAD_SCALE, 0), s
            continue
        assert st == oracle.OK, s
        prods = vals * e4[s]
        assert np.array_equal(torch_bf16_roundtrip(prods), prods)


def test_fp4_refusal_reports_lowest_index():
    codes = np.zeros((4, 32), dtype=np.uint8)
    sc = np.full((4, 2), 120, dtype=np.uint8)
    sc[2, 1] = 0xFF
    sc[3, 0] = 0xFF
    assert oracle.fp4_load_check(oracle.MXFP4, codes, sc) == (oracle.SCALE_FF, 5)
    sc = np.full((4, 2), 120, dtype=np.uint8)
    sc[1, 1] = 254  # 2^127: codes of magnitude >= 2 overflow bf16
    codes[1, 20] = 0x40  # columns 40 (code 0, ok) and 41 (code 4 = 2.0)
    codes[3, 30] = 0x07
    assert oracle.fp4_load_check(oracle.MXFP4, codes, sc) == (oracle.INEXACT, 1 * 64 + 41)
    nv = np.full((4, 4), 0x38, dtype=np.uint8)
    nv[2, 3] = 0x80  # -0
    assert oracle.fp4_load_check(oracle.NVFP4, codes, nv) == (oracle.BAD_SCALE, 11)


def test_fp4_dequant_matches_library_decoders():
    for fmt, (lo, hi) in ((oracle.MXFP4, (100, 160)), (oracle.NVFP4, (0x00, 0x7E))):
        L = I.host_fp4_linear(fmt, 24, 128, 1, 31 + fmt, scale_lo=lo, scale_hi=hi)
        slab = oracle.fp4_dequant_bf16(fmt, L.codes, L.scales)
        ref = library_weights(fmt, L.codes, L.scales)
        import torch
        ref_bits = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(slab, ref_bits)


# --- act_quant ----------------------------------------------------------------

def bf16_bits(values) -> np.ndarray:
    return I.round_to_bf16_bits(np.asarray(values, dtype=np.float32))


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def torch_e4m3_codes(v: np.ndarray) -> np.ndarray:
    """torch's nearest-even cast of float32 values to e4m3 bytes."""
    return I.round_to_e4m3(np.asarray(v, dtype=np.float32))


def check_act_quant_against_library(x_bits: np.ndarray):
    codes, scales = oracle.act_quant(x_bits)
    M, cols = x_bits.shape
    x = bf16_values(x_bits)
    for m in range(M):
        for b in range(scales.shape[1]):
            blk = x[m, 128 * b:128 * b + 128]
            e = int(scales[m, b]) - 127
            amax = np.max(np.abs(blk))
            # the scale is the smallest power of two in range that maps amax to <= 448
            assert -127 <= e <= 127
            assert amax <= 448.0 * 2.0 ** e
            assert e == -127 or amax > 448.0 * 2.0 ** (e - 1)
            # each code is torch's nearest-even e4m3 cast of x / 2^e (exact in
            # float32 here: the scaled values stay in float32's normal range or
            # are far below e4m3's smallest step)
            scaled = np.ldexp(blk, -e)
            assert np.array_equal(codes[m, 128 * b:128 * b + 128], torch_e4m3_codes(scaled))


def test_act_quant_hand_worked_block():
    """amax 500 needs 2^1 (448 < 500 <= 896): scale code 128. Then
    1.0 / 2 = 0.5 = 2^-1 -> exponent field 6, mantissa 0 -> 0x30;
    -3.0 / 2 = -1.5 -> field 7, mantissa 4 -> 0xBC;
    500 / 2 = 250 lies in [128, 256) where e4m3 steps by 16: 250/16 = 15.625
    rounds to 16 -> 256 = 2^8 -> field 15, mantissa 0 -> 0x78;
    1e-4 / 2 is below half the smallest step 2^-9 -> +0 -> 0x00;
    -1e-4 / 2 keeps its sign -> 0x80."""
    x = bf16_bits([1.0, -3.0, 500.0, 1e-4, -1e-4] + [0.0] * 123)
    codes, scales = oracle.act_quant(x)
    assert scales.tolist() == [[128]]
    assert codes[0, :5].tolist() == [0x30, 0xBC, 0x78, 0x00, 0x80]
    assert not codes[0, 5:].any()


def test_act_quant_every_bf16_value_is_rounded_like_torch():
    """Every finite bf16 pattern of magnitude <= 448, in blocks whose amax is
    448 (so 2^e = 1 and the codes are torch's cast of x itself)."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = bf16_values(pos.astype(np.uint16))
    pos = pos[vals <= 448.0]
    pats = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    per = 127
    nblk = -(-pats.size // per)
    x = np.zeros((nblk, 128), dtype=np.uint16)
    x[:, 0] = bf16_bits([448.0])[0]
    flat = np.zeros(nblk * per, dtype=np.uint16)
    flat[:pats.size] = pats
    x[:, 1:] = flat.reshape(nblk, per)
    codes, scales = oracle.act_quant(x)
    assert np.all(scales == 127)
    assert np.array_equal(codes, torch_e4m3_codes(bf16_values(x)))


@pytest.mark.parametrize("seed,mag", [(1, 1.0), (2, 1e-30), (3, 1e30), (4, 1e-38)])
def test_act_quant_random_blocks_against_library(seed, mag):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((3, 512)) * mag
    v[1, 128:256] = 0.0                         # an all-zero block
    v[2, 0:128] *= 10.0 ** rng.integers(-6, 6, 128)  # a block of widely spread magnitudes
    check_act_quant_against_library(bf16_bits(v))


def test_act_quant_extremes_and_ragged_tail():
    x = bf16_bits(np.concatenate([np.full(128, 3.0e38), np.full(72, -1.0e-40)]))[None, :]
    codes, scales = oracle.act_quant(x)
    assert scales.shape == (1, 2)
    # 3e38 / 448 lies in [2^119, 2^120]: scale 2^120; the second (ragged, 72
    # columns) block is bf16-subnormal: the smallest scale 2^-127
    assert scales.tolist() == [[127 + 120, 0]]
    check_act_quant_against_library(x)


# --- the native GEMV ----------------------------------------------------------

def library_act(xq: np.ndarray, xs: np.ndarray) -> np.ndarray:
    return torch_decode_e4m3(xq) * np.repeat(torch_decode_e8m0(xs), 128, axis=1)[:, :xq.shape[1]]


def spread_blocks(x_bits: np.ndarray) -> np.ndarray:
    """The activations with 128-column block b scaled by 16^(b mod 4) / 64,
    so that neighbouring blocks quantize with different scales."""
    v = bf16_values(x_bits)
    f = np.array([16.0 ** ((c // 128) % 4) / 64.0 for c in range(v.shape[1])])
    return bf16_bits(v * f)


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.NVFP4])
def test_fp4_gemv_matches_library_matmul(fmt):
    """Brute force on small shapes: torch's decoders and numpy's float64
    matmul give the same sum (every product is exact; the sums of a few
    hundred terms agree to float64 rounding)."""
    L = I.host_fp4_linear(fmt, 40, 512, 3, 50 + fmt)
    xq, xs = oracle.act_quant(spread_blocks(L.x))
    assert len(np.unique(xs)) >= 4  # the 128-column blocks carry different scales
    y, yabs = oracle.fp4_gemv_f64(fmt, L.codes, L.scales, xq, xs, L.global_scale)
    W = library_weights(fmt, L.codes, L.scales)
    A = library_act(xq, xs)
    ref = L.global_scale * (A @ W.T)
    refabs = abs(L.global_scale) * (np.abs(A) @ np.abs(W).T)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * refabs.max())
    assert np.allclose(yabs, refabs, rtol=1e-13)
    assert np.all(np.abs(y) <= yabs * (1 + 1e-12))


@pytest.mark.parametrize("fmt", [oracle.MXFP4, oracle.NVFP4])
def test_fp4_gemv_one_hot_closed_form(fmt):
    """A single nonzero weight (code 0x7 = 6.0 at (r, c)) and activation
    codes 0x38 (1.0) with scale 2^3: y[r] = g * 6 * scale(r, c) * 8, other
    rows 0."""
    rows, cols = 5, 256
    B = oracle.FP4_BLOCK[fmt]
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    r, c = 3, 77
    codes[r, c // 2] = 0x70 if c % 2 else 0x07
    scales = np.full((rows, cols // B), 127 if fmt == oracle.MXFP4 else 0x38, dtype=np.uint8)
    scales[r, c // B] = 125 if fmt == oracle.MXFP4 else 0x2C  # 2^-2 / e4m3 0.375
    s = 0.25 if fmt == oracle.MXFP4 else 0.375
    xq = np.full((1, cols), 0x38, dtype=np.uint8)
    xs = np.full((1, 2), 130, dtype=np.uint8)
    y, _ = oracle.fp4_gemv_f64(fmt, codes, scales, xq, xs, 0.75)
    expect = np.zeros((1, rows))
    expect[0, r] = 0.75 * 6.0 * s * 8.0
    assert np.array_equal(y, expect)


def test_fp4_gemv_global_scale_is_linear():
    L = I.host_fp4_linear(oracle.NVFP4, 16, 128, 2, 77)
    xq, xs = oracle.act_quant(L.x)
    y1, a1 = oracle.fp4_gemv_f64(oracle.NVFP4, L.codes, L.scales, xq, xs, 1.0)
    y8, a8 = oracle.fp4_gemv_f64(oracle.NVFP4, L.codes, L.scales, xq, xs, -8.0)
    assert np.array_equal(y8, -8.0 * y1) and np.array_equal(a8, 8.0 * a1)


def test_fp4_gemv_rows_are_independent_of_threads():
    L = I.host_fp4_linear(oracle.MXFP4, 33, 128, 2, 78)
    xq, xs = oracle.act_quant(L.x)
    y1, _ = oracle.fp4_gemv_f64(oracle.MXFP4, L.codes, L.scales, xq, xs, nthreads=1)
    y7, _ = oracle.fp4_gemv_f64(oracle.MXFP4, L.codes, L.scales, xq, xs, nthreads=7)
    assert np.array_equal(y1, y7)
