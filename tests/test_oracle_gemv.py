"""Pins for the oracle's GEMVs: O6 (double) and O7 (documented f32 order).

O6 is pinned by brute force with exact rationals on tiny shapes and by a
float64 matmul of PyTorch-decoded weights. O7 is pinned by cases where every
summation order gives the exact result (integer-valued inputs, one-hot x), by
the error bound against O6, and by its twin identity: slab-widened weights (A)
and in-register decoded weights (B) give the same bits, while each perturbed
order gives different bits (so the identity check has teeth)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8_fp8blk_amd import inputs


def _torch_weights(codes, scales):
    rows, cols = codes.shape
    e = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
    s_full = s.repeat_interleave(128, 0)[:rows].repeat_interleave(128, 1)[:, :cols]
    return (e * s_full).numpy()


def _torch_x(x):
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("cols", [16, 128, 144])
@pytest.mark.parametrize("rows,M", [(1, 1), (3, 2), (2, 3)])
def test_gemv_f64_brute_force_rationals(rows, cols, M):
    L = inputs.host_linear(rows, cols, M, 1000 + rows * 7 + cols + M, codes="uniform",
                           scale_lo=120, scale_hi=134)
    y, ya = oracle.gemv_f64(L.codes, L.scales, L.x)
    W = _torch_weights(L.codes, L.scales)
    X = _torch_x(L.x)
    for m in range(M):
        for r in range(rows):
            exact = sum(Fraction(float(W[r, c])) * Fraction(float(X[m, c])) for c in range(cols))
            eabs = sum(abs(Fraction(float(W[r, c])) * Fraction(float(X[m, c]))) for c in range(cols))
            bound = Fraction(cols) * Fraction(1, 2 ** 53) * eabs
            assert abs(Fraction(y[m, r]) - exact) <= bound
            assert abs(Fraction(ya[m, r]) - eabs) <= bound


def test_gemv_f64_matches_float64_matmul():
    L = inputs.host_linear(300, 1040, 3, 77)
    y, ya = oracle.gemv_f64(L.codes, L.scales, L.x)
    W, X = _torch_weights(L.codes, L.scales), _torch_x(L.x)
    ref = X @ W.T
    assert np.all(np.abs(y - ref) <= 1e-12 * ya + 1e-300)
    assert np.allclose(ya, np.abs(X)[:, None, :].__mul__(np.abs(W)[None]).sum(-1), rtol=1e-12)


def _integer_case(rows, cols, M, seed):
    """Codes whose values are integers in [-16, 16], scales 2^k with |k| <= 3,
    x integers in [-8, 8]: every partial sum is a multiple of 2^-3 well below
    2^21, so every f32 summation order is exact."""
    rng = np.random.default_rng(seed)
    e4 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    ok = [c for c in range(256) if not math.isnan(e4[c]) and float(e4[c]).is_integer() and abs(e4[c]) <= 16]
    codes = np.array(ok, dtype=np.uint8)[rng.integers(0, len(ok), size=(rows, cols))]
    gr, gc = inputs.grid_shape(rows, cols)
    scales = (127 + rng.integers(-3, 4, size=(gr, gc))).astype(np.uint8)
    xi = rng.integers(-8, 9, size=(M, cols)).astype(np.float32)
    x = inputs.round_to_bf16_bits(xi)
    W = _torch_weights(codes, scales)
    exact = xi.astype(np.float64) @ W.T  # exact in double here too
    return codes, scales, x, exact


@pytest.mark.parametrize("rows,cols,M", [(5, 16, 1), (130, 1040, 2), (64, 4096, 3), (3, 3088, 1)])
def test_gemv_f32_order_integer_exact(rows, cols, M):
    codes, scales, x, exact = _integer_case(rows, cols, M, rows + cols)
    yb = oracle.gemv_f32_order(x, codes=codes, scales=scales)
    ya = oracle.gemv_f32_order(x, w_bf16=oracle.dequant_bf16(codes, scales))
    assert np.array_equal(yb.astype(np.float64), exact)
    assert np.array_equal(ya.astype(np.float64), exact)
    y64, _ = oracle.gemv_f64(codes, scales, x)
    assert np.array_equal(y64, exact)


def test_one_hot_x_selects_a_column():
    L = inputs.host_linear(256, 2048, 1, 5)
    W = _torch_weights(L.codes, L.scales)
    for c in (0, 17, 1023, 1024, 2047):
        xf = np.zeros((1, 2048), dtype=np.float32)
        xf[0, c] = 1.0
        x = inputs.round_to_bf16_bits(xf)
        y = oracle.gemv_f32_order(x, codes=L.codes, scales=L.scales)
        y64, _ = oracle.gemv_f64(L.codes, L.scales, x)
        assert np.array_equal(y[0].astype(np.float64), W[:, c])
        assert np.array_equal(y64[0], W[:, c])


@pytest.mark.parametrize("rows,cols,M", [(256, 512, 1), (96, 3088, 3), (64, 16384, 2), (7, 1040, 4)])
def test_twin_identity_and_bound(rows, cols, M):
    L = inputs.host_linear(rows, cols, M, 31 + cols)
    slab = oracle.dequant_bf16(L.codes, L.scales)
    ya = oracle.gemv_f32_order(L.x, w_bf16=slab)
    yb = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales)
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x)
    T = -(-cols // 1024)
    d = 16 + 6 + (T - 1)  # longest chain of roundings from a product to the result
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    err = np.abs(yb.astype(np.float64) - y64)
    assert np.all(err <= gamma * yabs)
    assert np.all(err <= 1e-5 * yabs)


def test_products_are_exact_fma_equals_mul_add():
    L = inputs.host_linear(128, 4096, 2, 8)
    y0 = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales, variant=0)
    y4 = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales, variant=4)
    assert np.array_equal(y0.view(np.uint32), y4.view(np.uint32))


@pytest.mark.parametrize("variant", [1, 2, 3])
def test_teeth_perturbed_order_breaks_identity(variant):
    L = inputs.host_linear(256, 4096, 1, 9)
    slab = oracle.dequant_bf16(L.codes, L.scales)
    ya = oracle.gemv_f32_order(L.x, w_bf16=slab)
    yv = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales, variant=variant)
    assert not np.array_equal(ya.view(np.uint32), yv.view(np.uint32))
    # ... while staying a correct GEMV within the tolerance
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x)
    assert np.all(np.abs(yv.astype(np.float64) - y64) <= 1e-5 * yabs)


def test_teeth_transposed_scale_grid_is_caught():
    """A plausible indexing mistake (reading the grid as [c/128][r/128]) planted on
    the oracle side must fail the tolerance check against O6."""
    L = inputs.host_linear(512, 512, 1, 12)
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x)
    bad = oracle.gemv_f32_order(L.x, codes=L.codes, scales=np.ascontiguousarray(L.scales.T))
    assert np.any(np.abs(bad.astype(np.float64) - y64) > 1e-5 * yabs)


def test_teeth_dropped_term_is_caught():
    """A dropped term (one column's product left out) planted on the oracle side
    must change the integer-exact result."""
    codes, scales, x, exact = _integer_case(4, 1040, 1, 3)
    W = _torch_weights(codes, scales)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    c = next(c for c in range(1039, -1, -1) if xf[0, c] != 0 and np.any(W[:, c] != 0))
    x2 = x.copy()
    x2[0, c] = 0
    y = oracle.gemv_f32_order(x2, codes=codes, scales=scales)
    assert not np.array_equal(y.astype(np.float64), exact)


def test_batch_invariance_in_oracle():
    L = inputs.host_linear(64, 2048, 5, 21)
    yp = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales)
    for m in range(5):
        y1 = oracle.gemv_f32_order(L.x[m:m + 1], codes=L.codes, scales=L.scales)
        assert np.array_equal(yp[m].view(np.uint32), y1[0].view(np.uint32))


def test_sign_and_scale_invariances():
    L = inputs.host_linear(128, 1024, 1, 13)
    y = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales)
    yneg = oracle.gemv_f32_order(L.x, codes=L.codes ^ np.uint8(0x80), scales=L.scales)
    assert np.array_equal(yneg, -y)
    yx = oracle.gemv_f32_order(L.x ^ np.uint16(0x8000), codes=L.codes, scales=L.scales)
    assert np.array_equal(yx, -y)
    y2 = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales + np.uint8(3))
    assert np.array_equal(y2, y * np.float32(8))
