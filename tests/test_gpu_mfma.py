"""GPU parity of the matrix-core arm (fp8blk_gemv_mfma / bf16_gemv_twin_mfma).

The matrix core's internal summation order is not documented, so there is no
bitwise oracle for this arm. What is checked: the FP8 arm and its bf16 twin
give identical bits; row m of a panel equals the single-row call bit for bit;
inputs on which every summation order is exact give the exact result; and
every output is within 1e-5 * sum|w x| of the double GEMV (O6)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu


def _mf(D, x=None):
    from gpu_util import DEV
    x = D.x if x is None else x
    y = torch.full((x.shape[0], D.rows), float("nan"), dtype=torch.float32, device=DEV)
    fb.fp8blk_gemv_mfma(D.codes, D.grid, x, y)
    return y


def _mf_twin(D, slab, x=None):
    from gpu_util import DEV
    x = D.x if x is None else x
    y = torch.full((x.shape[0], D.rows), float("nan"), dtype=torch.float32, device=DEV)
    fb.bf16_gemv_twin_mfma(slab, x, y)
    return y


def _check(L, Ms=None, nthreads=None):
    from gpu_util import DevLinear, assert_within_tolerance, u32, say
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1)
    slab = D.slab()
    for M in (Ms or [L.M]):
        say(f"  mfma {L.name or (L.rows, L.cols)} M={M}")
        x = D.x[:M].contiguous()
        y8 = _mf(D, x).cpu().numpy()
        yt = _mf_twin(D, slab, x).cpu().numpy()
        assert np.array_equal(u32(y8), u32(yt)), "matrix-core FP8 arm and bf16 twin differ"
        y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x[:M], nthreads=nthreads)
        assert_within_tolerance(y8, y64, yabs, what=f"mfma {L.rows}x{L.cols} M={M}")


# The one-shot single calls (each wave's 2, 4 or 8 windows loaded at once) are
# among these: (1000, 1024, 4) with two row groups per workgroup, (300, 1008, 3)
# and (500, 4080, 2) with a ragged last window, (4099, 4080, 1) with four-wave
# workgroups and a ragged last row group; the others take the two-deep pipeline.
CASES = [(1, 16, 1), (3, 48, 2), (17, 1040, 3), (129, 2064, 16), (130, 3088, 5), (257, 4112, 8),
         (64, 16400, 2), (100, 4096, 16), (2, 65536, 1), (33, 65536, 16), (1000, 1024, 4), (4097, 272, 9),
         (300, 1008, 3), (500, 4080, 2), (4099, 4080, 1)]


@pytest.mark.parametrize("rows,cols,M", CASES)
def test_mfma_parity(gpu, rows, cols, M):
    _check(inputs.host_linear(rows, cols, M, 11 * rows + cols + M))


def test_mfma_batch_invariance(gpu):
    from gpu_util import DevLinear, u32
    L = inputs.host_linear(1536, 4096, 16, 77)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    slab = D.slab()
    singles = [u32(_mf(D, D.x[m:m + 1].contiguous())) for m in range(16)]
    for M in (2, 3, 4, 7, 8, 16):
        yp = u32(_mf(D, D.x[:M].contiguous()))
        ypt = u32(_mf_twin(D, slab, D.x[:M].contiguous()))
        for m in range(M):
            assert np.array_equal(yp[m], singles[m][0]), (M, m)
            assert np.array_equal(ypt[m], singles[m][0]), (M, m)


def test_mfma_integer_exact_and_one_hot(gpu):
    from gpu_util import DevLinear, DEV
    from test_gpu_gemv import _integer_case
    codes, scales, x, exact, W = _integer_case(260, 3088, 16, 9)
    D = DevLinear(codes, scales, x)
    D.check()
    assert np.array_equal(_mf(D).cpu().numpy().astype(np.float64), exact)
    cols_hit = [0, 7, 8, 15, 16, 63, 64, 3087]
    xf = np.zeros((len(cols_hit), 3088), dtype=np.float32)
    for k, c in enumerate(cols_hit):
        xf[k, c] = 1.0
    xo = torch.from_numpy(inputs.round_to_bf16_bits(xf).view(np.int16)).to(DEV)
    y = _mf(D, xo).cpu().numpy()
    for k, c in enumerate(cols_hit):
        assert np.array_equal(y[k].astype(np.float64), W[:, c])


def test_mfma_determinism(gpu):
    from gpu_util import DevLinear, u32
    L = inputs.host_linear(2048, 4096, 8, 5)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    y0 = u32(_mf(D))
    for _ in range(3):
        assert np.array_equal(u32(_mf(D)), y0)


def test_mfma_workloads(gpu):
    import os
    n = min(16, os.cpu_count() or 1)
    _check(inputs.decode_shape(), nthreads=n)
    for L in inputs.projection_pair():
        _check(L, nthreads=n)
    for L in inputs.verify_panel():
        _check(L, Ms=[1] + list(inputs.VERIFY_M), nthreads=n)


def test_mfma_refusals(gpu):
    lib = fb.load()
    P = 1 << 12
    assert lib.fp8blk_gemv_mfma(P, P, 4, 24, P, 1, P, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_mfma(P, P, 4, 16, P, 17, P, None) == fb.ERR_ARG
    assert lib.bf16_gemv_twin_mfma(P + 2, 4, 16, P, 1, P, None) == fb.ERR_ARG
