"""GPU parity: fp8blk_gemv and bf16_gemv_twin against the oracle, at sizes the
oracle finishes in seconds (several segments, ragged tails, every M).

For every case: the FP8 GEMV and its bf16 twin give identical bits; both
equal the documented-order f32 emulation (O7) bit for bit; both are within
1e-5 * sum|w x| of the double GEMV (O6)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu


def _run(L):
    from gpu_util import DevLinear
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1)
    slab = D.slab()
    y8 = D.gemv()
    yt = D.twin(slab)
    torch.cuda.synchronize()
    return D, slab, y8.cpu().numpy(), yt.cpu().numpy()


CASES = [
    # rows, cols, M, codes kind
    (1, 16, 1, "uniform"), (1, 1024, 1, "normal"), (3, 48, 2, "uniform"), (5, 1040, 3, "normal"),
    (128, 512, 1, "uniform"), (129, 2064, 4, "normal"), (130, 3088, 5, "normal"), (257, 4112, 1, "normal"),
    (64, 16400, 2, "normal"), (300, 8192, 8, "normal"), (100, 4096, 16, "normal"), (17, 6160, 7, "normal"),
    (2, 65536, 1, "normal"), (9, 65536, 16, "normal"), (1000, 1024, 1, "normal"), (4097, 272, 9, "uniform"),
]


@pytest.mark.parametrize("rows,cols,M,kind", CASES)
def test_gemv_parity(gpu, rows, cols, M, kind):
    from gpu_util import full_parity, say
    say(f"gemv parity rows={rows} cols={cols} M={M} {kind}")
    L = inputs.host_linear(rows, cols, M, 7 * rows + cols + M, codes=kind,
                           **({"scale_lo": 120, "scale_hi": 134} if kind == "uniform" else {}))
    _D, _s, y8, yt = _run(L)
    full_parity(L, L.codes, L.scales, L.x, y8, yt, what=f"{rows}x{cols} M={M}")


# M = 1 linears of 4096 rows or more take two rows per wave; from 16384 rows
# (at most 8 segments) two segments per wave, the row split over 2 or 4
# waves. Ragged rows and cols on each of these paths.
PLAN_CASES = [(4097, 3088), (8191, 8192), (16385, 2064), (16391, 5136)]


# M = 2 with at most 4 segments runs the same one-shot kernel with two
# activation rows: two rows per wave and four segments per wave from 4096
# rows (ragged rows and cols, 3 and 4 segments), two segments (cols 2048,
# ragged rows) and one (cols 1008, four rows per wave).
M2_CASES = [(4097, 3088), (5003, 2064), (4099, 2048), (257, 1008), (12288, 4096)]


@pytest.mark.parametrize("rows,cols", M2_CASES)
def test_gemv_parity_two_activation_rows(gpu, rows, cols):
    from gpu_util import full_parity, say
    say(f"gemv parity rows={rows} cols={cols} M=2 (one-shot, two activation rows)")
    L = inputs.host_linear(rows, cols, 2, 13 * rows + cols)
    _D, _s, y8, yt = _run(L)
    full_parity(L, L.codes, L.scales, L.x, y8, yt, nthreads=16, what=f"{rows}x{cols} M=2")


@pytest.mark.parametrize("rows,cols", PLAN_CASES)
def test_gemv_parity_two_rows_per_wave(gpu, rows, cols):
    from gpu_util import full_parity, say
    say(f"gemv parity rows={rows} cols={cols} M=1 (two rows per wave)")
    L = inputs.host_linear(rows, cols, 1, 11 * rows + cols)
    _D, _s, y8, yt = _run(L)
    full_parity(L, L.codes, L.scales, L.x, y8, yt, nthreads=16, what=f"{rows}x{cols} M=1")


def test_gemv_tiny_config(gpu):
    from gpu_util import full_parity
    L = inputs.tiny()
    _D, _s, y8, yt = _run(L)
    full_parity(L, L.codes, L.scales, L.x, y8, yt, what="tiny")


def _integer_case(rows, cols, M, seed):
    rng = np.random.default_rng(seed)
    e4 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    ok = [c for c in range(256) if not np.isnan(float(e4[c])) and float(e4[c]).is_integer()
          and abs(float(e4[c])) <= 16]
    codes = np.array(ok, dtype=np.uint8)[rng.integers(0, len(ok), size=(rows, cols))]
    gr, gc = inputs.grid_shape(rows, cols)
    scales = (127 + rng.integers(-3, 4, size=(gr, gc))).astype(np.uint8)
    xi = rng.integers(-8, 9, size=(M, cols)).astype(np.float32)
    W = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
         * torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64)
         .repeat_interleave(128, 0)[:rows].repeat_interleave(128, 1)[:, :cols]).numpy()
    return codes, scales, inputs.round_to_bf16_bits(xi), xi.astype(np.float64) @ W.T, W


@pytest.mark.parametrize("rows,cols,M", [(131, 3088, 3), (64, 16384, 1), (513, 1040, 16)])
def test_integer_exact_pin(gpu, rows, cols, M):
    """Every f32 order is exact on these inputs: the GPU must give the exact sum
    whatever order it uses (pins the layout, the scale mapping, every term)."""
    codes, scales, x, exact, _W = _integer_case(rows, cols, M, rows * cols)
    L = inputs.Linear(rows, cols, codes, scales, x, 0)
    _D, _s, y8, yt = _run(L)
    assert np.array_equal(y8.astype(np.float64), exact)
    assert np.array_equal(yt.astype(np.float64), exact)


def test_one_hot_x_reads_one_column(gpu):
    from gpu_util import DevLinear, DEV
    codes, scales, _x, _e, W = _integer_case(384, 2064, 1, 5)
    D = DevLinear(codes, scales)
    assert D.check(check=False) == (0, -1)
    cols_hit = [0, 15, 16, 1023, 1024, 1039, 2063]
    xf = np.zeros((len(cols_hit), 2064), dtype=np.float32)
    for i, c in enumerate(cols_hit):
        xf[i, c] = 1.0
    x = torch.from_numpy(inputs.round_to_bf16_bits(xf).view(np.int16)).to(DEV)
    y = D.gemv(x).cpu().numpy()
    for i, c in enumerate(cols_hit):
        assert np.array_equal(y[i].astype(np.float64), W[:, c])


def test_batch_invariance(gpu):
    """Row m of an M-row call equals the single-row call on x[m], bit for bit,
    for every panel size (the batched-verify requirement)."""
    from gpu_util import DevLinear, u32
    L = inputs.host_linear(1536, 4096, 16, 99)
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1)
    slab = D.slab()
    singles = [u32(D.gemv(D.x[m:m + 1].contiguous())) for m in range(16)]
    for M in (2, 3, 4, 5, 8, 11, 16):
        yp = u32(D.gemv(D.x[:M].contiguous()))
        ypt = u32(D.twin(slab, D.x[:M].contiguous()))
        for m in range(M):
            assert np.array_equal(yp[m], singles[m][0]), (M, m)
            assert np.array_equal(ypt[m], singles[m][0]), (M, m)


def test_invariances_sign_scale_determinism(gpu):
    from gpu_util import DevLinear, u32
    L = inputs.host_linear(700, 5136, 2, 123)
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1)
    y = D.gemv().cpu().numpy()
    for _ in range(3):
        assert np.array_equal(u32(D.gemv()), y.view(np.uint32))
    Dn = DevLinear(L.codes ^ np.uint8(0x80), L.scales, L.x)
    assert Dn.check(check=False) == (0, -1)
    assert np.array_equal(Dn.gemv().cpu().numpy(), -y)
    Dx = DevLinear(L.codes, L.scales, L.x ^ np.uint16(0x8000))
    Dx.check()
    assert np.array_equal(Dx.gemv().cpu().numpy(), -y)
    Ds = DevLinear(L.codes, L.scales + np.uint8(5), L.x)
    Ds.check()
    assert np.array_equal(Ds.gemv().cpu().numpy(), y * np.float32(32))


def test_extreme_scales_subnormal_weights(gpu):
    """Scale codes at the edges of the legal range: weights that are f32
    subnormals (2^-133 .. 2^-126) and weights near the top of bf16's range."""
    from gpu_util import full_parity
    rows, cols = 256, 1024
    rng = np.random.default_rng(4)
    codes = inputs.FINITE_E4M3[rng.integers(0, 254, size=(rows, cols))]
    scales = np.array([[3, 4, 5, 6, 230, 231, 232, 233], [126, 127, 128, 3, 4, 120, 130, 234]], dtype=np.uint8)
    c = codes  # every finite code is exact at scale codes 3..246
    assert oracle.load_check(c, scales)[0] == 0
    x = inputs.round_to_bf16_bits(rng.standard_normal((2, cols), dtype=np.float32))
    L = inputs.Linear(rows, cols, c, scales, x, 0)
    _D, _s, y8, yt = _run(L)
    assert np.all(np.isfinite(y8))
    full_parity(L, c, scales, x, y8, yt, what="extreme scales")


def test_zero_weights_give_positive_zero(gpu):
    from gpu_util import DevLinear, u32
    rows, cols = 130, 2048
    codes = np.zeros((rows, cols), dtype=np.uint8)
    codes[:, ::2] = 0x80  # -0.0 weights
    scales = np.full(inputs.grid_shape(rows, cols), 127, dtype=np.uint8)
    x = inputs.round_to_bf16_bits(np.random.default_rng(1).standard_normal((3, cols), dtype=np.float32))
    D = DevLinear(codes, scales, x)
    D.check()
    y = u32(D.gemv())
    y7 = oracle.gemv_f32_order(x, codes=codes, scales=scales)
    assert np.array_equal(y, y7.view(np.uint32))
    assert np.all(y == 0)  # +0.0 exactly: the chain starts from +0.0


def test_streams_and_ws_none(gpu):
    from gpu_util import DevLinear, DEV, u32
    L = inputs.host_linear(512, 2048, 1, 8)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    y0 = u32(D.gemv())
    s = torch.cuda.Stream(device=DEV)
    y = torch.empty((1, 512), dtype=torch.float32, device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fb.fp8blk_gemv(D.codes, D.grid, D.x, y, ws=None, stream=s)
    s.synchronize()
    assert np.array_equal(u32(y), y0)


def test_device_side_refusals(gpu):
    """Argument errors with real device buffers: status, and y left untouched."""
    from gpu_util import DevLinear, DEV
    L = inputs.host_linear(128, 1024, 1, 3)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    y = torch.full((1, 128), 7.0, device=DEV)
    lib = fb.load()
    assert lib.fp8blk_gemv(D.codes.data_ptr(), D.grid.data_ptr(), 128, 1024, D.x.data_ptr(), 0,
                           y.data_ptr(), None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(D.codes.data_ptr() + 1, D.grid.data_ptr(), 128, 1024, D.x.data_ptr(), 1,
                           y.data_ptr(), None, 0, None) == fb.ERR_ARG
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
