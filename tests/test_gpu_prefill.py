"""GPU: the staged prefill GEMM (fp8blk_gemm_staged: bf16 dequant slab, then
one hipBLASLt bf16 x bf16 -> f32 GEMM) and its twin over a caller-held slab.

The library GEMM's summation order is its own, so there is no bitwise oracle.
What is checked: the staged path and the twin give identical bits (the same
GEMM on the same exact slab); the slab the staged path writes equals the
oracle's dequant (O5); inputs on which every order is exact give the exact
result; every output is within gamma_cols * sum|w x| of the double GEMM (O6),
the bound for any order of exact f32 products; and panels of one row equal
the matching rows of a long panel to that bound."""
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
U = 2.0 ** -24


def gamma(k):
    return k * U / (1 - k * U)


def _ws(op, rows, cols, N):
    from gpu_util import DEV
    return torch.empty(fb.fp8blk_workspace_bytes(op, rows, cols, N), dtype=torch.uint8, device=DEV)


def _staged(D, x):
    from gpu_util import DEV
    y = torch.full((x.shape[0], D.rows), float("nan"), device=DEV)
    ws = _ws(fb.OP_GEMM_STAGED, D.rows, D.cols, x.shape[0])
    fb.fp8blk_gemm_staged(D.codes, D.grid, x, y, ws)
    return y, ws


def _twin(slab, x):
    from gpu_util import DEV
    rows, cols = slab.shape
    y = torch.full((x.shape[0], rows), float("nan"), device=DEV)
    fb.bf16_gemm_twin(slab, x, y, _ws(fb.OP_BF16_GEMM, rows, cols, x.shape[0]))
    return y


@pytest.mark.parametrize("rows,cols,N", [(256, 512, 64), (300, 4096, 128), (129, 2064, 33), (64, 16400, 7),
                                         (1, 16, 1), (1024, 4096, 256), (17, 1040, 300)])
def test_staged_gemm_parity(gpu, rows, cols, N):
    from gpu_util import DevLinear, say, u32
    say(f"  staged prefill {rows}x{cols} N={N}")
    L = inputs.host_linear(rows, cols, N, rows + 7 * cols + N)
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1)
    y, ws = _staged(D, D.x)
    torch.cuda.synchronize()
    # the slab it staged is the oracle's exact dequant
    slab = ws[: rows * cols * 2].view(torch.int16).view(rows, cols)
    assert np.array_equal(slab.cpu().numpy().view(np.uint16), oracle.dequant_bf16(L.codes, L.scales))
    yt = _twin(slab.clone(), D.x)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.array_equal(u32(yh), u32(yt)), "staged GEMM != bf16 twin GEMM"
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=NTHREADS)
    err = np.abs(yh.astype(np.float64) - y64)
    assert np.all(err <= gamma(cols) * yabs), float(np.max(err / np.maximum(yabs, 1e-300)))


def test_staged_gemm_integer_exact(gpu):
    from gpu_util import DevLinear
    from test_gpu_gemv import _integer_case
    codes, scales, x, exact, _W = _integer_case(260, 3088, 96, 21)
    D = DevLinear(codes, scales, x)
    D.check()
    y, _ = _staged(D, D.x)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), exact)


def test_staged_gemm_rows_of_a_long_panel(gpu):
    """A panel of one row and the same row inside a 512-row panel: both within
    the bound of the exact sum (the library may pick a different algorithm
    per shape, so the bits need not agree)."""
    from gpu_util import DevLinear
    L = inputs.host_linear(512, 4096, 512, 99)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    y, _ = _staged(D, D.x)
    y1, _ = _staged(D, D.x[5:6].contiguous())
    torch.cuda.synchronize()
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x[5:6], nthreads=NTHREADS)
    for row in (y[5:6].cpu().numpy(), y1.cpu().numpy()):
        assert np.all(np.abs(row.astype(np.float64) - y64) <= gamma(4096) * yabs)


def test_staged_gemm_workloads(gpu):
    """The decode-shape and projection linears as prefill panels of 2048 tokens:
    staged == twin bitwise, and sampled rows against the oracle."""
    from gpu_util import DEV, DevLinear, say, u32
    rng = np.random.default_rng(5)
    for L in [inputs.decode_shape()] + inputs.projection_pair():
        say(f"  prefill {L.name} {L.rows}x{L.cols} N=2048")
        D = DevLinear(L.codes, L.scales, None)
        assert D.check(check=False) == (0, -1)
        xh = inputs.round_to_bf16_bits(rng.standard_normal((2048, L.cols), dtype=np.float32))
        x = torch.from_numpy(xh.view(np.int16)).to(DEV)
        y, ws = _staged(D, x)
        slab = ws[: L.rows * L.cols * 2].view(torch.int16).view(L.rows, L.cols).clone()
        yt = _twin(slab, x)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), yt.view(torch.int32))
        tok = np.sort(rng.choice(2048, size=8, replace=False))
        r0 = 128 * int(rng.integers(0, L.rows // 128))
        y64, yabs = oracle.gemv_f64(L.codes[r0:r0 + 128], L.scales[r0 // 128:r0 // 128 + 1], xh[tok],
                                    nthreads=NTHREADS)
        got = y[torch.from_numpy(tok).to(DEV)][:, r0:r0 + 128].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - y64) <= gamma(L.cols) * yabs)


def test_staged_and_twin_share_the_algorithm(gpu):
    """Workspaces of different sizes and a graph-captured call still run the
    algorithm the shape's first call chose: staged == twin bitwise, and every
    replay of a captured twin call equals the eager call."""
    from gpu_util import DEV, DevLinear, say
    rows, cols, N = 768, 2048, 96
    L = inputs.host_linear(rows, cols, N, 4242)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    need_s = fb.fp8blk_workspace_bytes(fb.OP_GEMM_STAGED, rows, cols, N)
    need_t = fb.fp8blk_workspace_bytes(fb.OP_BF16_GEMM, rows, cols, N)
    ws_s = torch.empty(need_s + (3 << 20), dtype=torch.uint8, device=DEV)   # larger than needed
    ws_t = torch.empty(need_t + (9 << 20), dtype=torch.uint8, device=DEV)   # larger still
    y_s = torch.full((N, rows), float("nan"), device=DEV)
    fb.fp8blk_gemm_staged(D.codes, D.grid, D.x, y_s, ws_s)
    slab = ws_s[: rows * cols * 2].view(torch.int16).view(rows, cols).clone()
    y_t = torch.full((N, rows), float("nan"), device=DEV)
    fb.bf16_gemm_twin(slab, D.x, y_t, ws_t)
    torch.cuda.synchronize()
    assert torch.equal(y_s.view(torch.int32), y_t.view(torch.int32))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    y_g = torch.full((N, rows), float("nan"), device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        fb.bf16_gemm_twin(slab, D.x, y_g, ws_t, stream=cap)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"  captured prefill GEMM replay {rep}")
        y_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g.view(torch.int32), y_s.view(torch.int32)), rep
        _ = torch.randn(1 << 18, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()


def test_first_call_of_a_shape_under_capture_is_refused(gpu):
    """A shape's first call times the candidates, which capture cannot do: it
    returns FP8BLK_ERR_ARG, and an eager call afterwards works."""
    from gpu_util import DEV, DevLinear
    rows, cols, N = 384, 1024, 40  # a shape no other test uses
    L = inputs.host_linear(rows, cols, N, 4343)
    D = DevLinear(L.codes, L.scales, L.x)
    D.check()
    slab = D.slab()
    ws = _ws(fb.OP_BF16_GEMM, rows, cols, N)
    y = torch.full((N, rows), float("nan"), device=DEV)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        st = fb.bf16_gemm_twin(slab, D.x, y, ws, stream=cap, check=False)
    torch.cuda.synchronize()
    assert st == fb.ERR_ARG
    fb.bf16_gemm_twin(slab, D.x, y, ws)
    torch.cuda.synchronize()
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=NTHREADS)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - y64) <= gamma(cols) * yabs)
