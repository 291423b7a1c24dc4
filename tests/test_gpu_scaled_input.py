"""GPU: the scaled-input launches (fp8blk_gemv_scaled_input and its grouped
form), where a dependent linear reads x = bf16(c * src) of an earlier
linear's f32 output ("Module dsv4_gpu" page, DecodePath), formed inside the
kernel's x loads; and the next-input launches (fp8blk_gemv_next_input and its
grouped form), where the producer writes that x beside its output.

Checked: every output equals, bit for bit, fp8blk_gemv / fp8blk_gemv_grouped
on x formed on the host from the same src and c (the f32 product rounded to
nearest even, IEEE subnormals kept); on some shapes every output also
equals the oracle's documented order (O7) bit for bit and lies within 1e-5 of
the double GEMV (O6). Shapes cover every single-row plan (1 to 16 segments,
one to four rows per wave, split rows), ragged rows and a ragged last segment;
src covers ties, bf16 subnormals, overflow of c * src and infinities."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

# (rows, cols): T = 1, 2 (R = 4, 2), T = 3..4 under 4096 rows (R = 1), from
# 4096 rows (R = 2), from 16384 rows at T <= 8 (TPW = 2), split rows (sw = 2, 4)
SHAPES = [(5, 16), (257, 1008), (1031, 2048), (13, 3088), (4096, 4096), (4099, 4096), (16384, 4096),
          (1000, 8192), (4096, 16384), (600, 12304)]


def _src(n, seed, special=False):
    g = np.random.default_rng(seed)
    s = (g.standard_normal(n) * 3.0).astype(np.float32)
    if special:
        k = np.arange(n)
        # exact ties of the bf16 rounding (odd and even lower halves), bf16
        # subnormals, values whose product with c overflows, infinities
        s[k % 11 == 1] = np.float32(1.0 + 2.0 ** -8)
        s[k % 11 == 2] = np.float32(1.0 + 3 * 2.0 ** -8)
        s[k % 11 == 3] = np.float32(2.0 ** -130)
        s[k % 11 == 4] = np.float32(-3.0e-39)
        s[k % 97 == 5] = np.float32(3.0e38)
        s[k % 131 == 6] = np.float32(np.inf)
        s[k % 139 == 7] = np.float32(-np.inf)
    return s


def _x_host(src, c, dev):
    """x = bf16(c * src) formed on the host, as a [1, cols] device panel."""
    xh = inputs.round_to_bf16_bits(np.float32(c) * np.asarray(src, dtype=np.float32))
    return torch.from_numpy(xh.view(np.int16).reshape(1, -1).copy()).to(dev)


def _same(a, b):
    """Bitwise equal, NaN allowed where both are NaN."""
    a, b = a.view(torch.int32), b.view(torch.int32)
    an = torch.isnan(a.view(torch.float32))
    bn = torch.isnan(b.view(torch.float32))
    return bool(torch.equal(an, bn)) and bool(torch.equal(a[~an], b[~bn]))


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_scaled_input_equals_gemv_on_formed_x(gpu, rows, cols):
    from gpu_util import DEV, DevLinear, say
    say(f"  scaled input {rows}x{cols}")
    L = inputs.host_linear(rows, cols, 1, 1200 + rows % 97 + cols)
    D = DevLinear(L.codes, L.scales)
    assert D.check()[0] == fb.OK
    for special, c in ((False, 0.75), (True, 1.0), (True, 0.3)):
        sh = _src(cols, rows + cols, special)
        src = torch.from_numpy(sh).to(DEV)
        x = _x_host(sh, c, DEV)
        y_ref = torch.full((1, rows), float("nan"), dtype=torch.float32, device=DEV)
        fb.fp8blk_gemv(D.codes, D.grid, x, y_ref)
        y = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
        fb.fp8blk_gemv_scaled_input(D.codes, D.grid, src, c, y)
        torch.cuda.synchronize()
        assert _same(y, y_ref.view(-1)), (rows, cols, special, c)
        if not special:
            assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("rows,cols", [(1031, 2048), (4099, 4096), (600, 12304)])
def test_scaled_input_against_oracle(gpu, rows, cols):
    import oracle
    from gpu_util import DEV, DevLinear, assert_within_tolerance, say, u32
    say(f"  scaled input vs oracle {rows}x{cols}")
    L = inputs.host_linear(rows, cols, 1, 1300 + cols)
    D = DevLinear(L.codes, L.scales)
    assert D.check()[0] == fb.OK
    c = 0.625
    s = _src(cols, 77 + cols)
    y = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    fb.fp8blk_gemv_scaled_input(D.codes, D.grid, torch.from_numpy(s).to(DEV), c, y)
    yh = y.cpu().numpy().reshape(1, -1)
    x = inputs.round_to_bf16_bits(np.float32(c) * s).reshape(1, -1)
    y7 = oracle.gemv_f32_order(x, codes=L.codes, scales=L.scales)
    assert int(np.sum(u32(yh) != u32(y7))) == 0
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, x)
    assert_within_tolerance(yh, y64, yabs, what=f"scaled input {rows}x{cols}")


def test_grouped_scaled_input(gpu):
    """A group of three (ragged rows) and a group of one, twice in a row on
    the same outputs; each equals fp8blk_gemv_grouped on the formed x."""
    from gpu_util import DEV, DevLinear, say
    for cols, rows_list in ((4096, [1024, 77, 600]), (3088, [4099])):
        say(f"  grouped scaled input cols={cols} rows={rows_list}")
        Ds = []
        for k, rows in enumerate(rows_list):
            L = inputs.host_linear(rows, cols, 1, 1400 + 7 * k + cols)
            D = DevLinear(L.codes, L.scales)
            assert D.check()[0] == fb.OK
            Ds.append(D)
        sh = _src(cols, 9 + cols, True)
        src = torch.from_numpy(sh).to(DEV)
        c = 1.25
        x = _x_host(sh, c, DEV)
        ref = [torch.full((1, D.rows), float("nan"), dtype=torch.float32, device=DEV) for D in Ds]
        fb.fp8blk_gemv_grouped([(D.codes, D.grid, r) for D, r in zip(Ds, ref)], x)
        ys = [torch.full((D.rows,), float("nan"), dtype=torch.float32, device=DEV) for D in Ds]
        for rep in range(2):
            fb.fp8blk_gemv_grouped_scaled_input([(D.codes, D.grid, y) for D, y in zip(Ds, ys)], src, c)
            torch.cuda.synchronize()
            for D, y, r in zip(Ds, ys, ref):
                assert _same(y, r.view(-1)), (cols, D.rows, rep)


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_next_input_equals_gemv(gpu, rows, cols):
    """y equals fp8blk_gemv's bit for bit and x_next equals the host's
    bf16(c * y) (nearest even) bit for bit, with a c that makes some products
    overflow to infinity."""
    from gpu_util import DEV, DevLinear, say
    say(f"  next input {rows}x{cols}")
    L = inputs.host_linear(rows, cols, 1, 1500 + rows % 89 + cols)
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check()[0] == fb.OK
    x = D.x[:1].contiguous()
    y_ref = torch.full((1, rows), float("nan"), dtype=torch.float32, device=DEV)
    fb.fp8blk_gemv(D.codes, D.grid, x, y_ref)
    torch.cuda.synchronize()
    amax = float(y_ref.abs().max())
    for c in (0.75, min(1.0e39 / max(amax, 1e-30), 1.0e38)):
        y = torch.full((1, rows), float("nan"), dtype=torch.float32, device=DEV)
        xn = torch.full((rows,), -1, dtype=torch.int16, device=DEV)
        fb.fp8blk_gemv_next_input(D.codes, D.grid, x, y, c, xn)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), (rows, cols, c)
        want = inputs.round_to_bf16_bits(np.float32(c) * y.cpu().numpy().reshape(-1))
        assert np.array_equal(xn.cpu().numpy().view(np.uint16), want), (rows, cols, c)


def test_grouped_next_input(gpu):
    """A group of three (ragged rows): the outputs equal fp8blk_gemv_grouped's,
    and x_next is bf16(c * y) of the chosen linear, for each choice k."""
    from gpu_util import DEV, DevLinear, say
    cols, rows_list = 4096, [1024, 77, 600]
    Ds = []
    for j, rows in enumerate(rows_list):
        L = inputs.host_linear(rows, cols, 1, 1600 + 7 * j)
        D = DevLinear(L.codes, L.scales, L.x)
        assert D.check()[0] == fb.OK
        Ds.append(D)
    x = Ds[0].x[:1].contiguous()
    ref = [torch.full((1, D.rows), float("nan"), dtype=torch.float32, device=DEV) for D in Ds]
    fb.fp8blk_gemv_grouped([(D.codes, D.grid, r) for D, r in zip(Ds, ref)], x)
    for k in range(3):
        say(f"  grouped next input k={k}")
        ys = [torch.full((1, D.rows), float("nan"), dtype=torch.float32, device=DEV) for D in Ds]
        xn = torch.full((Ds[k].rows,), -1, dtype=torch.int16, device=DEV)
        fb.fp8blk_gemv_grouped_next_input([(D.codes, D.grid, y) for D, y in zip(Ds, ys)], x, k, 0.5, xn)
        torch.cuda.synchronize()
        for y, r in zip(ys, ref):
            assert torch.equal(y.view(torch.int32), r.view(torch.int32)), k
        want = inputs.round_to_bf16_bits(np.float32(0.5) * ys[k].cpu().numpy().reshape(-1))
        assert np.array_equal(xn.cpu().numpy().view(np.uint16), want), k
