"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (the same entry points and shapes).

Workloads 1-4 are drawn on the host and checked in full: FP8 == twin bitwise,
== documented order (O7) bitwise, within 1e-5 * sum|w x| of the double GEMV
(O6). The whole-step sweep (259 linears, ~3.2e9 codes) is drawn on the device;
FP8 == twin is checked on every output on the GPU, and every linear is copied
back whole and every output checked against O7 (bitwise) and O6."""
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


def _check_linear(L, Ms=None):
    from gpu_util import DevLinear, full_parity, say
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1), L.name
    slab = D.slab()
    for M in (Ms or [L.M]):
        say(f"  {L.name} M={M}")
        x = D.x[:M].contiguous()
        y8 = D.gemv(x).cpu().numpy()
        yt = D.twin(slab, x).cpu().numpy()
        full_parity(L, L.codes, L.scales, L.x[:M], y8, yt, nthreads=NTHREADS, what=f"{L.name} M={M}")


def test_config_decode_shape(gpu):
    _check_linear(inputs.decode_shape())


def test_config_projection_pair(gpu):
    for L in inputs.projection_pair():
        _check_linear(L)


def test_config_verify_panel(gpu):
    for L in inputs.verify_panel():
        _check_linear(L, Ms=list(inputs.VERIFY_M) + [1])


def test_config_whole_step_sweep(gpu):
    from gpu_util import DEV, assert_within_tolerance, say, u32
    sw = inputs.sweep_plan()
    xs = {c: inputs.device_x(c, 1, 7 + c, DEV) for c in {l.cols for l in sw.linears}}
    slab = torch.empty(max(l.rows * l.cols for l in sw.linears), dtype=torch.int16, device=DEV)
    for i, spec in enumerate(sw.linears):
        codes, scales = inputs.device_linear(spec.rows, spec.cols, spec.seed, DEV)
        from gpu_util import DevLinear
        D = DevLinear(codes, scales, xs[spec.cols])
        assert D.check(check=False) == (0, -1), spec.name
        s = slab[: spec.rows * spec.cols].view(spec.rows, spec.cols)
        fb.fp8blk_dequant_bf16(D.codes, D.grid, s)
        y8, yt = D.gemv(), D.twin(s)
        assert torch.equal(y8.view(torch.int32), yt.view(torch.int32)), spec.name
        # every row: the codes, scales and outputs come back whole
        xh = D.x.cpu().numpy().view(np.uint16)
        ch, sh = codes.cpu().numpy(), scales.cpu().numpy()
        yh = y8.cpu().numpy()
        y7 = oracle.gemv_f32_order(xh, codes=ch, scales=sh, nthreads=NTHREADS)
        assert np.array_equal(u32(yh), y7.view(np.uint32)), spec.name
        y64, yabs = oracle.gemv_f64(ch, sh, xh, nthreads=NTHREADS)
        assert_within_tolerance(yh, y64, yabs, what=spec.name)
        del ch, sh, yh, y7, y64, yabs
        if i % 43 == 0 or spec.name == "head":
            say(f"  sweep linear {i} {spec.name} {spec.rows}x{spec.cols} ok")
        del codes, scales, D
