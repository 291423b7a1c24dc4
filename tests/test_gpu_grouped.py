"""GPU: a grouped launch gives, for every member, the same bits as a call of
its own (FP8 arm and bf16 twin, single-row and panel kernels), and each
member's output equals the oracle's documented-order f32 emulation (O7) bit
for bit and lies within 1e-5 * sum|w x| of the double GEMV (O6)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows_list,cols,M", [
    ((4096, 1024), 4096, 1),            # q + kv
    ((2048, 2048), 4096, 1),            # gate + up
    ((129, 3, 1000), 2064, 1),          # ragged rows, 3 segments
    ((256, 256, 512, 17, 1, 300, 64, 5), 1040, 1),  # eight members
    ((300, 77), 16400, 1),              # more than 16 segments: the panel kernel
    ((1536, 512), 4096, 16),            # verify panel
    ((130, 260), 3088, 5),
])
def test_grouped_equals_separate(gpu, rows_list, cols, M):
    from gpu_util import DevLinear, DEV, u32
    from gpu_util import assert_within_tolerance
    x = xh = None
    Ds, Ls, ys_sep, ys_grp, slabs, ts_sep, ts_grp = [], [], [], [], [], [], []
    for k, rows in enumerate(rows_list):
        L = inputs.host_linear(rows, cols, M, 1000 * k + rows + cols)
        Ls.append(L)
        if x is None:
            xh = L.x
            x = torch.from_numpy(L.x.view(np.int16)).to(DEV)
        D = DevLinear(L.codes, L.scales, x)
        D.check()
        Ds.append(D)
        slabs.append(D.slab())
        ys_sep.append(D.gemv(x))
        ts_sep.append(D.twin(slabs[-1], x))
        ys_grp.append(torch.full((M, rows), float("nan"), device=DEV))
        ts_grp.append(torch.full((M, rows), float("nan"), device=DEV))
    fb.fp8blk_gemv_grouped([(D.codes, D.grid, y) for D, y in zip(Ds, ys_grp)], x)
    fb.bf16_gemv_twin_grouped([(s, y) for s, y in zip(slabs, ts_grp)], x)
    torch.cuda.synchronize()
    for L, a, b, c, d in zip(Ls, ys_sep, ys_grp, ts_sep, ts_grp):
        assert np.array_equal(u32(a), u32(b))
        assert np.array_equal(u32(c), u32(d))
        assert np.array_equal(u32(a), u32(d))
        yg = b.cpu().numpy()
        y7 = oracle.gemv_f32_order(xh, codes=L.codes, scales=L.scales)
        assert np.array_equal(u32(yg), y7.view(np.uint32)), (L.rows, "grouped != documented order")
        y64, yabs = oracle.gemv_f64(L.codes, L.scales, xh)
        assert_within_tolerance(yg, y64, yabs, what=f"grouped member {L.rows}x{cols} M={M}")
