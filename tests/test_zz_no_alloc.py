"""GPU: fp8blk_load_check_noalloc, the load check for callers that cannot
allocate device memory, against fp8blk_load_check (which takes a workspace).

Two calls in a row, the second on a smaller input, for each outcome: the
static scratch keeps the previous call's verdict, so a refusal followed by a
clean, smaller linear checks that every call starts from cleared slots. The
status, first_bad and the decoded f32 grid must equal the workspace entry
point's, and the oracle's (O4)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu


def _both(codes, scales):
    from gpu_util import DEV, to_dev
    c, s = to_dev(codes), to_dev(scales)
    g_ws = torch.full(scales.shape, float("nan"), dtype=torch.float32, device=DEV)
    g_na = torch.full(scales.shape, float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(fb.fp8blk_workspace_bytes(fb.OP_LOAD_CHECK, *codes.shape), dtype=torch.uint8, device=DEV)
    r_ws = fb.fp8blk_load_check(c, s, g_ws, ws, check=False)
    r_na = fb.fp8blk_load_check_noalloc(c, s, g_na, check=False)
    return r_ws, r_na, g_ws.cpu().numpy(), g_na.cpu().numpy()


def _linear(rows, cols, seed, bad=None):
    L = inputs.host_linear(rows, cols, 1, seed, codes="uniform", scale_lo=120, scale_hi=134)
    codes, scales = L.codes.copy(), L.scales.copy()
    if bad == "nan":
        codes[rows // 2, cols - 3] = 0x7F
        codes[rows - 1, 5] = 0xFF
    elif bad == "scale_ff":
        scales[-1, -1] = 0xFF
    elif bad == "inexact":
        codes[1, 17] = 0x01  # 2^-9 ...
        scales[0, 0] = 0     # ... times 2^-127 is below bf16's spacing
    return codes, scales


@pytest.mark.parametrize("first,second", [("nan", None), ("scale_ff", "inexact"), (None, "nan"),
                                          ("inexact", None), (None, None)])
def test_noalloc_matches_workspace_entry_point(gpu, first, second):
    from gpu_util import say
    for k, (rows, cols, bad) in enumerate([(1000, 4112, first), (130, 272, second)]):
        say(f"load check without allocation: call {k + 1}, {rows}x{cols}, {bad or 'clean'}")
        codes, scales = _linear(rows, cols, 60 + 7 * k + len(str(first)), bad)
        r_ws, r_na, g_ws, g_na = _both(codes, scales)
        ost, ofb, ogrid = oracle.load_check(codes, scales)
        assert r_na == r_ws == (ost, ofb), (k, bad, r_na, r_ws, (ost, ofb))
        if ost == 0:
            assert np.array_equal(g_na.view(np.uint32), g_ws.view(np.uint32))
            assert np.array_equal(g_na.view(np.uint32), ogrid.view(np.uint32))


def test_noalloc_allocates_nothing(gpu):
    """The call leaves torch's allocator untouched and needs no workspace."""
    from gpu_util import DEV, to_dev
    codes, scales = _linear(256, 512, 3)
    c, s = to_dev(codes), to_dev(scales)
    g = torch.empty(scales.shape, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0)
    for _ in range(3):
        assert fb.fp8blk_load_check_noalloc(c, s, g) == (0, -1)
    after = torch.cuda.memory_stats(DEV).get("allocation.all.allocated", 0)
    assert after == before


def test_noalloc_argument_errors(gpu):
    lib = fb.load()
    P = 1 << 12
    fbad = __import__("ctypes").c_int64(7)
    assert lib.fp8blk_load_check_noalloc(None, P, 4, 16, P, __import__("ctypes").byref(fbad), None) == fb.ERR_ARG
    assert fbad.value == -1
    assert lib.fp8blk_load_check_noalloc(P, P, 4, 24, P, None, None) == fb.ERR_ARG
    assert lib.fp8blk_load_check_noalloc(P + 1, P, 4, 16, P, None, None) == fb.ERR_ARG
