"""GPU parity: fp8blk_load_check and fp8blk_dequant_bf16 against the oracle.

Verdicts (status and first bad index) must equal the oracle's; the f32 grid
and the bf16 slab must be bit-identical to the oracle's."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

FINITE = inputs.FINITE_E4M3


def _both(codes, scales):
    from gpu_util import DevLinear
    D = DevLinear(codes, scales)
    st, first = D.check(check=False)
    ost, ofirst, ogrid = oracle.load_check(codes, scales)
    assert (st, first) == (ost, ofirst), f"GPU ({st}, {first}) vs oracle ({ost}, {ofirst})"
    if st == 0:
        assert np.array_equal(D.grid.cpu().numpy().view(np.uint32), ogrid.view(np.uint32))
    return D, st, first


def _table():
    """Row block s (s = 0..254) has scale code s; row 0 of each block holds the
    254 finite codes then two zeros (256 columns = 2 column blocks with the
    same scale); every other element is 0."""
    rows, cols = 128 * 255, 256
    codes = np.zeros((rows, cols), dtype=np.uint8)
    for s in range(255):
        codes[128 * s, :254] = FINITE
    scales = np.repeat(np.arange(255, dtype=np.uint8)[:, None], 2, axis=1)
    return codes, scales


def _oracle_inexact_indices(codes, scales):
    """Row-major indices of the table's elements that the oracle calls inexact
    (O3 on e4m3(code) * e8m0(scale)), in increasing order."""
    out = []
    for s in range(255):
        sv = oracle.e8m0(s)
        for col, code in enumerate(FINITE):
            if not oracle.is_bf16_exact(oracle.e4m3(int(code)) * sv):
                out.append((128 * s) * 256 + col)
    return out


def test_exhaustive_inexact_set_matches_oracle(gpu):
    """Every (finite code, scale code) pair: clearing the reported first bad
    element until the check passes walks the GPU's whole inexact set in index
    order; it must be the oracle's set."""
    codes, scales = _table()
    want = _oracle_inexact_indices(codes, scales)
    st, first, _ = oracle.load_check(codes, scales)
    assert (st, first) == (fb.ERR_INEXACT, want[0])
    from gpu_util import DevLinear
    D = DevLinear(codes, scales)
    got = []
    for _ in range(len(want) + 1):
        st, first = D.check(check=False)
        if st == 0:
            break
        assert st == fb.ERR_INEXACT
        got.append(first)
        D.codes.view(-1)[first] = 0
    assert got == want
    rows_bad = {i // 256 // 128 for i in got}
    assert rows_bad == set(range(0, 3)) | set(range(247, 255))


def test_exhaustive_dequant_table(gpu):
    """All exact (code, scale) pairs, including every subnormal code at every
    scale and the f32-subnormal scales 2^-127..2^-125: bf16 slab bit-exact."""
    codes, scales = _table()
    c = codes.copy()
    c.reshape(-1)[_oracle_inexact_indices(codes, scales)] = 0
    D, st, _ = _both(c, scales)
    assert st == 0
    got = D.slab().cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.dequant_bf16(c, scales))


def test_refusals_and_precedence(gpu):
    L = inputs.host_linear(256, 384, 1, 11, codes="uniform", scale_lo=120, scale_hi=134)
    c1, s1 = L.codes.copy(), L.scales.copy()
    s1[1, 0] = 254
    c1[128:256, 0:128] = 0x38
    c1[130, 5] = 0x7E
    _, st, first = _both(c1, s1)
    assert (st, first) == (fb.ERR_INEXACT, 130 * 384 + 5)
    c2, s2 = L.codes.copy(), L.scales.copy()
    s2[0, 2] = 1
    c2[0:128, 256:384] = 0x38
    c2[7, 300] = 0x01
    c2[9, 260] = 0x81
    _, st, first = _both(c2, s2)
    assert (st, first) == (fb.ERR_INEXACT, 7 * 384 + 300)
    c3 = c2.copy()
    c3[20, 1] = 0xFF
    c3[5, 383] = 0x7F
    _, st, first = _both(c3, s2)
    assert (st, first) == (fb.ERR_NAN_CODE, 5 * 384 + 383)
    s4 = s2.copy()
    s4[1, 2] = 0xFF
    s4[1, 1] = 0xFF
    _, st, first = _both(c3, s4)
    assert (st, first) == (fb.ERR_SCALE_FF, 4)


@pytest.mark.parametrize("pos", [0, 15, 16, 1023, 131071, 200 * 272 + 271])
def test_nan_code_positions(gpu, pos):
    L = inputs.host_linear(256, 512, 1, 3, codes="uniform", scale_lo=124, scale_hi=130)
    c = L.codes.copy()
    c.reshape(-1)[pos] = 0xFF if pos % 2 else 0x7F
    _, st, first = _both(c, L.scales)
    assert (st, first) == (fb.ERR_NAN_CODE, pos)


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (129, 272), (200, 1040), (300, 4112)])
def test_ragged_shapes_check_and_dequant(gpu, rows, cols):
    L = inputs.host_linear(rows, cols, 1, rows + cols, codes="uniform", scale_lo=120, scale_hi=134)
    D, st, _ = _both(L.codes, L.scales)
    assert st == 0
    got = D.slab().cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.dequant_bf16(L.codes, L.scales))


def test_dequant_full_size_configs(gpu):
    from gpu_util import say
    for L in [inputs.tiny(), inputs.decode_shape(), inputs.projection_pair()[2]]:
        say("dequant", L.name)
        D, st, _ = _both(L.codes, L.scales)
        assert st == 0
        got = D.slab().cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.dequant_bf16(L.codes, L.scales)), L.name


def test_check_is_repeatable_and_ws_contents_irrelevant(gpu):
    L = inputs.tiny()
    from gpu_util import DevLinear
    D = DevLinear(L.codes, L.scales)
    D.ws.fill_(0)  # a stale "found at 0" must not leak into the verdict
    assert D.check(check=False) == (0, -1)
    D.ws.fill_(0xAB)
    assert D.check(check=False) == (0, -1)


def test_stream_argument_is_honoured(gpu):
    L = inputs.tiny()
    from gpu_util import DevLinear, DEV
    D = DevLinear(L.codes, L.scales)
    s = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(s):
        st, first = fb.fp8blk_load_check(D.codes, D.scales, D.grid, D.ws, stream=s)
    assert (st, first) == (0, -1)
