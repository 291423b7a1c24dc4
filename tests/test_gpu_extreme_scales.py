"""GPU parity of every dense arm at the edges of what the load check accepts.

"Module dsv4_gpu" page, struct Fp8Dense: every weight the load check accepts
is an exact bf16 value, and the arms that read it agree. These cases put whole
rows at the extremes, so the small values are not hidden in the tolerance of
larger ones in the same row:
  - scale codes 3..9: weights down to 2^-133 (bf16 subnormals), products in
    f32's subnormal range;
  - scale codes 0..2 with only the codes the load check accepts there;
  - the 14 subnormal e4m3 codes (and signed zeros) at small and middle scales;
  - scale codes 238..246: weights up to 1.75 * 2^127 (x scaled down so that no
    sum passes f32's largest value);
  - bf16-subnormal activations against ordinary weights.
For each: the matrix-core single call and its twin, the matrix-core sequence
and its twin, the vector GEMV and its twin give identical bits within their
arm; every output is within 1e-5 * sum|w x| of the double GEMV (O6); the
vector arm equals the documented order (O7) bit for bit; row m of a panel
equals the one-row call on x[m]."""
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
E4M3_SUBNORMAL = np.array([b | s for s in (0x00, 0x80) for b in range(0, 8)], dtype=np.uint8)  # incl. +-0


def _accepted_codes_at(scale_codes):
    """The finite e4m3 codes that the oracle's load check accepts at every one
    of the given scale codes (one 1x16 probe per code and scale)."""
    ok = []
    for c in inputs.FINITE_E4M3:
        probe = np.full((1, 16), c, dtype=np.uint8)
        if all(oracle.load_check(probe, np.array([[s]], dtype=np.uint8))[0] == 0 for s in scale_codes):
            ok.append(c)
    return np.array(ok, dtype=np.uint8)


def _case(kind, rows, cols, M, seed):
    rng = np.random.default_rng(seed)
    gr, gc = inputs.grid_shape(rows, cols)
    xv = rng.standard_normal((M, cols), dtype=np.float32)
    if kind == "tiny_scales":
        codes = inputs.FINITE_E4M3[rng.integers(0, 254, size=(rows, cols))]
        scales = rng.integers(3, 10, size=(gr, gc)).astype(np.uint8)
    elif kind == "scales_0_2":
        pool = _accepted_codes_at([0, 1, 2])
        assert 0 < pool.size < 254
        codes = pool[rng.integers(0, pool.size, size=(rows, cols))]
        scales = rng.integers(0, 3, size=(gr, gc)).astype(np.uint8)
    elif kind == "subnormal_codes":
        codes = E4M3_SUBNORMAL[rng.integers(0, E4M3_SUBNORMAL.size, size=(rows, cols))]
        # row blocks alternate between scale codes 3..9 and 124..130
        tiny_row = (np.arange(gr) % 2 == 0)[:, None]
        scales = np.where(tiny_row, rng.integers(3, 10, size=(gr, gc)),
                          rng.integers(124, 131, size=(gr, gc))).astype(np.uint8)
    elif kind == "large_scales":
        codes = inputs.FINITE_E4M3[rng.integers(0, 254, size=(rows, cols))]
        scales = rng.integers(238, 247, size=(gr, gc)).astype(np.uint8)
        xv *= np.float32(2.0 ** -40)  # |w x| <= 2^128 * 2^-37: every sum stays finite
    elif kind == "subnormal_x":
        codes = inputs.round_to_e4m3(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.05))
        scales = rng.integers(124, 131, size=(gr, gc)).astype(np.uint8)
        xv *= np.float32(2.0 ** -130)  # bf16 subnormals (some round to zero)
    else:
        raise ValueError(kind)
    x = inputs.round_to_bf16_bits(xv)
    if kind == "subnormal_x":
        mag = x & np.uint16(0x7FFF)
        assert np.mean((mag > 0) & (mag < 0x0080)) > 0.5  # mostly bf16 subnormal
    st, _fb, _grid = oracle.load_check(codes, scales)
    assert st == 0, kind
    return inputs.Linear(rows, cols, np.ascontiguousarray(codes), scales, x, seed, kind)


KINDS = ["tiny_scales", "scales_0_2", "subnormal_codes", "large_scales", "subnormal_x"]
# ragged rows and a ragged last window; 13 windows: the single matrix-core call splits rows into parts
SHAPE = (301, 1552)
M = 5


def _dev(L):
    from gpu_util import DevLinear
    D = DevLinear(L.codes, L.scales, L.x)
    assert D.check(check=False) == (0, -1)
    return D


def _y(M_, rows):
    from gpu_util import DEV
    return torch.full((M_, rows), float("nan"), dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("kind", KINDS)
def test_matrix_core_single_call_extreme(gpu, kind):
    from gpu_util import assert_within_tolerance, say, u32
    rows, cols = SHAPE
    L = _case(kind, rows, cols, M, 3100 + KINDS.index(kind))
    say(f"matrix-core single call, {kind}, {rows}x{cols} M={M}")
    D = _dev(L)
    slab = D.slab()
    y8, yt = _y(M, rows), _y(M, rows)
    fb.fp8blk_gemv_mfma(D.codes, D.grid, D.x, y8)
    fb.bf16_gemv_twin_mfma(slab, D.x, yt)
    torch.cuda.synchronize()
    a = y8.cpu().numpy()
    assert np.array_equal(u32(a), u32(yt)), f"{kind}: matrix-core FP8 arm and twin differ"
    y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=NTHREADS)
    assert np.all(yabs > 0) or kind == "subnormal_x"
    assert_within_tolerance(a, y64, yabs, what=f"matrix-core {kind}")
    for m in range(M):
        y1 = _y(1, rows)
        fb.fp8blk_gemv_mfma(D.codes, D.grid, D.x[m:m + 1].contiguous(), y1)
        torch.cuda.synchronize()
        assert np.array_equal(u32(y1)[0], u32(a)[m]), (kind, m)


@pytest.mark.parametrize("kind", KINDS)
def test_vector_arm_extreme(gpu, kind):
    from gpu_util import full_parity, say
    rows, cols = SHAPE
    L = _case(kind, rows, cols, M, 3200 + KINDS.index(kind))
    say(f"vector GEMV, {kind}, {rows}x{cols} M={M}")
    D = _dev(L)
    slab = D.slab()
    y8 = D.gemv().cpu().numpy()
    yt = D.twin(slab).cpu().numpy()
    full_parity(L, L.codes, L.scales, L.x, y8, yt, nthreads=NTHREADS, what=f"vector {kind}")


@pytest.mark.parametrize("Mp", [1, 5, 16])
def test_sequences_extreme(gpu, Mp):
    """All five cases as one list, for the matrix-core sequence (and its twin)
    and, at M = 1, the vector sequence (and its twin); against the single calls
    of their arm and the oracle."""
    from gpu_util import assert_within_tolerance, say, u32
    members = []
    for k, kind in enumerate(KINDS):
        rows, cols = (SHAPE if k % 2 == 0 else (260, 4096))
        L = _case(kind, rows, cols, Mp, 3300 + 7 * k + Mp)
        D = _dev(L)
        members.append((L, D, D.slab()))
    y8 = [_y(Mp, D.rows) for _, D, _ in members]
    yt = [_y(Mp, D.rows) for _, D, _ in members]
    s8 = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, D.x, y) for (_, D, _), y in zip(members, y8)])
    st = fb.fp8blk_sequence_init(fb.ARM_BF16_MFMA, [(s, D.x, y) for (_, D, s), y in zip(members, yt)])
    say(f"matrix-core sequence, extreme cases, M={Mp}")
    fb.fp8blk_gemv_mfma_sequence(s8)
    fb.bf16_gemv_twin_mfma_sequence(st)
    torch.cuda.synchronize()
    for (L, D, _), a, b in zip(members, y8, yt):
        av = a.cpu().numpy()
        assert np.array_equal(u32(av), u32(b)), (L.name, "matrix-core sequence FP8 != twin")
        y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=NTHREADS)
        assert_within_tolerance(av, y64, yabs, what=f"matrix-core sequence {L.name} M={Mp}")
    if Mp == 1:
        v8 = [_y(1, D.rows) for _, D, _ in members]
        vt = [_y(1, D.rows) for _, D, _ in members]
        q8 = fb.fp8blk_sequence_init(fb.ARM_FP8, [(D.codes, D.grid, D.x, y) for (_, D, _), y in zip(members, v8)])
        qt = fb.fp8blk_sequence_init(fb.ARM_BF16, [(s, D.x, y) for (_, D, s), y in zip(members, vt)])
        say("vector sequence, extreme cases, M=1")
        fb.fp8blk_gemv_sequence(q8)
        fb.bf16_gemv_twin_sequence(qt)
        torch.cuda.synchronize()
        for (L, D, _), a, b in zip(members, v8, vt):
            assert np.array_equal(u32(a), u32(D.gemv())), (L.name, "vector sequence != single call")
            assert np.array_equal(u32(a), u32(b)), (L.name, "vector sequence FP8 != twin")
