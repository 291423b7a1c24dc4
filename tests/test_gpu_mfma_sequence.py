"""GPU: the matrix-core sequence launch (fp8blk_gemv_mfma_sequence and its
bf16 twin) over lists of independent linears with an M-row panel.

There is no bitwise oracle for the matrix core's internal order. What is
checked: the FP8 arm and its bf16 twin give identical bits; row m of an M-row
sequence equals the 1-row sequence on x[m], bit for bit; a list member whose
single matrix-core call takes its row in one part gives that call's bits;
inputs on which every summation order is exact give the exact result; and
every output is within 1e-5 * sum|w x| of the double GEMV (O6), also at the
whole-step sweep's full size with a 16-row panel."""
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)

# ragged rows and cols, one to many windows, partial last window
SHAPES = [(256, 512), (13, 1024), (130, 16), (257, 2048), (3, 1040), (129, 2064), (64, 3072), (300, 4096),
          (77, 4112), (40, 8192), (33, 16400), (5, 65536), (1, 16)]


def _members(shapes, M, seed0):
    from gpu_util import DevLinear
    out = []
    for k, (rows, cols) in enumerate(shapes):
        L = inputs.host_linear(rows, cols, M, seed0 + 13 * k)
        D = DevLinear(L.codes, L.scales, L.x)
        assert D.check(check=False) == (0, -1)
        out.append((L, D, D.slab()))
    return out


def _run(members, x_of=lambda D: D.x):
    from gpu_util import DEV
    y8, yt = [], []
    for _, D, _ in members:
        M = x_of(D).shape[0]
        y8.append(torch.full((M, D.rows), float("nan"), device=DEV))
        yt.append(torch.full((M, D.rows), float("nan"), device=DEV))
    s8 = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, x_of(D), y)
                                                   for (_, D, _), y in zip(members, y8)])
    st = fb.fp8blk_sequence_init(fb.ARM_BF16_MFMA, [(s, x_of(D), y) for (_, D, s), y in zip(members, yt)])
    fb.fp8blk_gemv_mfma_sequence(s8)
    fb.bf16_gemv_twin_mfma_sequence(st)
    torch.cuda.synchronize()
    return y8, yt


@pytest.mark.parametrize("M", [1, 2, 5, 16])
def test_mfma_sequence_twin_and_tolerance(gpu, M):
    from gpu_util import assert_within_tolerance, say, u32
    members = _members(SHAPES, M, 300 + M)
    y8, yt = _run(members)
    for (L, D, _), a, b in zip(members, y8, yt):
        say(f"  mfma sequence {D.rows}x{D.cols} M={M}")
        ya = a.cpu().numpy()
        assert np.array_equal(u32(ya), u32(b)), (D.rows, D.cols, "FP8 != twin")
        y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=NTHREADS)
        assert_within_tolerance(ya, y64, yabs, what=f"mfma sequence {D.rows}x{D.cols} M={M}")


def test_mfma_sequence_batch_invariance(gpu):
    from gpu_util import u32
    members = _members([(300, 4096), (77, 4112), (257, 2048)], 16, 41)
    singles = [_run(members, x_of=lambda D, m=m: D.x[m:m + 1].contiguous())[0] for m in range(16)]
    for M in (2, 3, 8, 16):
        y8, yt = _run(members, x_of=lambda D, M=M: D.x[:M].contiguous())
        for i in range(len(members)):
            for m in range(M):
                assert np.array_equal(u32(y8[i][m]), u32(singles[m][i][0])), (M, i, m)
                assert np.array_equal(u32(yt[i][m]), u32(singles[m][i][0])), (M, i, m)


def test_mfma_sequence_matches_single_call_in_one_part(gpu):
    """Linears with at most 7 column windows: the single matrix-core call takes
    every row in one part, the sequence's order, so the bits agree."""
    from gpu_util import DEV, u32
    members = _members([(256, 512), (100, 896), (33, 16), (1000, 128)], 16, 5)
    y8, _ = _run(members)
    for (_, D, _), a in zip(members, y8):
        ref = torch.full_like(a, float("nan"))
        fb.fp8blk_gemv_mfma(D.codes, D.grid, D.x, ref)
        torch.cuda.synchronize()
        assert np.array_equal(u32(a), u32(ref)), (D.rows, D.cols)


def test_mfma_sequence_integer_exact(gpu):
    from gpu_util import DevLinear, DEV
    from test_gpu_gemv import _integer_case
    cases = [_integer_case(260, 3088, 16, 9), _integer_case(70, 4096, 16, 10)]
    Ds, ys = [], []
    for codes, scales, x, exact, W in cases:
        D = DevLinear(codes, scales, x)
        D.check()
        Ds.append(D)
        ys.append(torch.full((16, D.rows), float("nan"), device=DEV))
    seq = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, D.x, y) for D, y in zip(Ds, ys)])
    fb.fp8blk_gemv_mfma_sequence(seq)
    torch.cuda.synchronize()
    for (codes, scales, x, exact, W), y in zip(cases, ys):
        assert np.array_equal(y.cpu().numpy().astype(np.float64), exact)


def test_mfma_sequence_whole_step_sweep(gpu):
    """The 259 linears of the whole-step sweep with a 16-row verify panel in one
    matrix-core sequence: every output of every linear against the oracle's
    double GEMV (1e-5 * sum|w x|), and the FP8 arm against the twin on the
    first layer and the head."""
    from gpu_util import DEV, DevLinear, assert_within_tolerance, say, u32
    sw = inputs.sweep_plan()
    xs = {c: inputs.device_x(c, 16, 7 + c, DEV) for c in {l.cols for l in sw.linears}}
    lins, ys = [], []
    for spec in sw.linears:
        codes, scales = inputs.device_linear(spec.rows, spec.cols, spec.seed, DEV)
        D = DevLinear(codes, scales, xs[spec.cols])
        assert D.check(check=False) == (0, -1), spec.name
        lins.append((spec, D))
        ys.append(torch.full((16, spec.rows), float("nan"), device=DEV))
    seq = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, D.x, y) for (_, D), y in zip(lins, ys)])
    fb.fp8blk_gemv_mfma_sequence(seq)
    torch.cuda.synchronize()
    say("  mfma sweep sequence launched")
    twin_idx = [0, 1, 2, 3, 4, 5, len(lins) - 1]
    slabs = {i: lins[i][1].slab() for i in twin_idx}
    yt = {i: torch.full_like(ys[i], float("nan")) for i in twin_idx}
    st = fb.fp8blk_sequence_init(fb.ARM_BF16_MFMA, [(slabs[i], lins[i][1].x, yt[i]) for i in twin_idx])
    fb.bf16_gemv_twin_mfma_sequence(st)
    torch.cuda.synchronize()
    for i in twin_idx:
        assert torch.equal(ys[i].view(torch.int32), yt[i].view(torch.int32)), lins[i][0].name
    for i, (spec, D) in enumerate(lins):
        ch, sh = D.codes.cpu().numpy(), D.scales.cpu().numpy()
        xh = D.x.cpu().numpy().view(np.uint16)
        y64, yabs = oracle.gemv_f64(ch, sh, xh, nthreads=NTHREADS)
        assert_within_tolerance(ys[i].cpu().numpy(), y64, yabs, what=f"{spec.name} M=16")
        if i % 43 == 0 or spec.name == "head":
            say(f"  sweep linear {i} {spec.name}: every output within tolerance")
    assert all(not torch.isnan(y).any() for y in ys)
    say(f"  {len(lins)} sweep linears at M=16 checked")
    # The decode / verify pairing of this arm ("Struct Dsv4Gpu" page,
    # spec_greedy_batched_with): row m of the 16-row verify sweep equals the
    # one-row sweep on x[m], bit for bit, for every output of every linear.
    for m in range(16):
        y1 = [torch.full((1, spec.rows), float("nan"), device=DEV) for spec, _ in lins]
        s1 = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, D.x[m:m + 1], y)
                                                       for (_, D), y in zip(lins, y1)])
        fb.fp8blk_gemv_mfma_sequence(s1)
        torch.cuda.synchronize()
        bad = [lins[i][0].name for i in range(len(lins))
               if not torch.equal(ys[i][m].view(torch.int32), y1[i][0].view(torch.int32))]
        assert not bad, (m, bad[:5])
    say("  M=16 sweep rows == M=1 sweeps on each x[m], bit for bit")


@pytest.mark.parametrize("M", [2, 5, 8, 11, 16])
def test_mfma_sequence_more_units_than_held(gpu, M):
    """A list long enough that every wave finishes more units than its LDS part
    and its registers hold (about 14 units per wave with 1.8M rows of 128
    columns): the outputs kept back to the end of the launch, the ones parked in
    registers and the ones written when they finish all equal the single
    matrix-core call (one part at these cols), and the twin, bit for bit.
    Below 8 rows nothing is held, and the FP8 arm runs three workgroups per
    compute unit against the twin's two: the two arms deal the same units to
    different waves, and their bits must still agree."""
    from gpu_util import DEV, DevLinear, assert_within_tolerance, say, u32
    shapes = [(900000, 128), (5000, 256), (900001, 128)]
    members, y8, yt, slabs = [], [], [], []
    for k, (rows, cols) in enumerate(shapes):
        codes, scales = inputs.device_linear(rows, cols, 900 + k, DEV)
        D = DevLinear(codes, scales, inputs.device_x(cols, M, 950 + k, DEV))
        assert D.check(check=False) == (0, -1)
        members.append(D)
        slabs.append(D.slab())
        y8.append(torch.full((M, rows), float("nan"), device=DEV))
        yt.append(torch.full((M, rows), float("nan"), device=DEV))
    s8 = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, D.x, y) for D, y in zip(members, y8)])
    st = fb.fp8blk_sequence_init(fb.ARM_BF16_MFMA, [(s, D.x, y) for D, s, y in zip(members, slabs, yt)])
    say(f"  long mfma sequence M={M}: {s8.handle.units_dense} units over {s8.handle.grid_dense * 4} waves")
    fb.fp8blk_gemv_mfma_sequence(s8)
    fb.bf16_gemv_twin_mfma_sequence(st)
    torch.cuda.synchronize()
    for D, a, b in zip(members, y8, yt):
        ref = torch.full_like(a, float("nan"))
        fb.fp8blk_gemv_mfma(D.codes, D.grid, D.x, ref)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), ref.view(torch.int32)), (D.rows, D.cols, "sequence != single call")
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (D.rows, D.cols, "FP8 != twin")
        r0 = 128 * ((D.rows - 200) // 128)  # the last rows, from a scale-block boundary
        ch = D.codes[r0:].cpu().numpy()
        sh = D.scales[r0 // 128:].cpu().numpy()
        y64, yabs = oracle.gemv_f64(ch, sh, D.x.cpu().numpy().view(np.uint16), nthreads=NTHREADS)
        assert_within_tolerance(a[:, r0:].cpu().numpy(), y64, yabs, what=f"{D.rows}x{D.cols} tail M={M}")
