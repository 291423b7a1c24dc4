"""GPU: a sequence launch (one persistent kernel over a list of independent
M = 1 linears) gives every linear the same bits as a call of its own, for the
FP8 arm and the bf16 twin, over every plan shape: 1, 2 and 4 rows per step
(1, 2 and 3-4 segments), rows and columns past the last full step, and rows
of more than 4 segments walked over several steps."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu

# (rows, cols): one segment (4 rows per step, also fewer columns than a
# segment), two (2 rows per step), three and four (one row), more than four
# (several steps per row, a partial last step), ragged rows everywhere.
SHAPES = [(256, 512), (13, 1024), (130, 16), (257, 2048), (3, 1040), (129, 2064), (64, 3072), (300, 4096),
          (77, 4112), (40, 8192), (33, 16400), (5, 65536), (1, 16)]


def _members(shapes, seed0):
    from gpu_util import DevLinear, DEV
    out = []
    for k, (rows, cols) in enumerate(shapes):
        L = inputs.host_linear(rows, cols, 1, seed0 + 7 * k)
        D = DevLinear(L.codes, L.scales, L.x)
        assert D.check(check=False) == (0, -1)
        out.append((L, D, D.slab()))
    return out


def _run_sequence(members):
    from gpu_util import DEV
    y8 = [torch.full((1, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    yt = [torch.full((1, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    s8 = fb.fp8blk_sequence_init(fb.ARM_FP8, [(D.codes, D.grid, D.x, y) for (_, D, _), y in zip(members, y8)])
    st = fb.fp8blk_sequence_init(fb.ARM_BF16, [(s, D.x, y) for (_, D, s), y in zip(members, yt)])
    fb.fp8blk_gemv_sequence(s8)
    fb.bf16_gemv_twin_sequence(st)
    torch.cuda.synchronize()
    return s8, st, y8, yt


def test_sequence_equals_separate_calls(gpu):
    from gpu_util import say, u32
    members = _members(SHAPES, 500)
    _, _, y8, yt = _run_sequence(members)
    for (L, D, slab), a, b in zip(members, y8, yt):
        say(f"  {D.rows}x{D.cols}")
        ref = D.gemv()
        assert np.array_equal(u32(a), u32(ref)), (D.rows, D.cols)
        assert np.array_equal(u32(b), u32(ref)), (D.rows, D.cols)


def test_sequence_matches_oracle(gpu):
    """Against the oracle directly: the documented order bitwise (O7) and the
    double GEMV within 1e-5 * sum|w x| (O6)."""
    from gpu_util import assert_within_tolerance, u32
    members = _members([(256, 512), (257, 2048), (129, 2064), (33, 16400), (300, 4096)], 900)
    _, _, y8, yt = _run_sequence(members)
    for (L, D, _), a, b in zip(members, y8, yt):
        ya = a.cpu().numpy()
        assert np.array_equal(u32(ya), u32(b))
        y7 = oracle.gemv_f32_order(L.x, codes=L.codes, scales=L.scales, nthreads=8)
        assert np.array_equal(u32(ya), y7.view(np.uint32)), (D.rows, D.cols)
        y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=8)
        assert_within_tolerance(ya, y64, yabs, what=f"{D.rows}x{D.cols}")


def test_sequence_relaunch_and_single_member(gpu):
    """The plan keeps pointers, not values: a second launch after x changes
    gives the new result; a launch is deterministic; a list of one works, and
    a list with fewer units than the grid's waves leaves the idle waves out."""
    from gpu_util import DEV, u32
    members = _members([(5, 4096), (2, 1024)], 77)
    s8, _, y8, _ = _run_sequence(members)
    first = [y.clone() for y in y8]
    fb.fp8blk_gemv_sequence(s8)
    torch.cuda.synchronize()
    for a, b in zip(first, y8):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    for _, D, _ in members:
        D.x.copy_(torch.flip(D.x, dims=[1]))
    fb.fp8blk_gemv_sequence(s8)
    torch.cuda.synchronize()
    for (_, D, _), y in zip(members, y8):
        assert np.array_equal(u32(y), u32(D.gemv()))
    one = _members([(1, 16)], 3)
    _, _, y1, t1 = _run_sequence(one)
    assert np.array_equal(u32(y1[0]), u32(one[0][1].gemv()))
    assert np.array_equal(u32(t1[0]), u32(y1[0]))


def test_sequence_whole_step_sweep(gpu):
    """The benchmark's launch: the 259 linears of the whole-step sweep in one
    sequence. Every output equals the per-linear call bitwise (on the GPU);
    128-row windows of a few linears are checked against the oracle."""
    from gpu_util import DEV, DevLinear, assert_within_tolerance, say, u32
    sw = inputs.sweep_plan()
    xs = {c: inputs.device_x(c, 1, 7 + c, DEV) for c in {l.cols for l in sw.linears}}
    lins, ys = [], []
    for spec in sw.linears:
        codes, scales = inputs.device_linear(spec.rows, spec.cols, spec.seed, DEV)
        D = DevLinear(codes, scales, xs[spec.cols])
        assert D.check(check=False) == (0, -1), spec.name
        lins.append((spec, D))
        ys.append(torch.full((1, spec.rows), float("nan"), device=DEV))
    seq = fb.fp8blk_sequence_init(fb.ARM_FP8, [(D.codes, D.grid, D.x, y) for (_, D), y in zip(lins, ys)])
    fb.fp8blk_gemv_sequence(seq)
    torch.cuda.synchronize()
    say("  sweep sequence launched")
    for i, ((spec, D), y) in enumerate(zip(lins, ys)):
        ref = D.gemv()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), (i, spec.name)
        if i in (0, 1, 2, 3, 4, 5, len(lins) - 1):
            r0 = 128 * (spec.rows // 256)
            ch = D.codes[r0:r0 + 128].cpu().numpy()
            sh = D.scales[r0 // 128:r0 // 128 + 1].cpu().numpy()
            xh = D.x.cpu().numpy().view(np.uint16)
            yw = y[:, r0:r0 + 128].cpu().numpy()
            y7 = oracle.gemv_f32_order(xh, codes=ch, scales=sh, nthreads=8)
            assert np.array_equal(u32(yw), y7.view(np.uint32)), (spec.name, r0)
            y64, yabs = oracle.gemv_f64(ch, sh, xh, nthreads=8)
            assert_within_tolerance(yw, y64, yabs, what=f"{spec.name} rows {r0}..")
    say(f"  {len(lins)} sweep linears equal their single calls")


def test_sequence_graph_replays(gpu):
    """A sequence launch captured in a HIP graph: every replay, with eager work
    and synchronizations between the replays, gives the eager bits (vector and
    matrix-core arms)."""
    from gpu_util import DEV, u32
    members = _members([(300, 4096), (257, 2048), (13, 1024), (77, 4112)], 31)
    y_eager = [torch.full((1, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    y_graph = [torch.full((1, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    s_e = fb.fp8blk_sequence_init(fb.ARM_FP8, [(D.codes, D.grid, D.x, y) for (_, D, _), y in zip(members, y_eager)])
    s_g = fb.fp8blk_sequence_init(fb.ARM_FP8, [(D.codes, D.grid, D.x, y) for (_, D, _), y in zip(members, y_graph)])
    x16 = [torch.from_numpy(inputs.host_linear(D.rows, D.cols, 16, 9 + k).x.view(np.int16)).to(DEV)
           for k, (_, D, _) in enumerate(members)]
    m_e = [torch.full((16, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    m_g = [torch.full((16, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    sm_e = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, x, y) for (_, D, _), x, y in
                                                     zip(members, x16, m_e)])
    sm_g = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, x, y) for (_, D, _), x, y in
                                                     zip(members, x16, m_g)])
    call_v = fb.prepared("fp8blk_gemv_sequence", s_g)
    call_m = fb.prepared("fp8blk_gemv_mfma_sequence", sm_g)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        call_v2 = fb.prepared("fp8blk_gemv_sequence", s_g, stream=cap)
        call_m2 = fb.prepared("fp8blk_gemv_mfma_sequence", sm_g, stream=cap)
        assert call_v2() == 0 and call_m2() == 0
    torch.cuda.synchronize()
    for rep in range(4):
        for y in y_graph + m_g:
            y.fill_(float("nan"))
        # eager work between replays: change x, run the eager sequences
        for _, D, _ in members:
            D.x.copy_(torch.roll(D.x, shifts=rep + 1, dims=1))
        for x in x16:
            x.copy_(torch.roll(x, shifts=1, dims=0))
        fb.fp8blk_gemv_sequence(s_e)
        fb.fp8blk_gemv_mfma_sequence(sm_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(y_eager + m_e, y_graph + m_g):
            assert np.array_equal(u32(a), u32(b)), rep
    assert call_v() == 0 and call_m() == 0


def test_sequence_many_small_linears(gpu):
    """600 small linears of mixed shapes (most of them ragged, so both launches
    run; a wave's next unit often lies several linears ahead): every output
    equals its single call, on both vector arms and the matrix-core arm."""
    from gpu_util import DEV, DevLinear, u32
    rng = np.random.default_rng(17)
    cols_choices = [16, 48, 512, 1024, 1040, 2048, 3072, 4096]
    members = []
    for k in range(600):
        rows = int(rng.integers(1, 40))
        cols = int(cols_choices[rng.integers(0, len(cols_choices))])
        L = inputs.host_linear(rows, cols, 4, 1000 + k)
        D = DevLinear(L.codes, L.scales, L.x)
        assert D.check(check=False) == (0, -1)
        members.append((L, D, D.slab()))
    x1 = [D.x[:1].contiguous() for _, D, _ in members]
    y8 = [torch.full((1, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    yt = [torch.full((1, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    ym = [torch.full((4, D.rows), float("nan"), device=DEV) for _, D, _ in members]
    s8 = fb.fp8blk_sequence_init(fb.ARM_FP8, [(D.codes, D.grid, x, y) for (_, D, _), x, y in zip(members, x1, y8)])
    st = fb.fp8blk_sequence_init(fb.ARM_BF16, [(s, x, y) for (_, D, s), x, y in zip(members, x1, yt)])
    sm = fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(D.codes, D.grid, D.x, y) for (_, D, _), y in zip(members, ym)])
    assert s8.handle.units_general > 0 and s8.handle.units_dense > 0
    fb.fp8blk_gemv_sequence(s8)
    fb.bf16_gemv_twin_sequence(st)
    fb.fp8blk_gemv_mfma_sequence(sm)
    torch.cuda.synchronize()
    from gpu_util import assert_within_tolerance
    for (L, D, _), x, a, b, m in zip(members, x1, y8, yt, ym):
        ref = D.gemv(x)
        assert np.array_equal(u32(a), u32(ref)), (D.rows, D.cols)
        assert np.array_equal(u32(b), u32(ref)), (D.rows, D.cols)
        # the matrix-core sequence: its own order; within the tolerance of the
        # double GEMV, and the single matrix-core call's bits where that call
        # takes each row in one part (at most 7 column windows)
        mh = m.cpu().numpy()
        y64, yabs = oracle.gemv_f64(L.codes, L.scales, L.x, nthreads=8)
        assert_within_tolerance(mh, y64, yabs, what=f"mfma sequence {D.rows}x{D.cols}")
        if D.cols <= 896:
            one = torch.full_like(m, float("nan"))
            fb.fp8blk_gemv_mfma(D.codes, D.grid, D.x, one)
            assert np.array_equal(u32(mh), u32(one)), (D.rows, D.cols)
