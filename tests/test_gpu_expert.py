"""GPU parity of the native expert arm against the oracle
(oracle/fp4_expert_oracle.c): act_quant, the FP4 load check and bf16 slab
are bit-exact; the native GEMV is within 1e-5 * |g| * sum|q w| of the exact
sum (and exact where every partial sum is representable); the sequence
launch equals the single call bitwise; the bf16-dequant arm composes with the
bf16 twin GEMV in the documented order.

Source passages: "Module dsv4_gpu" page, enums ExpertArm, ExpertKind and
DecodePath, and the rungs paragraph."""
import os

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8_fp8blk_amd import inputs as I

pytestmark = pytest.mark.gpu

MX, NV = I.MXFP4, I.NVFP4
NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def gu(gpu):
    import gpu_util
    return gpu_util


def dev(gu, a):
    return gu.to_dev(a)


def act_quant_gpu(gpu, x_dev):
    M, cols = x_dev.shape
    xq = torch.full((M, cols), 0x7F, dtype=torch.uint8, device=x_dev.device)
    xs = torch.full((M, -(-cols // 128)), 0xFF, dtype=torch.uint8, device=x_dev.device)
    gpu.fp8blk_act_quant(x_dev, xq, xs)
    return xq, xs


def expert_gemv_gpu(gpu, fmt, codes, scales, g, xq, xs, rows):
    y = torch.full((xq.shape[0], rows), float("nan"), dtype=torch.float32, device=codes.device)
    gpu.fp4_expert_gemv(fmt, codes, scales, g, xq, xs, y)
    return y


def bf16_bits(v):
    return I.round_to_bf16_bits(np.asarray(v, dtype=np.float32))


# --- act_quant ----------------------------------------------------------------

def test_act_quant_every_bf16_value(gpu, gu):
    """Every finite bf16 pattern of magnitude <= 448 (both signs), in blocks
    whose amax is 448, then the same patterns scaled so that every block gets
    another scale; bit-exact codes and scales."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pos << 16).view(np.float32)
    pos = pos[vals <= 448.0]
    pats = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    per = 127
    nblk = -(-pats.size // per)
    x = np.zeros((nblk, 128), dtype=np.uint16)
    x[:, 0] = bf16_bits([448.0])[0]
    flat = np.zeros(nblk * per, dtype=np.uint16)
    flat[:pats.size] = pats
    x[:, 1:] = flat.reshape(nblk, per)
    x = x.reshape(1, -1)
    gu.say(f"act_quant exhaustive: cols {x.shape[1]}")
    xq, xs = act_quant_gpu(gpu, dev(gu, x))
    cq, cs = oracle.act_quant(x)
    assert np.array_equal(xs.cpu().numpy(), cs)
    assert np.array_equal(xq.cpu().numpy(), cq)


@pytest.mark.parametrize("seed,mag,M,cols", [(1, 1.0, 1, 4096), (2, 1e-30, 3, 2048), (3, 1e30, 16, 4096),
                                             (4, 1e-38, 5, 512), (5, 1.0, 16, 208), (6, 3.0e38, 2, 144)])
def test_act_quant_random(gpu, gu, seed, mag, M, cols):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((M, cols)) * mag
    v *= 10.0 ** rng.integers(-8, 8, size=(M, cols)) if seed % 2 else 1.0
    if cols >= 256:
        v[0, 128:256] = 0.0
    v = np.clip(v, -3.0e38, 3.0e38)
    x = bf16_bits(v)
    gu.say(f"act_quant seed {seed} M {M} cols {cols}")
    xq, xs = act_quant_gpu(gpu, dev(gu, x))
    cq, cs = oracle.act_quant(x)
    assert np.array_equal(xs.cpu().numpy(), cs)
    assert np.array_equal(xq.cpu().numpy(), cq)


# --- load check and the bf16 slab -----------------------------------------------

def check_gpu(gpu, gu, fmt, codes, scales):
    ws = torch.empty(256, dtype=torch.uint8, device=gu.DEV)
    return gpu.fp4_load_check(fmt, dev(gu, codes), dev(gu, scales), ws, check=False)


@pytest.mark.parametrize("fmt", [MX, NV])
def test_load_check_matches_oracle(gpu, gu, fmt):
    rows, cols = 300, 512
    L = I.host_fp4_linear(fmt, rows, cols, 1, 40 + fmt)
    gu.say(f"fp4 load check fmt {fmt}")
    assert check_gpu(gpu, gu, fmt, L.codes, L.scales) == oracle.fp4_load_check(fmt, L.codes, L.scales) == (0, -1)
    rng = np.random.default_rng(9)
    for trial in range(6):
        sc = L.scales.copy()
        codes = L.codes.copy()
        for _ in range(3):
            r, b = rng.integers(0, rows), rng.integers(0, sc.shape[1])
            if fmt == MX:
                sc[r, b] = rng.choice([0xFF, 253, 254])
                codes[r, (b * 32) // 2:(b * 32 + 32) // 2] = rng.integers(0, 256, 16)
            else:
                sc[r, b] = rng.choice([0x7F, 0xFF, 0x80, 0x9A])
        want = oracle.fp4_load_check(fmt, codes, sc)
        got = check_gpu(gpu, gu, fmt, codes, sc)
        assert got == want, (trial, got, want)


@pytest.mark.parametrize("fmt,lo,hi", [(MX, 0, 252), (NV, 0x00, 0x7E)])
def test_dequant_bf16_bit_exact(gpu, gu, fmt, lo, hi):
    """Every code byte with scales over the whole accepted range."""
    L = I.host_fp4_linear(fmt, 1024, 1024, 1, 60 + fmt, scale_lo=lo, scale_hi=hi)
    if fmt == MX:  # 253 and 254 are accepted only with small codes: keep them out
        assert oracle.fp4_load_check(fmt, L.codes, L.scales)[0] == oracle.OK
    gu.say(f"fp4 dequant fmt {fmt}")
    out = torch.empty((1024, 1024), dtype=torch.int16, device=gu.DEV)
    gpu.fp4_dequant_bf16(fmt, dev(gu, L.codes), dev(gu, L.scales), out)
    want = oracle.fp4_dequant_bf16(fmt, L.codes, L.scales)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


def test_dequant_arm_composes_with_the_bf16_twin(gpu, gu):
    """The bf16-dequant arm: the slab, then bf16_gemv_twin with the bf16
    activation, equals the documented-order GEMV over the oracle's slab."""
    L = I.host_fp4_linear(NV, 2048, 4096, 1, 70)
    gu.say("dequant arm 2048x4096")
    slab = torch.empty((L.rows, L.cols), dtype=torch.int16, device=gu.DEV)
    gpu.fp4_dequant_bf16(NV, dev(gu, L.codes), dev(gu, L.scales), slab)
    y = torch.empty((1, L.rows), dtype=torch.float32, device=gu.DEV)
    gpu.bf16_gemv_twin(slab, dev(gu, L.x), y)
    want = oracle.gemv_f32_order(L.x, w_bf16=oracle.fp4_dequant_bf16(NV, L.codes, L.scales))
    assert np.array_equal(gu.u32(y), gu.u32(want))


# --- the native GEMV --------------------------------------------------------------

def native_parity(gpu, gu, L, M=None, what=""):
    x = L.x if M is None else L.x[:M]
    xq_d, xs_d = act_quant_gpu(gpu, dev(gu, x))
    xq, xs = oracle.act_quant(x)
    assert np.array_equal(xq_d.cpu().numpy(), xq) and np.array_equal(xs_d.cpu().numpy(), xs)
    gu.say(f"native gemv {what}: fmt {L.fmt} rows {L.rows} cols {L.cols} M {x.shape[0]}")
    y = expert_gemv_gpu(gpu, L.fmt, dev(gu, L.codes), dev(gu, L.scales), L.global_scale, xq_d, xs_d, L.rows)
    y64, yabs = oracle.fp4_gemv_f64(L.fmt, L.codes, L.scales, xq, xs, L.global_scale)
    gu.assert_within_tolerance(y.cpu().numpy(), y64, yabs, what=what)
    return y


@pytest.mark.parametrize("fmt", [MX, NV])
@pytest.mark.parametrize("rows,cols,M", [(256, 512, 1), (1000, 384, 3), (17, 128, 16), (64, 1152, 2),
                                         (200, 640, 5), (48, 256, 9), (2048, 4096, 1), (4096, 2048, 1),
                                         # one activation row (its own load layout): a window shorter than 4
                                         # steps, ragged rows and a last partial window
                                         (17, 128, 1), (1000, 384, 1), (45, 1152, 1), (100, 2176, 1)])
def test_native_gemv_parity(gpu, gu, fmt, rows, cols, M):
    L = I.host_fp4_linear(fmt, rows, cols, M, 1000 + rows + cols + M)
    native_parity(gpu, gu, L, what=f"{rows}x{cols}")


@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("fmt,lo,hi", [(MX, 0, 6), (MX, 230, 238), (NV, 0x01, 0x0F), (NV, 0x70, 0x7E)])
def test_native_gemv_extreme_scales(gpu, gu, fmt, lo, hi, M):
    """Block scales near the ends of the range the load check accepts: MXFP4
    codes 0..6 (2^-127..2^-121, code 0 included) and 230..238, NVFP4 e4m3
    subnormal and largest scales. (Larger MXFP4 codes are accepted too, but
    their outputs over 1024 columns can pass f32's largest value, where f32
    accumulation ends in infinity whatever the order.)"""
    L = I.host_fp4_linear(fmt, 256, 1024, M, 1500 + lo, scale_lo=lo, scale_hi=hi)
    ws = torch.empty(256, dtype=torch.uint8, device=gu.DEV)
    assert gpu.fp4_load_check(fmt, dev(gu, L.codes), dev(gu, L.scales), ws, check=False) == (0, -1)
    native_parity(gpu, gu, L, what=f"scales {lo}..{hi}")


@pytest.mark.parametrize("fmt", [MX, NV])
def test_native_gemv_integer_exact(gpu, gu, fmt):
    """Unit scales and activation codes of magnitude <= 8: every partial sum
    is a multiple of 1/4 below 2^21, exact in f32 in any order, so the GPU
    equals the exact sum bit for bit."""
    rows, cols, M = 300, 4096, 4
    L = I.host_fp4_linear(fmt, rows, cols, M, 90 + fmt)
    scales = np.full_like(L.scales, 127 if fmt == MX else 0x38)  # 1.0
    rng = np.random.default_rng(91)
    xv = rng.integers(-16, 17, size=(M, cols)).astype(np.float32) / 2.0  # |x| <= 8, steps of 1/2
    xv[:, 0] = 448.0  # every block's amax 448 -> act scale 1
    xv[:, 128::128] = 448.0
    x = bf16_bits(xv)
    xq, xs = oracle.act_quant(x)
    assert np.all(xs == 127)
    y = expert_gemv_gpu(gpu, fmt, dev(gu, L.codes), dev(gu, scales), 1.0, dev(gu, xq), dev(gu, xs), rows)
    y64, _ = oracle.fp4_gemv_f64(fmt, L.codes, scales, xq, xs, 1.0)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y64)


@pytest.mark.parametrize("fmt", [MX, NV])
def test_native_gemv_batch_invariance(gpu, gu, fmt):
    """Row m of an M-row call equals the 1-row call on row m, bit for bit."""
    L = I.host_fp4_linear(fmt, 700, 2048, 16, 95 + fmt)
    xq, xs = act_quant_gpu(gpu, dev(gu, L.x))
    c, s = dev(gu, L.codes), dev(gu, L.scales)
    gu.say(f"batch invariance fmt {fmt}")
    full = expert_gemv_gpu(gpu, fmt, c, s, L.global_scale, xq, xs, L.rows)
    for M in (1, 2, 3, 4, 7, 8, 11, 16):
        part = expert_gemv_gpu(gpu, fmt, c, s, L.global_scale, xq[:M].contiguous(), xs[:M].contiguous(), L.rows)
        assert torch.equal(part.view(torch.int32), full[:M].view(torch.int32)), M
    for m in (0, 5, 15):
        one = expert_gemv_gpu(gpu, fmt, c, s, L.global_scale, xq[m:m + 1].contiguous(), xs[m:m + 1].contiguous(),
                              L.rows)
        assert torch.equal(one.view(torch.int32), full[m:m + 1].view(torch.int32)), m


@pytest.mark.parametrize("fmt,M", [(MX, 1), (NV, 1), (MX, 4), (NV, 4), (NV, 16)])
def test_sequence_equals_single_calls(gpu, gu, fmt, M):
    """One launch over mixed expert linears (gate, up, down shapes, ragged
    rows, short reductions) equals the single calls bit for bit; every output
    is checked against the oracle."""
    shapes = [(2048, 4096), (2048, 4096), (4096, 2048), (300, 512), (17, 128), (1000, 384)]
    lins, ins = [], []
    for k, (r, c) in enumerate(shapes):
        L = I.host_fp4_linear(fmt, r, c, M, 300 + 10 * k + fmt)
        xq_d, xs_d = act_quant_gpu(gpu, dev(gu, L.x))
        y = torch.full((M, r), float("nan"), dtype=torch.float32, device=gu.DEV)
        ins.append((L, dev(gu, L.codes), dev(gu, L.scales), xq_d, xs_d, y))
        lins.append((ins[-1][1], ins[-1][2], L.global_scale, xq_d, xs_d, y))
    gu.say(f"expert sequence fmt {fmt} M {M}: {len(lins)} linears")
    seq = gpu.fp4_expert_sequence_init(fmt, lins)
    assert seq.handle.arm == (gpu.ARM_MXFP4 if fmt == MX else gpu.ARM_NVFP4)
    gpu.fp4_expert_sequence(seq)
    torch.cuda.synchronize()
    for L, c, s, xq_d, xs_d, y in ins:
        single = expert_gemv_gpu(gpu, fmt, c, s, L.global_scale, xq_d, xs_d, L.rows)
        assert torch.equal(y.view(torch.int32), single.view(torch.int32)), (L.rows, L.cols)
        xq, xs = oracle.act_quant(L.x)
        y64, yabs = oracle.fp4_gemv_f64(fmt, L.codes, L.scales, xq, xs, L.global_scale)
        gu.assert_within_tolerance(y.cpu().numpy(), y64, yabs, what=f"sequence {L.rows}x{L.cols}")
    # a second launch of the same plan gives the same bits
    first = [t[-1].clone() for t in ins]
    gpu.fp4_expert_sequence(seq)
    torch.cuda.synchronize()
    for a, t in zip(first, ins):
        assert torch.equal(a.view(torch.int32), t[-1].view(torch.int32))


@pytest.mark.parametrize("fmt,M", [(MX, 1), (NV, 1), (NV, 12)])
def test_sequence_many_units_per_wave(gpu, gu, fmt, M):
    """Far more units than the persistent kernel has waves (each wave walks
    several units of different linears, carrying its addressing across unit
    and register-set boundaries), with reductions of 1 to 5 pipeline windows
    and ragged rows: every output equals its single call bit for bit; a sample
    is checked against the oracle."""
    rng = np.random.default_rng(500 + fmt + M)
    rows_choices, cols_choices = (45, 48, 100, 2048, 4096), (384, 640, 1152, 2176, 4096)
    lins, ins = [], []
    acts = {}
    for k in range(360):
        r, c = int(rng.choice(rows_choices)), int(rng.choice(cols_choices))
        if c not in acts:
            x = I.host_fp4_linear(fmt, 1, c, M, 700 + c).x
            xq_d, xs_d = act_quant_gpu(gpu, dev(gu, x))
            acts[c] = (x, xq_d, xs_d)
        codes, scales = I.device_fp4_linear(fmt, r, c, 800 + k, gu.DEV)
        y = torch.full((M, r), float("nan"), dtype=torch.float32, device=gu.DEV)
        ins.append((r, c, codes, scales, y))
        lins.append((codes, scales, 0.75, acts[c][1], acts[c][2], y))
    seq = gpu.fp4_expert_sequence_init(fmt, lins)
    units, waves = seq.handle.units_dense, 4 * seq.handle.grid_dense
    gu.say(f"expert sequence fmt {fmt} M {M}: {len(lins)} linears, {units} units, {waves} waves")
    assert units >= sum(-(-r // 32) for r, *_ in ins) and units > 4 * waves
    gpu.fp4_expert_sequence(seq)
    torch.cuda.synchronize()
    for k, (r, c, codes, scales, y) in enumerate(ins):
        single = expert_gemv_gpu(gpu, fmt, codes, scales, 0.75, acts[c][1], acts[c][2], r)
        assert torch.equal(y.view(torch.int32), single.view(torch.int32)), (k, r, c)
    for k in (0, 7, 123, 359):
        r, c, codes, scales, y = ins[k]
        x, _, _ = acts[c]
        xq, xs = oracle.act_quant(x)
        y64, yabs = oracle.fp4_gemv_f64(fmt, codes.cpu().numpy(), scales.cpu().numpy(), xq, xs, 0.75)
        gu.assert_within_tolerance(y.cpu().numpy(), y64, yabs, what=f"linear {k} {r}x{c}")


@pytest.mark.parametrize("fmt,M", [(MX, 1), (NV, 1), (MX, 8), (NV, 8)])
def test_expert_sweep_as_benchmarked(gpu, gu, fmt, M):
    """The benchmark's launch: the 1032 routed-expert linears of one decode
    step (device-drawn, load-checked) in one sequence launch, at M = 1 and with
    an 8-row panel (then each wave finishes ~43 units, more than it holds back
    to the end of the launch: the held and the directly written outputs are
    both checked). Every output equals its single call bitwise; every output
    of every 4th linear (M = 1) or 16th (M = 8), and of the last, lies within
    tolerance of the oracle's double GEMV."""
    plan = I.expert_sweep_plan()
    ws = torch.empty(256, dtype=torch.uint8, device=gu.DEV)
    acts = {}
    for c in sorted({sp.cols for sp in plan}):
        x = gu.to_dev(I.host_fp4_linear(fmt, 1, c, M, 70 + c).x)
        acts[c] = (x, *act_quant_gpu(gpu, x))
    g = 1.0 if fmt == MX else 2.0 ** -6
    lins, ins = [], []
    for sp in plan:
        codes, scales = I.device_fp4_linear(fmt, sp.rows, sp.cols, sp.seed, gu.DEV)
        assert gpu.fp4_load_check(fmt, codes, scales, ws, check=False) == (0, -1), sp.name
        y = torch.full((M, sp.rows), float("nan"), dtype=torch.float32, device=gu.DEV)
        ins.append((sp, codes, scales, y))
        lins.append((codes, scales, g, acts[sp.cols][1], acts[sp.cols][2], y))
    seq = gpu.fp4_expert_sequence_init(fmt, lins)
    gpu.fp4_expert_sequence(seq)
    torch.cuda.synchronize()
    gu.say(f"  expert sweep fmt {fmt} M {M}: {len(lins)} linears launched")
    xqs = {c: oracle.act_quant(a[0].cpu().numpy().view(np.uint16)) for c, a in acts.items()}
    for i, (sp, codes, scales, y) in enumerate(ins):
        single = expert_gemv_gpu(gpu, fmt, codes, scales, g, acts[sp.cols][1], acts[sp.cols][2], sp.rows)
        assert torch.equal(y.view(torch.int32), single.view(torch.int32)), (i, sp.name)
        if i % (4 if M == 1 else 16) == 0 or i == len(ins) - 1:
            ch, sh = codes.cpu().numpy(), scales.cpu().numpy()
            y64, yabs = oracle.fp4_gemv_f64(fmt, ch, sh, *xqs[sp.cols], g, nthreads=NTHREADS)
            gu.assert_within_tolerance(y.cpu().numpy(), y64, yabs, what=sp.name)


@pytest.mark.parametrize("M", [1, 8])
def test_expert_sequence_graph_replays(gpu, gu, M):
    """An expert sequence captured in a HIP graph: every replay, with eager
    work and synchronizations between the replays, gives the eager bits (at
    M = 8 the outputs are held in LDS until each wave's last unit)."""
    shapes = [(2048, 4096), (300, 512), (4096, 2048), (17, 384)]
    for fmt in (MX, NV):
        lins_e, lins_g, ys_e, ys_g = [], [], [], []
        for k, (r, c) in enumerate(shapes):
            L = I.host_fp4_linear(fmt, r, c, M, 900 + k)
            xq, xs = act_quant_gpu(gpu, dev(gu, L.x))
            codes, scales = dev(gu, L.codes), dev(gu, L.scales)
            ye = torch.full((M, r), float("nan"), dtype=torch.float32, device=gu.DEV)
            yg = torch.full((M, r), float("nan"), dtype=torch.float32, device=gu.DEV)
            lins_e.append((codes, scales, L.global_scale, xq, xs, ye))
            lins_g.append((codes, scales, L.global_scale, xq, xs, yg))
            ys_e.append(ye)
            ys_g.append(yg)
        s_e = gpu.fp4_expert_sequence_init(fmt, lins_e)
        s_g = gpu.fp4_expert_sequence_init(fmt, lins_g)
        gpu.fp4_expert_sequence(s_e)
        torch.cuda.synchronize()
        assert gpu.prepared("fp4_expert_sequence", s_g)() == gpu.OK  # an eager launch first
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            assert gpu.prepared("fp4_expert_sequence", s_g, stream=cap)() == gpu.OK
        for rep in range(3):
            for y in ys_g:
                y.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            junk = torch.randn(1 << 20, device=gu.DEV).sum()  # eager work between replays
            torch.cuda.synchronize()
            for ye, yg in zip(ys_e, ys_g):
                assert torch.equal(ye.view(torch.int32), yg.view(torch.int32)), (fmt, rep)
        del junk
