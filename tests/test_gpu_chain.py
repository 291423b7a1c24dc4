"""GPU: the sweep's linears as a dependent decode chain (each group's input
is the previous group's output, "Module dsv4_gpu" page, DecodePath: one
launch per projection), captured once in a HIP graph and replayed.

Checked: after every replay (with eager work between replays) every output
of the chain equals, bit for bit, a separate fp8blk_gemv call on the input
buffer that fed it; the replays agree with each other; every output is
finite. The separate calls are themselves checked against the oracle by the
other GPU tests."""
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb
from block_scaled_fp8_fp8blk_amd import inputs

pytestmark = pytest.mark.gpu


def test_chain_graph_matches_per_linear_calls(gpu):
    import bench
    from gpu_util import DEV, say
    sw = bench.Sweep(torch, fb, inputs, DEV, 2, "fp8")
    ch = bench.Chain(torch, fb, sw, DEV)
    ch.calibrate()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        bench.run_calls(ch.calls(stream=cap))
    torch.cuda.synchronize()
    first = None
    for rep in range(3):
        say(f"  chain replay {rep}")
        for l in sw.lins:
            l["y"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ys = [l["y"].clone() for l in sw.lins]
        assert all(bool(torch.isfinite(y).all()) for y in ys)
        if first is None:
            first = ys
        else:
            assert all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(first, ys)), rep
        _ = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
    for kind, members, x in ch.groups:
        if kind != "launch":
            continue
        for m in members:
            y = torch.full_like(m["y"], float("nan"))
            fb.fp8blk_gemv(m["w"], m["grid"], x, y)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), m["y"].view(torch.int32)), m["spec"].name


def test_chained_launch_matches_per_linear_calls(gpu):
    """fp8blk_gemv_chain over the same groups (one cooperative launch): three
    launches in a row (the hand-off epoch moves on each time), each output
    equal bit for bit to a fp8blk_gemv call on the input that the group reads,
    x = bf16(c * y) formed by torch from the chain's own outputs, and to the
    graph chain's outputs."""
    import bench
    from gpu_util import DEV, say
    sw = bench.Sweep(torch, fb, inputs, DEV, 2, "fp8")
    ch = bench.Chain(torch, fb, sw, DEV)
    ch.calibrate()
    graph_ys = [l["y"].clone() for l in sw.lins]  # the eager calibration pass is the graph chain's arithmetic
    pc = bench.persistent_chain(torch, fb, ch)
    launches = [g for g in ch.groups if g[0] == "launch"]
    first = None
    for rep in range(3):
        say(f"  chained launch {rep}")
        for l in sw.lins:
            l["y"].fill_(float("nan"))
        fb.fp8blk_gemv_chain(pc, ch.x_in[0])
        assert fb.fp8blk_chain_status(pc) == fb.OK
        ys = [l["y"].clone() for l in sw.lins]
        assert all(bool(torch.isfinite(y).all()) for y in ys)
        if first is None:
            first = ys
        else:
            assert all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(first, ys)), rep
    for gi, (_kind, members, _x) in enumerate(launches):
        if gi == 0:
            x = ch.x_in[0]
        else:
            src = launches[gi - 1][1][0]["y"]
            x = torch.empty((1, src.numel()), dtype=torch.bfloat16, device=DEV)
            torch.mul(src, ch.c[gi - 1], out=x)
        for m in members:
            y = torch.full_like(m["y"], float("nan"))
            fb.fp8blk_gemv(m["w"], m["grid"], x, y)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int32), m["y"].view(torch.int32)), (gi, m["spec"].name)
    assert all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(graph_ys, first))


def _bf16_of_scaled(c, y_f32):
    """x = bf16(c * y): the float32 product, rounded to bf16 to nearest even."""
    import numpy as np
    return inputs.round_to_bf16_bits(np.float32(c) * np.asarray(y_f32, dtype=np.float32))


def test_chained_launch_shapes_against_oracle(gpu):
    """Every cols the chained launch takes (1024, 2048, 3072, 4096), ragged
    rows (not a multiple of a unit's 4, 8 or 16 rows), a group of three, a
    group reading an output five groups back, a middle group reading the chain
    input, and a linear feeding two later groups: each output equals the
    oracle's documented order (O7) bit for bit on the input the group reads
    (formed on the host from the chain's own outputs) and lies within 1e-5 of
    the double GEMV (O6)."""
    import numpy as np
    import oracle
    from gpu_util import DEV, DevLinear, assert_within_tolerance, say, to_dev, u32

    # (members as (rows, cols), src, c); src = (group, member) or None
    spec = [
        ([(1024, 2048), (77, 2048)], None, 1.0),          # g0: reads x0 (2048 cols)
        ([(3072, 1024), (13, 1024), (600, 1024)], (0, 0), 0.75),  # g1: cols 1024 from g0 m0 (1024 rows)
        ([(4096, 3072)], (1, 0), 1.25),                   # g2: cols 3072 from g1 m0
        ([(999, 4096), (2048, 4096)], (2, 0), 0.5),       # g3: cols 4096 from g2 m0
        ([(1031, 2048)], (3, 1), 2.0),                    # g4: cols 2048 from g3 m1 (2048 rows)
        ([(3072, 2048)], None, 1.0),                      # g5: reads x0 again
        ([(513, 3072)], (5, 0), 0.625),                   # g6: cols 3072 from g5 m0
        ([(45, 4096)], (2, 0), 1.5),                      # g7: g2 m0 again, from four groups back
    ]
    x0 = inputs.host_linear(1, 2048, 1, 900).x
    lins, groups, seed = [], [], 910
    for gi, (members, src, c) in enumerate(spec):
        mem = []
        for rows, cols in members:
            L = inputs.host_linear(rows, cols, 1, seed)
            seed += 1
            D = DevLinear(L.codes, L.scales)
            assert D.check()[0] == fb.OK
            y = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
            lins.append((L, D, y))
            mem.append((D.codes, D.grid, y))
        groups.append((mem, src, c))
    first = [0]
    for members, _s, _c in spec:
        first.append(first[-1] + len(members))
    pc = fb.fp8blk_chain_init(groups)
    x0d = to_dev(x0.reshape(-1))
    for rep in range(2):
        say(f"  chained launch over {len(spec)} groups, launch {rep}")
        for _L, _D, y in lins:
            y.fill_(float("nan"))
        fb.fp8blk_gemv_chain(pc, x0d)
        assert fb.fp8blk_chain_status(pc) == fb.OK
        ys = [y.cpu().numpy() for _L, _D, y in lins]
        for gi, (members, src, c) in enumerate(spec):
            if src is None:
                x = np.ascontiguousarray(x0[:, :members[0][1]])  # a group reads the first cols entries of x0
            else:
                x = _bf16_of_scaled(c, ys[first[src[0]] + src[1]]).reshape(1, -1)
            for k in range(len(members)):
                L = lins[first[gi] + k][0]
                y = ys[first[gi] + k].reshape(1, -1)
                y7 = oracle.gemv_f32_order(x, codes=L.codes, scales=L.scales)
                nd = int(np.sum(u32(y) != u32(y7)))
                assert nd == 0, f"group {gi} linear {k} ({L.rows}x{L.cols}): {nd} outputs differ from O7"
                y64, yabs = oracle.gemv_f64(L.codes, L.scales, x)
                assert_within_tolerance(y, y64, yabs, what=f"group {gi} linear {k}")


def test_chain_with_glue_in_launches(gpu):
    """The chain's launches with the glue inside them (scaled-input launches,
    captured in a graph and replayed three times): every output equals, bit
    for bit, the graph chain's (its x formed by a torch kernel between the
    launches) and the chained launch's."""
    import bench
    from gpu_util import DEV, say
    sw = bench.Sweep(torch, fb, inputs, DEV, 2, "fp8")
    ch = bench.Chain(torch, fb, sw, DEV)
    ch.calibrate()
    graph_ys = [l["y"].clone() for l in sw.lins]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        bench.run_calls(ch.scaled_calls(stream=cap))
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"  glue-in-launch chain replay {rep}")
        for l in sw.lins:
            l["y"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a.view(torch.int32), l["y"].view(torch.int32)) for a, l in zip(graph_ys, sw.lins)), rep
        _ = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
    pc = bench.persistent_chain(torch, fb, ch)
    for l in sw.lins:
        l["y"].fill_(float("nan"))
    fb.fp8blk_gemv_chain(pc, ch.x_in[0])
    assert fb.fp8blk_chain_status(pc) == fb.OK
    assert all(torch.equal(a.view(torch.int32), l["y"].view(torch.int32)) for a, l in zip(graph_ys, sw.lins))


def test_chain_with_glue_in_producer(gpu):
    """The chain's launches with the glue in the producer (next-input
    launches, captured in a graph and replayed three times): every output and
    every group input equals, bit for bit, the graph chain's."""
    import bench
    from gpu_util import DEV, say
    sw = bench.Sweep(torch, fb, inputs, DEV, 2, "fp8")
    ch = bench.Chain(torch, fb, sw, DEV)
    ch.calibrate()
    graph_ys = [l["y"].clone() for l in sw.lins]
    xs = [g[2] for g in ch.groups if g[0] == "launch"]
    graph_xs = [x.clone() for x in xs]
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        bench.run_calls(ch.next_calls(stream=cap))
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"  glue-in-producer chain replay {rep}")
        for l in sw.lins:
            l["y"].fill_(float("nan"))
        for x in xs[1:]:
            x.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a.view(torch.int32), l["y"].view(torch.int32)) for a, l in zip(graph_ys, sw.lins)), rep
        assert all(torch.equal(a.view(torch.int16), x.view(torch.int16)) for a, x in zip(graph_xs, xs)), rep
        _ = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
