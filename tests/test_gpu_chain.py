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
