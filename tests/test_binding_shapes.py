"""CPU: the Python binding refuses mis-shaped tensors before any launch.

The C ABI takes plain pointers and sizes and cannot see a buffer's size, so a
tensor that holds fewer elements than the shapes imply would be read or
written out of bounds on the device. Every wrapper checks the shapes first
and raises ValueError; with the right shapes the same call goes on to the
device check, which CPU tensors fail with TypeError (no GPU is touched)."""
import pytest
import torch

import block_scaled_fp8_fp8blk_amd as fb

U8, F32, BF = torch.uint8, torch.float32, torch.bfloat16


def z(*shape, dtype=U8):
    return torch.zeros(shape, dtype=dtype)


R, C, M = 256, 512, 3  # 2 x 4 block grid


def good():
    return dict(codes=z(R, C), scales=z(2, 4), grid=z(2, 4, dtype=F32), x=z(M, C, dtype=BF), y=z(M, R, dtype=F32),
                slab=z(R, C, dtype=BF), ws=z(256))


CASES = {
    "load_check": (lambda t: fb.fp8blk_load_check(t["codes"], t["scales"], t["grid"], t["ws"]),
                   [("scales", z(2, 3)), ("grid", z(1, 4, dtype=F32)), ("codes", z(R * C))]),
    "load_check_noalloc": (lambda t: fb.fp8blk_load_check_noalloc(t["codes"], t["scales"], t["grid"]),
                           [("scales", z(3, 4)), ("grid", z(2, 5, dtype=F32))]),
    "dequant": (lambda t: fb.fp8blk_dequant_bf16(t["codes"], t["grid"], t["slab"]),
                [("slab", z(R - 1, C, dtype=BF)), ("grid", z(2, 3, dtype=F32))]),
    "gemv": (lambda t: fb.fp8blk_gemv(t["codes"], t["grid"], t["x"], t["y"]),
             [("x", z(M, C - 16, dtype=BF)), ("y", z(M, R - 1, dtype=F32)), ("y", z(M - 1, R, dtype=F32)),
              ("grid", z(1, 4, dtype=F32)), ("x", z(M * C, dtype=BF))]),
    "twin": (lambda t: fb.bf16_gemv_twin(t["slab"], t["x"], t["y"]),
             [("x", z(M, C + 16, dtype=BF)), ("y", z(M, R + 4, dtype=F32))]),
    "mfma": (lambda t: fb.fp8blk_gemv_mfma(t["codes"], t["grid"], t["x"], t["y"]),
             [("y", z(1, R, dtype=F32)), ("grid", z(9, dtype=F32))]),
    "twin_mfma": (lambda t: fb.bf16_gemv_twin_mfma(t["slab"], t["x"], t["y"]),
                  [("y", z(M, R - 8, dtype=F32))]),
    "grouped": (lambda t: fb.fp8blk_gemv_grouped([(t["codes"], t["grid"], t["y"])], t["x"]),
                [("y", z(M, R // 2, dtype=F32)), ("grid", z(4, 4, dtype=F32))]),
    "twin_grouped": (lambda t: fb.bf16_gemv_twin_grouped([(t["slab"], t["y"])], t["x"]),
                     [("x", z(M, C // 2, dtype=BF))]),
    "gemm_staged": (lambda t: fb.fp8blk_gemm_staged(t["codes"], t["grid"], t["x"], t["y"], t["ws"]),
                    [("y", z(M, R - 1, dtype=F32))]),
    "gemm_twin": (lambda t: fb.bf16_gemm_twin(t["slab"], t["x"], t["y"], t["ws"]),
                  [("x", z(M, C - 1, dtype=BF))]),
    "sequence": (lambda t: fb.fp8blk_sequence_init(fb.ARM_FP8_MFMA, [(t["codes"], t["grid"], t["x"], t["y"])], ws=t["ws"]),
                 [("y", z(M, R + 1, dtype=F32)), ("grid", z(2, 2, dtype=F32))]),
    "twin_sequence": (lambda t: fb.fp8blk_sequence_init(fb.ARM_BF16, [(t["slab"], t["x"], t["y"])], ws=t["ws"]),
                      [("x", z(M, 16, dtype=BF))]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_misshaped_call_raises_value_error(name):
    call, bad = CASES[name]
    with pytest.raises(TypeError):  # right shapes: stops at the CUDA-tensor check
        call(good())
    for key, tensor in bad:
        t = good()
        t[key] = tensor
        with pytest.raises(ValueError):
            call(t)


def test_expert_wrappers_check_shapes():
    rows, cols, Mx = 64, 256, 2
    codes, sc_mx = z(rows, cols // 2), z(rows, cols // 32)
    xq, xs, y = z(Mx, cols), z(Mx, cols // 128), z(Mx, rows, dtype=F32)
    with pytest.raises(TypeError):
        fb.fp4_expert_gemv(fb.FMT_MXFP4, codes, sc_mx, 1.0, xq, xs, y)
    for args in [(z(rows, cols // 16), xq, xs, y), (sc_mx, z(Mx, cols - 2), xs, y), (sc_mx, xq, z(Mx, 1), y),
                 (sc_mx, xq, xs, z(Mx, rows - 1, dtype=F32))]:
        with pytest.raises(ValueError):
            fb.fp4_expert_gemv(fb.FMT_MXFP4, codes, args[0], 1.0, *args[1:])
    with pytest.raises(ValueError):
        fb.fp4_dequant_bf16(fb.FMT_NVFP4, codes, z(rows, cols // 16), z(rows, cols - 2, dtype=BF))
    with pytest.raises(ValueError):
        fb.fp4_load_check(fb.FMT_NVFP4, codes, z(rows, cols // 32), z(256))
    with pytest.raises(ValueError):
        fb.fp8blk_act_quant(z(Mx, cols, dtype=BF), z(Mx, cols), z(Mx, 3))
    with pytest.raises(ValueError):
        fb.fp4_expert_sequence_init(fb.FMT_MXFP4, [(codes, sc_mx, 1.0, xq, xs, z(Mx + 1, rows, dtype=F32))],
                                    ws=z(256))


def test_one_device_rule():
    t = good()
    t["y"] = torch.zeros((M, R), dtype=F32, device="meta")
    with pytest.raises(ValueError):
        fb.fp8blk_gemv(t["codes"], t["grid"], t["x"], t["y"])
