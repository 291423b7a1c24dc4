"""Helpers for the GPU parity tests: upload seeded inputs, run the C ABI
through the binding, and compare with the oracle."""
import sys

import numpy as np
import torch

import block_scaled_fp8_fp8blk_amd as fb
import oracle

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def u32(t) -> np.ndarray:
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else t
    return np.ascontiguousarray(a).view(np.uint32)


class DevLinear:
    """A linear's inputs on the device, load-checked, with its f32 grid."""

    def __init__(self, codes, scales, x=None):
        self.codes = codes if isinstance(codes, torch.Tensor) else to_dev(codes)
        self.scales = scales if isinstance(scales, torch.Tensor) else to_dev(scales)
        self.rows, self.cols = self.codes.shape
        self.grid = torch.empty(self.scales.shape, dtype=torch.float32, device=DEV)
        self.ws = torch.empty(fb.fp8blk_workspace_bytes(fb.OP_LOAD_CHECK, self.rows, self.cols),
                              dtype=torch.uint8, device=DEV)
        self.x = None if x is None else (x if isinstance(x, torch.Tensor) else to_dev(x))

    def check(self, check=True):
        return fb.fp8blk_load_check(self.codes, self.scales, self.grid, self.ws, check=check)

    def slab(self) -> torch.Tensor:
        out = torch.empty((self.rows, self.cols), dtype=torch.int16, device=DEV)
        fb.fp8blk_dequant_bf16(self.codes, self.grid, out)
        return out

    def gemv(self, x=None) -> torch.Tensor:
        x = self.x if x is None else x
        y = torch.full((x.shape[0], self.rows), float("nan"), dtype=torch.float32, device=DEV)
        fb.fp8blk_gemv(self.codes, self.grid, x, y)
        return y

    def twin(self, slab, x=None) -> torch.Tensor:
        x = self.x if x is None else x
        y = torch.full((x.shape[0], self.rows), float("nan"), dtype=torch.float32, device=DEV)
        fb.bf16_gemv_twin(slab, x, y)
        return y


def assert_within_tolerance(y_gpu: np.ndarray, y64: np.ndarray, yabs: np.ndarray, rel=1e-5, what=""):
    """|y - y64| <= rel * sum|w x| per element; a zero sum demands y == 0."""
    y = y_gpu.astype(np.float64)
    err = np.abs(y - y64)
    bad = err > rel * yabs
    assert not np.any(bad), (f"{what}: {int(bad.sum())} outputs beyond {rel} * sum|wx|; worst "
                             f"{float(np.max(err / np.maximum(yabs, 1e-300))):.3e}")


def full_parity(L, codes, scales, x, y8: np.ndarray, yt: np.ndarray, nthreads=None, what=""):
    """FP8 == twin bitwise, both == documented order (O7) bitwise, both within
    1e-5 of the double GEMV (O6)."""
    assert np.array_equal(u32(y8), u32(yt)), f"{what}: FP8 GEMV and bf16 twin differ"
    y7 = oracle.gemv_f32_order(x, codes=codes, scales=scales, nthreads=nthreads)
    nd = int(np.sum(u32(y8) != u32(y7)))
    assert nd == 0, f"{what}: {nd} outputs differ from the documented order"
    y64, yabs = oracle.gemv_f64(codes, scales, x, nthreads=nthreads)
    assert_within_tolerance(y8, y64, yabs, what=what)
