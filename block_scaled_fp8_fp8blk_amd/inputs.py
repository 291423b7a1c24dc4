"""Seeded synthetic inputs for the FP8-blk dense linear.

This module only draws inputs. It holds none of the method's arithmetic: it
never decodes an e4m3 or e8m0 code and never forms a product or a sum of the
linear. Both the HIP path's tests and benchmark and the CPU oracle's tests
draw from here, and nothing else is shared between them.

Layouts (row-major, contiguous):
  codes  uint8  [rows, cols]            e4m3 code bytes, rows = output features
  scales uint8  [ceil(rows/128), ceil(cols/128)]   e8m0 block-scale codes
  x      uint16 [M, cols]               bf16 bit patterns of the activations

Draw order from one ``numpy.random.default_rng(seed)``: codes, then scales,
then x.  Rounding to e4m3 and to bf16 is round-to-nearest-even, done by
PyTorch's own dtype casts (``float8_e4m3fn``, ``bfloat16``) on the CPU.

The whole-step sweep (259 linears, ~3.2e9 codes) is drawn on the device with
torch's seeded Philox generator instead (``device_linear``): a host draw of
that size takes minutes. Its distributions are the same.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 128

# Finite e4m3 bytes: everything except the two NaN patterns 0x7F and 0xFF.
FINITE_E4M3 = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)


def grid_shape(rows: int, cols: int) -> tuple[int, int]:
    return (-(-rows // BLOCK), -(-cols // BLOCK))


def _torch():
    import torch
    return torch


def round_to_e4m3(values_f32: np.ndarray) -> np.ndarray:
    """Nearest-even e4m3 code bytes of float32 values (PyTorch's cast)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def round_to_bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns (uint16) of float32 values."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Linear:
    rows: int
    cols: int
    codes: np.ndarray
    scales: np.ndarray
    x: np.ndarray
    seed: int
    name: str = ""

    @property
    def M(self) -> int:
        return self.x.shape[0]

    def weight_bytes(self) -> int:
        """Codes plus the f32 scale grid: the bytes the FP8-blk GEMV must read."""
        gr, gc = grid_shape(self.rows, self.cols)
        return self.rows * self.cols + 4 * gr * gc


def host_linear(rows: int, cols: int, M: int, seed: int, *, codes: str = "normal",
                sigma: float = 0.05, scale_lo: int = 124, scale_hi: int = 130,
                name: str = "") -> Linear:
    """One synthetic FP8-blk linear drawn on the host.

    codes="uniform": uniform over the 254 finite e4m3 bytes.
    codes="normal":  e4m3 rounding of float32 N(0,1) * sigma.
    Scale codes are uniform integers in [scale_lo, scale_hi].
    x rows are bf16 roundings of float32 N(0,1).
    """
    rng = np.random.default_rng(seed)
    if codes == "uniform":
        idx = rng.integers(0, FINITE_E4M3.size, size=(rows, cols))
        c = FINITE_E4M3[idx]
    elif codes == "normal":
        v = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)
        c = round_to_e4m3(v)
    else:
        raise ValueError(f"unknown code distribution {codes!r}")
    gr, gc = grid_shape(rows, cols)
    s = rng.integers(scale_lo, scale_hi + 1, size=(gr, gc), dtype=np.int64).astype(np.uint8)
    xv = rng.standard_normal((M, cols), dtype=np.float32)
    x = round_to_bf16_bits(xv)
    return Linear(rows, cols, np.ascontiguousarray(c, dtype=np.uint8), s, x, seed, name)


# ---------------------------------------------------------------------------
# The five workloads (shapes, distributions and seeds).
# ---------------------------------------------------------------------------

def tiny() -> Linear:
    """256 x 512 (2 x 4 grid of 128 x 128 blocks), M=1; codes uniform over the
    finite bytes; scales uniform in [120, 134]; seed 0."""
    return host_linear(256, 512, 1, 0, codes="uniform", scale_lo=120, scale_hi=134, name="tiny")


def decode_shape() -> Linear:
    """4096 x 4096, M=1; codes e4m3(N(0,1)*0.05); scales in [124, 130]; seed 1."""
    return host_linear(4096, 4096, 1, 1, name="decode_4096x4096")


def projection_pair() -> list[Linear]:
    """gate and up 16384 x 4096, down 4096 x 16384, M=1; seeds 2, 3, 4."""
    return [host_linear(16384, 4096, 1, 2, name="gate_16384x4096"),
            host_linear(16384, 4096, 1, 3, name="up_16384x4096"),
            host_linear(4096, 16384, 1, 4, name="down_4096x16384")]


VERIFY_M = (2, 4, 8, 16)
# (rows, cols, panel rows, seed) of the batched-verify workload.
VERIFY_SPECS = ((12288, 4096, 16, 5), (4096, 4096, 16, 6))


def verify_panel() -> list[Linear]:
    """12288 x 4096 and 4096 x 4096 with a 16-row activation panel (seeds 5, 6).
    The M in {2, 4, 8} panels are the leading rows of the 16-row panel."""
    return [host_linear(r, c, m, s, name=f"verify_{r}x{c}") for r, c, m, s in VERIFY_SPECS]


@dataclass
class SweepLinear:
    name: str
    rows: int
    cols: int
    seed: int

    def weight_bytes(self) -> int:
        gr, gc = grid_shape(self.rows, self.cols)
        return self.rows * self.cols + 4 * gr * gc


@dataclass
class Sweep:
    linears: list = field(default_factory=list)

    def weight_bytes(self) -> int:
        return sum(l.weight_bytes() for l in self.linears)


SWEEP_LAYERS = 43
# (name, rows = out features, cols = in features) of one layer's dense linears.
SWEEP_LAYER_SHAPES = (("q", 4096, 4096), ("kv", 1024, 4096), ("o", 4096, 4096),
                      ("gate", 2048, 4096), ("up", 2048, 4096), ("down", 4096, 2048))
SWEEP_HEAD = ("head", 129280, 4096)


def sweep_plan(layers: int = SWEEP_LAYERS) -> Sweep:
    """The whole-step dense sweep: per layer q, kv, o, shared-expert gate, up,
    down, then the head; linear i is drawn with seed 100 + i."""
    out = []
    i = 0
    for layer in range(layers):
        for nm, r, c in SWEEP_LAYER_SHAPES:
            out.append(SweepLinear(f"L{layer}.{nm}", r, c, 100 + i))
            i += 1
    nm, r, c = SWEEP_HEAD
    out.append(SweepLinear(nm, r, c, 100 + i))
    return Sweep(out)


def device_linear(rows: int, cols: int, seed: int, device, *, sigma: float = 0.05,
                  scale_lo: int = 124, scale_hi: int = 130):
    """Codes and scales drawn on ``device`` with torch's seeded generator:
    e4m3 rounding of float32 N(0,1)*sigma and uniform scale codes.
    Returns (codes uint8 [rows, cols], scales uint8 [grid]) device tensors."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    step = max(1, (1 << 28) // cols)  # bound the float32 temporary to ~1 GiB
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        v = torch.randn((r1 - r0, cols), generator=g, dtype=torch.float32, device=device)
        v.mul_(sigma)
        codes[r0:r1] = v.to(torch.float8_e4m3fn).view(torch.uint8)
        del v
    gr, gc = grid_shape(rows, cols)
    scales = torch.randint(scale_lo, scale_hi + 1, (gr, gc), generator=g, dtype=torch.int32,
                           device=device).to(torch.uint8)
    return codes, scales


def device_x(cols: int, M: int, seed: int, device):
    """bf16 bit patterns (as int16) of float32 N(0,1), drawn on ``device``."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    v = torch.randn((M, cols), generator=g, dtype=torch.float32, device=device)
    return v.to(torch.bfloat16).view(torch.int16)


# ---------------------------------------------------------------------------
# Native expert arm: FP4 (e2m1) weight slabs in the MXFP4 and NVFP4 recipes.
#   codes  uint8 [rows, cols/2]   two e2m1 codes per byte (even column in the
#                                 low nibble), drawn as uniform random bytes
#   scales uint8 [rows, cols/B]   MXFP4 (B = 32): e8m0 codes; NVFP4 (B = 16):
#                                 e4m3 codes, non-negative and finite
#   global_scale                  NVFP4's per-tensor f32 output scale (1.0 for
#                                 MXFP4)
#   x      uint16 [M, cols]       bf16 activations, N(0,1)
# Draw order from one generator: codes, scales, global scale, x.
# ---------------------------------------------------------------------------

MXFP4, NVFP4 = 0, 1
FP4_BLOCK = {MXFP4: 32, NVFP4: 16}
FP4_NAMES = {MXFP4: "mxfp4", NVFP4: "nvfp4"}
# Default scale-code ranges: MXFP4 2^-9 .. 2^-1; NVFP4 e4m3 bytes 0x28 .. 0x58
# (2^-2 .. 2^4, every mantissa).
FP4_SCALE_RANGE = {MXFP4: (118, 126), NVFP4: (0x28, 0x58)}


@dataclass
class Fp4Linear:
    fmt: int
    rows: int
    cols: int
    codes: np.ndarray
    scales: np.ndarray
    global_scale: float
    x: np.ndarray
    seed: int
    name: str = ""

    @property
    def M(self) -> int:
        return self.x.shape[0]

    def weight_bytes(self) -> int:
        return fp4_weight_bytes(self.fmt, self.rows, self.cols)


def fp4_weight_bytes(fmt: int, rows: int, cols: int) -> int:
    """Packed codes plus the block-scale bytes: what the expert GEMV must read."""
    return rows * cols // 2 + rows * (cols // FP4_BLOCK[fmt])


def host_fp4_linear(fmt: int, rows: int, cols: int, M: int, seed: int, *, scale_lo: int | None = None,
                    scale_hi: int | None = None, name: str = "") -> Fp4Linear:
    """One synthetic FP4 expert linear drawn on the host. NVFP4's global
    scale is a float32 drawn uniformly in [2^-7, 2^-5)."""
    B = FP4_BLOCK[fmt]
    assert cols % B == 0
    lo, hi = FP4_SCALE_RANGE[fmt]
    lo = lo if scale_lo is None else scale_lo
    hi = hi if scale_hi is None else scale_hi
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.int64).astype(np.uint8)
    scales = rng.integers(lo, hi + 1, size=(rows, cols // B), dtype=np.int64).astype(np.uint8)
    g = rng.uniform(1.0, 4.0) * 2.0 ** -7
    g = float(np.float32(g)) if fmt == NVFP4 else 1.0
    xv = rng.standard_normal((M, cols), dtype=np.float32)
    return Fp4Linear(fmt, rows, cols, codes, scales, g, round_to_bf16_bits(xv), seed, name)


def device_fp4_linear(fmt: int, rows: int, cols: int, seed: int, device):
    """Codes and scales of an FP4 expert linear drawn on ``device`` with
    torch's seeded generator (same distributions as host_fp4_linear).
    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/B])."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    codes = torch.randint(0, 256, (rows, cols // 2), generator=g, dtype=torch.int32, device=device).to(torch.uint8)
    lo, hi = FP4_SCALE_RANGE[fmt]
    scales = torch.randint(lo, hi + 1, (rows, cols // FP4_BLOCK[fmt]), generator=g, dtype=torch.int32,
                           device=device).to(torch.uint8)
    return codes, scales


# Routed-expert projections of one decode step: per layer, the activated
# experts' gate, up (intermediate 2048 from hidden 4096) and down.
EXPERT_LAYERS = 43
EXPERTS_PER_TOKEN = 8
EXPERT_SHAPES = (("gate", 2048, 4096), ("up", 2048, 4096), ("down", 4096, 2048))


@dataclass
class ExpertSweepLinear:
    name: str
    rows: int
    cols: int
    seed: int


def expert_sweep_plan(layers: int = EXPERT_LAYERS, experts: int = EXPERTS_PER_TOKEN) -> list:
    """The routed-expert sweep of one decode step: layers x activated experts x
    (gate, up, down); linear i is drawn with seed 20000 + i."""
    out = []
    i = 0
    for layer in range(layers):
        for e in range(experts):
            for nm, r, c in EXPERT_SHAPES:
                out.append(ExpertSweepLinear(f"L{layer}.e{e}.{nm}", r, c, 20000 + i))
                i += 1
    return out
