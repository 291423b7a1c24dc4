"""Python binding of libfp8blk.so (the FP8-blk dense linear for MI355X).

Argument marshalling only: every function here forwards device pointers,
sizes and the caller's stream to the C ABI declared in include/fp8blk.h, and
every step of the computation runs in the library's HIP kernels. PyTorch is
used for device memory and streams only. If the shared library has not been
built, the first call raises: there is no fallback of any kind.

Tensors must be contiguous CUDA (HIP) tensors of these dtypes:
  codes, scales_e8m0      torch.uint8
  scales_f32, y           torch.float32
  x_bf16, w_bf16, out     torch.bfloat16, torch.int16 or torch.uint16 (bf16 bit patterns)
  ws                      any dtype, or None when the op needs no workspace
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8blk.so")

OK, ERR_ARG, ERR_SCALE_FF, ERR_NAN_CODE, ERR_INEXACT, ERR_WORKSPACE, ERR_HIP, ERR_BAD_SCALE, ERR_TIMEOUT = range(9)
OP_LOAD_CHECK, OP_DEQUANT_BF16, OP_GEMV, OP_BF16_TWIN, OP_GEMM_STAGED, OP_BF16_GEMM = range(6)
MIN_COLS, MAX_COLS, MAX_M, MAX_PANEL = 16, 65536, 16, 65536

# Every symbol include/fp8blk.h declares.
EXPORTS = ("fp8blk_abi_version", "fp8blk_strerror", "fp8blk_workspace_bytes", "fp8blk_load_check",
           "fp8blk_load_check_noalloc",
           "fp8blk_dequant_bf16", "fp8blk_gemv", "bf16_gemv_twin", "fp8blk_gemv_grouped", "bf16_gemv_twin_grouped",
           "fp8blk_gemv_scaled_input", "fp8blk_gemv_grouped_scaled_input", "fp8blk_gemv_next_input",
           "fp8blk_gemv_grouped_next_input",
           "fp8blk_gemv_mfma", "bf16_gemv_twin_mfma", "fp8blk_sequence_bytes", "fp8blk_sequence_init",
           "fp8blk_gemv_sequence", "bf16_gemv_twin_sequence", "fp8blk_gemv_mfma_sequence",
           "bf16_gemv_twin_mfma_sequence", "fp8blk_gemm_staged", "bf16_gemm_twin", "fp8blk_act_quant",
           "fp4_load_check", "fp4_dequant_bf16", "fp4_expert_gemv", "fp4_expert_sequence_init",
           "fp4_expert_sequence", "fp8blk_chain_bytes", "fp8blk_chain_init", "fp8blk_gemv_chain",
           "fp8blk_chain_status")
MAX_GROUP = 8
MAX_SEQ = 65536
MAX_CHAIN = 65536
CHAIN_COLS = (1024, 2048, 3072, 4096)
ARM_FP8, ARM_BF16, ARM_FP8_MFMA, ARM_BF16_MFMA, ARM_MXFP4, ARM_NVFP4 = 0, 1, 2, 3, 4, 5
FMT_MXFP4, FMT_NVFP4 = 0, 1


class Linear(ctypes.Structure):
    """fp8blk_linear: one member of a grouped launch."""
    _fields_ = [("w", ctypes.c_void_p), ("scales_f32", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("y", ctypes.c_void_p)]



class SeqLinear(ctypes.Structure):
    """fp8blk_seq_linear: one member of a sequence launch."""
    _fields_ = [("w", ctypes.c_void_p), ("scales_f32", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("M", ctypes.c_int64), ("x_bf16", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class Fp4ExpertLinear(ctypes.Structure):
    """fp4_expert_linear: one member of an expert sequence launch."""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_float),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("M", ctypes.c_int64), ("xq", ctypes.c_void_p),
                ("xs", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class SequenceHandle(ctypes.Structure):
    """fp8blk_sequence: the host-side record of a planned sequence."""
    _fields_ = [("plan", ctypes.c_void_p), ("units_dense", ctypes.c_int64), ("units_general", ctypes.c_int64),
                ("n", ctypes.c_int32), ("arm", ctypes.c_int32), ("grid_dense", ctypes.c_int32),
                ("grid_general", ctypes.c_int32), ("M", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ChainGroup(ctypes.Structure):
    """fp8blk_chain_group: one group of a chained launch."""
    _fields_ = [("first", ctypes.c_int32), ("n", ctypes.c_int32), ("cols", ctypes.c_int64), ("src", ctypes.c_int32),
                ("c", ctypes.c_float)]


class ChainHandle(ctypes.Structure):
    """fp8blk_chain: the host-side record of a planned chained launch."""
    _fields_ = [("plan", ctypes.c_void_p), ("units", ctypes.c_int64), ("n_linears", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("grid", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


class Fp8BlkError(RuntimeError):
    def __init__(self, status: int, where: str, first_bad: int = -1):
        self.status = status
        self.first_bad = first_bad
        msg = f"{where}: {fp8blk_strerror(status)} (status {status})"
        if first_bad >= 0:
            msg += f", first bad index {first_bad}"
        super().__init__(msg)


def load():
    """Load libfp8blk.so (built by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    L.fp8blk_abi_version.argtypes, L.fp8blk_abi_version.restype = [], i32
    L.fp8blk_strerror.argtypes, L.fp8blk_strerror.restype = [i32], ctypes.c_char_p
    L.fp8blk_workspace_bytes.argtypes, L.fp8blk_workspace_bytes.restype = [i32, i64, i64, i64], sz
    L.fp8blk_load_check.argtypes = [vp, vp, i64, i64, vp, vp, sz, ctypes.POINTER(i64), vp]
    L.fp8blk_load_check.restype = i32
    L.fp8blk_load_check_noalloc.argtypes = [vp, vp, i64, i64, vp, ctypes.POINTER(i64), vp]
    L.fp8blk_load_check_noalloc.restype = i32
    L.fp8blk_dequant_bf16.argtypes, L.fp8blk_dequant_bf16.restype = [vp, vp, i64, i64, vp, vp], i32
    L.fp8blk_gemv.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, sz, vp]
    L.fp8blk_gemv.restype = i32
    L.bf16_gemv_twin.argtypes = [vp, i64, i64, vp, i64, vp, vp, sz, vp]
    L.bf16_gemv_twin.restype = i32
    L.fp8blk_gemv_grouped.argtypes = [ctypes.POINTER(Linear), i32, i64, vp, i64, vp]
    L.fp8blk_gemv_grouped.restype = i32
    L.bf16_gemv_twin_grouped.argtypes = [ctypes.POINTER(Linear), i32, i64, vp, i64, vp]
    L.bf16_gemv_twin_grouped.restype = i32
    L.fp8blk_gemv_scaled_input.argtypes = [vp, vp, i64, i64, vp, ctypes.c_float, vp, vp]
    L.fp8blk_gemv_scaled_input.restype = i32
    L.fp8blk_gemv_grouped_scaled_input.argtypes = [ctypes.POINTER(Linear), i32, i64, vp, ctypes.c_float, vp]
    L.fp8blk_gemv_grouped_scaled_input.restype = i32
    L.fp8blk_gemv_next_input.argtypes = [vp, vp, i64, i64, vp, vp, ctypes.c_float, vp, vp]
    L.fp8blk_gemv_next_input.restype = i32
    L.fp8blk_gemv_grouped_next_input.argtypes = [ctypes.POINTER(Linear), i32, i64, vp, i32, ctypes.c_float, vp, vp]
    L.fp8blk_gemv_grouped_next_input.restype = i32
    L.fp8blk_gemv_mfma.argtypes, L.fp8blk_gemv_mfma.restype = [vp, vp, i64, i64, vp, i64, vp, vp], i32
    L.bf16_gemv_twin_mfma.argtypes, L.bf16_gemv_twin_mfma.restype = [vp, i64, i64, vp, i64, vp, vp], i32
    L.fp8blk_sequence_bytes.argtypes, L.fp8blk_sequence_bytes.restype = [i32], sz
    L.fp8blk_sequence_init.argtypes = [ctypes.POINTER(SequenceHandle), i32, ctypes.POINTER(SeqLinear), i32, vp, sz,
                                       vp]
    L.fp8blk_sequence_init.restype = i32
    L.fp8blk_gemv_sequence.argtypes = [ctypes.POINTER(SequenceHandle), vp]
    L.fp8blk_gemv_sequence.restype = i32
    L.bf16_gemv_twin_sequence.argtypes = [ctypes.POINTER(SequenceHandle), vp]
    L.bf16_gemv_twin_sequence.restype = i32
    L.fp8blk_gemm_staged.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, sz, vp]
    L.fp8blk_gemm_staged.restype = i32
    L.bf16_gemm_twin.argtypes = [vp, i64, i64, vp, i64, vp, vp, sz, vp]
    L.bf16_gemm_twin.restype = i32
    L.fp8blk_gemv_mfma_sequence.argtypes = [ctypes.POINTER(SequenceHandle), vp]
    L.fp8blk_gemv_mfma_sequence.restype = i32
    L.bf16_gemv_twin_mfma_sequence.argtypes = [ctypes.POINTER(SequenceHandle), vp]
    L.bf16_gemv_twin_mfma_sequence.restype = i32
    f32 = ctypes.c_float
    L.fp8blk_act_quant.argtypes, L.fp8blk_act_quant.restype = [vp, i64, i64, vp, vp, vp], i32
    L.fp4_load_check.argtypes = [i32, vp, vp, i64, i64, vp, sz, ctypes.POINTER(i64), vp]
    L.fp4_load_check.restype = i32
    L.fp4_dequant_bf16.argtypes, L.fp4_dequant_bf16.restype = [i32, vp, vp, i64, i64, vp, vp], i32
    L.fp4_expert_gemv.argtypes = [i32, vp, vp, f32, i64, i64, vp, vp, i64, vp, vp]
    L.fp4_expert_gemv.restype = i32
    L.fp4_expert_sequence_init.argtypes = [ctypes.POINTER(SequenceHandle), i32, ctypes.POINTER(Fp4ExpertLinear),
                                           i32, vp, sz, vp]
    L.fp4_expert_sequence_init.restype = i32
    L.fp4_expert_sequence.argtypes, L.fp4_expert_sequence.restype = [ctypes.POINTER(SequenceHandle), vp], i32
    L.fp8blk_chain_bytes.argtypes = [ctypes.POINTER(Linear), i32, ctypes.POINTER(ChainGroup), i32]
    L.fp8blk_chain_bytes.restype = sz
    L.fp8blk_chain_init.argtypes = [ctypes.POINTER(ChainHandle), ctypes.POINTER(Linear), i32,
                                    ctypes.POINTER(ChainGroup), i32, vp, sz, vp]
    L.fp8blk_chain_init.restype = i32
    L.fp8blk_gemv_chain.argtypes, L.fp8blk_gemv_chain.restype = [ctypes.POINTER(ChainHandle), vp, vp], i32
    L.fp8blk_chain_status.argtypes, L.fp8blk_chain_status.restype = [ctypes.POINTER(ChainHandle), vp], i32
    _lib = L
    return L


def fp8blk_abi_version() -> int:
    return load().fp8blk_abi_version()


def fp8blk_strerror(status: int) -> str:
    return load().fp8blk_strerror(status).decode()


def fp8blk_workspace_bytes(op: int, rows: int, cols: int, M: int = 1) -> int:
    return load().fp8blk_workspace_bytes(op, rows, cols, M)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtypes, name):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _bf16_dtypes():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


# Shape checks. The C ABI takes plain pointers and sizes and cannot see how
# large a buffer is, so every wrapper checks here, before any launch, that
# each tensor holds exactly what the shapes it passes imply and that all of
# them are on one device; a mismatch raises ValueError.

def _grid_cells(rows, cols):
    return (-(-rows // 128)) * (-(-cols // 128))


def _weights(w, name="codes"):
    if w.dim() != 2:
        raise ValueError(f"{name} must be a 2-D [rows, cols] tensor, got shape {tuple(w.shape)}")
    return w.shape


def _numel(t, n, name, what):
    if t is not None and t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements ({what}), it holds {t.numel()}")


def _one_device(*ts):
    devs = {str(t.device) for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(devs)}")


def _panel(x, rows, cols, y, xname="x_bf16"):
    """x is [M, cols] and y holds M * rows elements; returns M."""
    if x.dim() != 2 or x.shape[1] != cols:
        raise ValueError(f"{xname} must be [M, cols={cols}], got shape {tuple(x.shape)}")
    M = x.shape[0]
    _numel(y, M * rows, "y", f"[M={M}, rows={rows}]")
    return M


def _check_linear(w, grid, x, y, wname="codes"):
    """A linear's weights [rows, cols], f32 grid (FP8 arms; None for a slab),
    panel x [M, cols] and output y [M, rows]; returns (rows, cols, M)."""
    rows, cols = _weights(w, wname)
    if grid is not None:
        _numel(grid, _grid_cells(rows, cols), "scales_f32", "the ceil(rows/128) x ceil(cols/128) grid")
    M = _panel(x, rows, cols, y)
    _one_device(w, grid, x, y)
    return rows, cols, M


def _ws(ws):
    if ws is None:
        return None, 0
    return _dev(ws, None, "ws"), ws.numel() * ws.element_size()


def fp8blk_load_check(codes, scales_e8m0, scales_f32_out, ws, stream=None, check=True):
    """Validate codes/scales and decode the f32 scale grid. Waits on the stream.
    Returns (status, first_bad); raises Fp8BlkError on a refusal if check."""
    import torch
    rows, cols = _weights(codes)
    _numel(scales_e8m0, _grid_cells(rows, cols), "scales_e8m0", "the block grid")
    _numel(scales_f32_out, _grid_cells(rows, cols), "scales_f32_out", "the block grid")
    _one_device(codes, scales_e8m0, scales_f32_out, ws)
    wsp, wsb = _ws(ws)
    fb = ctypes.c_int64(-1)
    st = load().fp8blk_load_check(_dev(codes, (torch.uint8,), "codes"),
                                  _dev(scales_e8m0, (torch.uint8,), "scales_e8m0"), rows, cols,
                                  _dev(scales_f32_out, (torch.float32,), "scales_f32_out"), wsp, wsb,
                                  ctypes.byref(fb), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_load_check", fb.value)
    return st, fb.value


def fp8blk_load_check_noalloc(codes, scales_e8m0, scales_f32_out, stream=None, check=True):
    """fp8blk_load_check with the library's static scratch instead of a
    workspace: allocates nothing. Calls that overlap on one GPU race.
    Returns (status, first_bad); raises Fp8BlkError on a refusal if check."""
    import torch
    rows, cols = _weights(codes)
    _numel(scales_e8m0, _grid_cells(rows, cols), "scales_e8m0", "the block grid")
    _numel(scales_f32_out, _grid_cells(rows, cols), "scales_f32_out", "the block grid")
    _one_device(codes, scales_e8m0, scales_f32_out)
    fb = ctypes.c_int64(-1)
    st = load().fp8blk_load_check_noalloc(_dev(codes, (torch.uint8,), "codes"),
                                          _dev(scales_e8m0, (torch.uint8,), "scales_e8m0"), rows, cols,
                                          _dev(scales_f32_out, (torch.float32,), "scales_f32_out"),
                                          ctypes.byref(fb), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_load_check_noalloc", fb.value)
    return st, fb.value


def fp8blk_dequant_bf16(codes, scales_f32, out_bf16, stream=None, check=True):
    import torch
    rows, cols = _weights(codes)
    _numel(scales_f32, _grid_cells(rows, cols), "scales_f32", "the block grid")
    _numel(out_bf16, rows * cols, "out_bf16", f"[rows={rows}, cols={cols}]")
    _one_device(codes, scales_f32, out_bf16)
    st = load().fp8blk_dequant_bf16(_dev(codes, (torch.uint8,), "codes"),
                                    _dev(scales_f32, (torch.float32,), "scales_f32"), rows, cols,
                                    _dev(out_bf16, _bf16_dtypes(), "out_bf16"), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_dequant_bf16")
    return st


def fp8blk_gemv(codes, scales_f32, x_bf16, y, ws=None, stream=None, check=True):
    """y[M, rows] = decode(codes, scales) @ x^T, in the library's fixed order."""
    import torch
    rows, cols, M = _check_linear(codes, scales_f32, x_bf16, y)
    _one_device(codes, ws)
    wsp, wsb = _ws(ws)
    st = load().fp8blk_gemv(_dev(codes, (torch.uint8,), "codes"),
                            _dev(scales_f32, (torch.float32,), "scales_f32"), rows, cols,
                            _dev(x_bf16, _bf16_dtypes(), "x_bf16"), M,
                            _dev(y, (torch.float32,), "y"), wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv")
    return st


def bf16_gemv_twin(w_bf16, x_bf16, y, ws=None, stream=None, check=True):
    """The bf16-slab twin of fp8blk_gemv (same order, same bits)."""
    import torch
    rows, cols, M = _check_linear(w_bf16, None, x_bf16, y, "w_bf16")
    _one_device(w_bf16, ws)
    wsp, wsb = _ws(ws)
    st = load().bf16_gemv_twin(_dev(w_bf16, _bf16_dtypes(), "w_bf16"), rows, cols,
                               _dev(x_bf16, _bf16_dtypes(), "x_bf16"), M,
                               _dev(y, (torch.float32,), "y"), wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "bf16_gemv_twin")
    return st


def _group(members, fp8, x):
    import torch
    arr = (Linear * len(members))()
    cols = None
    for k, mem in enumerate(members):
        w, grid, y = mem if fp8 else (mem[0], None, mem[1])
        rows, c = _weights(w, "w")
        cols = c if cols is None else cols
        if c != cols:
            raise ValueError("grouped linears must share cols")
        _check_linear(w, grid, x, y, "w")
        arr[k].w = _dev(w, (torch.uint8,) if fp8 else _bf16_dtypes(), "w")
        arr[k].scales_f32 = _dev(grid, (torch.float32,), "scales_f32") if fp8 else None
        arr[k].rows = rows
        arr[k].y = _dev(y, (torch.float32,), "y")
    return arr, cols


def _scaled(members, src_f32):
    """Descriptors of FP8 linears [(codes, scales_f32, y), ...] that read
    x = bf16(c * src_f32) (M = 1, y of rows values), and src's pointer."""
    import torch
    arr = (Linear * len(members))()
    cols = None
    for k, (w, grid, y) in enumerate(members):
        rows, c = _weights(w, "codes")
        cols = c if cols is None else cols
        if c != cols:
            raise ValueError("grouped linears must share cols")
        _numel(grid, _grid_cells(rows, cols), "scales_f32", "the ceil(rows/128) x ceil(cols/128) grid")
        _numel(y, rows, "y", "rows outputs (one activation row)")
        _one_device(w, grid, y, src_f32)
        arr[k].w = _dev(w, (torch.uint8,), "codes")
        arr[k].scales_f32 = _dev(grid, (torch.float32,), "scales_f32")
        arr[k].rows = rows
        arr[k].y = _dev(y, (torch.float32,), "y")
    _numel(src_f32, cols, "src_f32", "cols values")
    return arr, cols, _dev(src_f32, (torch.float32,), "src_f32")


def fp8blk_gemv_scaled_input(codes, scales_f32, src_f32, c, y, stream=None, check=True):
    """y[rows] = fp8blk_gemv on x = bf16(c * src_f32) (one activation row),
    the conversion done inside the kernel's x loads (same bits)."""
    arr, cols, srcp = _scaled([(codes, scales_f32, y)], src_f32)
    st = load().fp8blk_gemv_scaled_input(arr[0].w, arr[0].scales_f32, arr[0].rows, cols, srcp, float(c), arr[0].y,
                                         _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_scaled_input")
    return st


def fp8blk_gemv_grouped_scaled_input(members, src_f32, c, stream=None, check=True):
    """fp8blk_gemv_grouped on x = bf16(c * src_f32), formed in the kernel."""
    arr, cols, srcp = _scaled(members, src_f32)
    st = load().fp8blk_gemv_grouped_scaled_input(arr, len(members), cols, srcp, float(c), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_grouped_scaled_input")
    return st


def _next(members, x_bf16, k, x_next):
    """Descriptors for a next-input launch (M = 1): x_next holds rows of
    linear k bf16 values."""
    import torch
    arr, cols = _group(members, True, x_bf16)
    if x_bf16.shape[0] != 1:
        raise ValueError("a next-input launch takes one activation row")
    if not 0 <= k < len(members):
        raise ValueError(f"k = {k} names no linear of the group")
    _numel(x_next, arr[k].rows, "x_next", "the rows of linear k")
    _one_device(x_bf16, x_next)
    return arr, cols, _dev(x_next, _bf16_dtypes(), "x_next")


def fp8blk_gemv_next_input(codes, scales_f32, x_bf16, y, c, x_next, stream=None, check=True):
    """fp8blk_gemv at M = 1 that also writes x_next = bf16(c * y)."""
    arr, cols, xnp = _next([(codes, scales_f32, y)], x_bf16, 0, x_next)
    st = load().fp8blk_gemv_next_input(arr[0].w, arr[0].scales_f32, arr[0].rows, cols,
                                       _dev(x_bf16, _bf16_dtypes(), "x_bf16"), arr[0].y, float(c), xnp,
                                       _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_next_input")
    return st


def fp8blk_gemv_grouped_next_input(members, x_bf16, k, c, x_next, stream=None, check=True):
    """fp8blk_gemv_grouped at M = 1; linear k also writes x_next = bf16(c * y_k)."""
    arr, cols, xnp = _next(members, x_bf16, k, x_next)
    st = load().fp8blk_gemv_grouped_next_input(arr, len(members), cols, _dev(x_bf16, _bf16_dtypes(), "x_bf16"), k,
                                               float(c), xnp, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_grouped_next_input")
    return st


def fp8blk_gemv_grouped(members, x_bf16, stream=None, check=True):
    """One launch for [(codes, scales_f32, y), ...] sharing x (same bits as
    separate fp8blk_gemv calls)."""
    arr, cols = _group(members, True, x_bf16)
    st = load().fp8blk_gemv_grouped(arr, len(members), cols, _dev(x_bf16, _bf16_dtypes(), "x_bf16"),
                                    x_bf16.shape[0], _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_grouped")
    return st


def bf16_gemv_twin_grouped(members, x_bf16, stream=None, check=True):
    """One launch for [(w_bf16, y), ...] sharing x."""
    arr, cols = _group(members, False, x_bf16)
    st = load().bf16_gemv_twin_grouped(arr, len(members), cols, _dev(x_bf16, _bf16_dtypes(), "x_bf16"),
                                       x_bf16.shape[0], _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "bf16_gemv_twin_grouped")
    return st


def fp8blk_gemv_mfma(codes, scales_f32, x_bf16, y, stream=None, check=True):
    """Matrix-core arm of fp8blk_gemv (bitwise twin of bf16_gemv_twin_mfma)."""
    import torch
    rows, cols, _M = _check_linear(codes, scales_f32, x_bf16, y)
    st = load().fp8blk_gemv_mfma(_dev(codes, (torch.uint8,), "codes"),
                                 _dev(scales_f32, (torch.float32,), "scales_f32"), rows, cols,
                                 _dev(x_bf16, _bf16_dtypes(), "x_bf16"), x_bf16.shape[0],
                                 _dev(y, (torch.float32,), "y"), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_mfma")
    return st


def bf16_gemv_twin_mfma(w_bf16, x_bf16, y, stream=None, check=True):
    import torch
    rows, cols, _M = _check_linear(w_bf16, None, x_bf16, y, "w_bf16")
    st = load().bf16_gemv_twin_mfma(_dev(w_bf16, _bf16_dtypes(), "w_bf16"), rows, cols,
                                    _dev(x_bf16, _bf16_dtypes(), "x_bf16"), x_bf16.shape[0],
                                    _dev(y, (torch.float32,), "y"), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "bf16_gemv_twin_mfma")
    return st


def fp8blk_sequence_bytes(n: int) -> int:
    return load().fp8blk_sequence_bytes(n)


class Sequence:
    """A planned sequence launch (fp8blk_sequence_init): the plan lives in
    `ws` (a device byte tensor this object keeps alive) and `handle` is the
    host record the launch entry points take. `keep` holds the tensors whose
    addresses the plan records."""

    def __init__(self, handle, ws, keep):
        self.handle = handle
        self.ws = ws
        self.keep = keep


def fp8blk_sequence_init(arm: int, linears, ws=None, stream=None, check=True):
    """Plan a sequence launch over independent linears.
    linears: [(codes, scales_f32, x_bf16, y), ...] for ARM_FP8 / ARM_FP8_MFMA,
             [(w_bf16, x_bf16, y), ...] for ARM_BF16 / ARM_BF16_MFMA;
             x_bf16 is [M, cols] and y is [M, rows] (M = 1 on the vector arms,
             and the same M for every linear).
    ws: a device uint8 tensor of at least fp8blk_sequence_bytes(n) bytes, or
        None to allocate one here. Waits for the plan's copy to the device."""
    import torch
    n = len(linears)
    arr = (SeqLinear * max(n, 1))()
    keep = []
    fp8 = arm in (ARM_FP8, ARM_FP8_MFMA)
    for k, lin in enumerate(linears):
        w, grid, x, y = lin if fp8 else (lin[0], None, lin[1], lin[2])
        try:
            rows, cols, M = _check_linear(w, grid, x, y, "w")
        except ValueError as e:
            raise ValueError(f"linear {k}: {e}") from None
        if fp8:
            arr[k].w = _dev(w, (torch.uint8,), "codes")
            arr[k].scales_f32 = _dev(grid, (torch.float32,), "scales_f32")
        else:
            arr[k].w = _dev(w, _bf16_dtypes(), "w_bf16")
            arr[k].scales_f32 = None
        arr[k].rows, arr[k].cols, arr[k].M = rows, cols, M
        arr[k].x_bf16 = _dev(x, _bf16_dtypes(), "x_bf16")
        arr[k].y = _dev(y, (torch.float32,), "y")
        keep.append((w, grid, x, y))
    if ws is None:
        nb = fp8blk_sequence_bytes(n) if 1 <= n <= MAX_SEQ else 64
        ws = torch.empty(max(nb, 64), dtype=torch.uint8, device=(linears[0][0].device if n else "cuda"))
    wsp, wsb = _ws(ws)
    h = SequenceHandle()
    st = load().fp8blk_sequence_init(ctypes.byref(h), arm, arr, n, wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_sequence_init")
    return Sequence(h, ws, keep) if st == OK else st


class Chain:
    """A planned chained launch (fp8blk_chain_init): the plan, the hand-off
    words and the control words live in `ws` (a device byte tensor this object
    keeps alive); `handle` is the host record; `keep` holds the tensors whose
    addresses the plan records."""

    def __init__(self, handle, ws, keep):
        self.handle = handle
        self.ws = ws
        self.keep = keep


def _chain_arrays(groups):
    """groups: [(members, src, c), ...] with members [(codes, scales_f32, y), ...]
    and src None (the chain input) or (g, k): member k of an earlier group g.
    Returns the C arrays and the tensors they point at."""
    import torch
    lins, gs, keep = [], [], []
    first = []
    for gi, (members, src, c) in enumerate(groups):
        if not members:
            raise ValueError(f"group {gi}: no linears")
        first.append(len(lins))
        cols = None
        for k, (w, grid, y) in enumerate(members):
            if w.dim() != 2:
                raise ValueError(f"group {gi} linear {k}: codes must be [rows, cols]")
            rows, wc = int(w.shape[0]), int(w.shape[1])
            cols = wc if cols is None else cols
            if wc != cols:
                raise ValueError(f"group {gi} linear {k}: cols {wc} differs from the group's {cols}")
            if y.numel() != rows:
                raise ValueError(f"group {gi} linear {k}: y holds {y.numel()} values, expected {rows}")
            want = (-(-rows // 128)) * (-(-cols // 128))
            if grid.numel() != want:
                raise ValueError(f"group {gi} linear {k}: scale grid holds {grid.numel()} values, expected {want}")
            lins.append((_dev(w, (torch.uint8,), "codes"), _dev(grid, (torch.float32,), "scales_f32"), rows,
                         _dev(y, (torch.float32,), "y")))
            keep.append((w, grid, y))
        if src is None:
            s = -1
        else:
            sg, sk = src
            if not (0 <= sg < gi) or not (0 <= sk < len(groups[sg][0])):
                raise ValueError(f"group {gi}: src {src} is not a linear of an earlier group")
            s = first[sg] + sk
        gs.append((first[-1], len(members), cols, s, float(c)))
    devs = {t.device for trio in keep for t in trio}
    if len(devs) != 1:
        raise ValueError(f"the chain's tensors lie on {len(devs)} devices")
    la = (Linear * len(lins))()
    for k, (w, grid, rows, y) in enumerate(lins):
        la[k].w, la[k].scales_f32, la[k].rows, la[k].y = w, grid, rows, y
    ga = (ChainGroup * len(gs))()
    for k, (f, n, cols, s, c) in enumerate(gs):
        ga[k].first, ga[k].n, ga[k].cols, ga[k].src, ga[k].c = f, n, cols, s, c
    x0_cols = max([g[2] for g in gs if g[3] < 0], default=0)
    return la, len(lins), ga, len(gs), (keep, x0_cols)


def fp8blk_chain_bytes(groups) -> int:
    """Workspace bytes of a chained launch over `groups` (see fp8blk_chain_init);
    0 if the library refuses the list."""
    la, nl, ga, ng, _ = _chain_arrays(groups)
    return int(load().fp8blk_chain_bytes(la, nl, ga, ng))


def fp8blk_chain_init(groups, ws=None, stream=None, check=True):
    """Plan a chained launch.
    groups: [(members, src, c), ...] in order; members [(codes, scales_f32, y), ...]
            share cols (1024, 2048, 3072 or 4096) and one input: the chain
            input x0 (src None) or bf16(c * y) of member k of an earlier group g
            (src (g, k)).
    ws: a device uint8 tensor of at least fp8blk_chain_bytes(groups) bytes
        (256-byte aligned), or None to allocate one here. Waits for `stream`."""
    import torch
    la, nl, ga, ng, (keep, x0_cols) = _chain_arrays(groups)
    if ws is None:
        nb = int(load().fp8blk_chain_bytes(la, nl, ga, ng))
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=groups[0][0][0][0].device)
    wsp, wsb = _ws(ws)
    h = ChainHandle()
    st = load().fp8blk_chain_init(ctypes.byref(h), la, nl, ga, ng, wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_chain_init")
    if st != OK:
        return st
    ch = Chain(h, ws, keep)
    ch.x0_cols = x0_cols
    ch.device = keep[0][0].device
    return ch


def fp8blk_gemv_chain(chain, x0_bf16, stream=None, check=True):
    """One cooperative launch of the whole chained list on x0 ([cols] bf16 of
    the first group)."""
    import torch
    if x0_bf16.dtype not in _bf16_dtypes() or not x0_bf16.is_contiguous():
        raise ValueError("x0_bf16 must be a contiguous bf16 (or int16/uint16) tensor")
    if x0_bf16.numel() < chain.x0_cols:
        raise ValueError(f"x0_bf16 holds {x0_bf16.numel()} values, the chain reads {chain.x0_cols}")
    if x0_bf16.device != chain.device:
        raise ValueError("x0_bf16 lies on another device than the chain")
    st = load().fp8blk_gemv_chain(ctypes.byref(chain.handle), _dev(x0_bf16, _bf16_dtypes(), "x0_bf16"),
                                  _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_chain")
    return st


def fp8blk_chain_status(chain, stream=None) -> int:
    """Wait for `stream`; FP8BLK_OK, or ERR_TIMEOUT if a launch since the last
    check stopped waiting for an input (the record is then cleared)."""
    return int(load().fp8blk_chain_status(ctypes.byref(chain.handle), _stream(stream)))


def fp8blk_gemv_sequence(seq, stream=None, check=True):
    """One persistent launch of every linear of an ARM_FP8 sequence."""
    st = load().fp8blk_gemv_sequence(ctypes.byref(seq.handle), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_sequence")
    return st


def bf16_gemv_twin_sequence(seq, stream=None, check=True):
    """One persistent launch of every linear of an ARM_BF16 sequence."""
    st = load().bf16_gemv_twin_sequence(ctypes.byref(seq.handle), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "bf16_gemv_twin_sequence")
    return st


def fp8blk_gemv_mfma_sequence(seq, stream=None, check=True):
    """One persistent launch of every linear of an ARM_FP8_MFMA sequence."""
    st = load().fp8blk_gemv_mfma_sequence(ctypes.byref(seq.handle), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemv_mfma_sequence")
    return st


def bf16_gemv_twin_mfma_sequence(seq, stream=None, check=True):
    """One persistent launch of every linear of an ARM_BF16_MFMA sequence."""
    st = load().bf16_gemv_twin_mfma_sequence(ctypes.byref(seq.handle), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "bf16_gemv_twin_mfma_sequence")
    return st


def fp8blk_gemm_staged(codes, scales_f32, x_bf16, y, ws, stream=None, check=True):
    """Prefill: y[N, rows] = x[N, cols] . dequant(codes, scales)^T via the bf16
    slab (written into ws) and one library GEMM. ws: fp8blk_workspace_bytes(
    OP_GEMM_STAGED, rows, cols, N) bytes, 256-byte aligned."""
    import torch
    rows, cols, _N = _check_linear(codes, scales_f32, x_bf16, y)
    _one_device(codes, ws)
    wsp, wsb = _ws(ws)
    st = load().fp8blk_gemm_staged(_dev(codes, (torch.uint8,), "codes"),
                                   _dev(scales_f32, (torch.float32,), "scales_f32"), rows, cols,
                                   _dev(x_bf16, _bf16_dtypes(), "x_bf16"), x_bf16.shape[0],
                                   _dev(y, (torch.float32,), "y"), wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_gemm_staged")
    return st


def bf16_gemm_twin(w_bf16, x_bf16, y, ws, stream=None, check=True):
    """The same GEMM over a bf16 slab the caller holds. ws: fp8blk_workspace_bytes(
    OP_BF16_GEMM, rows, cols, N) bytes, 256-byte aligned."""
    import torch
    rows, cols, _N = _check_linear(w_bf16, None, x_bf16, y, "w_bf16")
    _one_device(w_bf16, ws)
    wsp, wsb = _ws(ws)
    st = load().bf16_gemm_twin(_dev(w_bf16, _bf16_dtypes(), "w_bf16"), rows, cols,
                               _dev(x_bf16, _bf16_dtypes(), "x_bf16"), x_bf16.shape[0],
                               _dev(y, (torch.float32,), "y"), wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "bf16_gemm_twin")
    return st


# --- native expert arm ---------------------------------------------------------

def fp8blk_act_quant(x_bf16, xq, xs, stream=None, check=True):
    """act_quant: x [M, cols] bf16 -> xq [M, cols] e4m3 codes, xs [M, ceil(cols/128)]
    e8m0 scale codes (uint8 tensors)."""
    import torch
    if x_bf16.dim() != 2:
        raise ValueError(f"x_bf16 must be [M, cols], got shape {tuple(x_bf16.shape)}")
    M, cols = x_bf16.shape
    _numel(xq, M * cols, "xq", f"[M={M}, cols={cols}]")
    _numel(xs, M * (-(-cols // 128)), "xs", f"[M={M}, ceil(cols/128)]")
    _one_device(x_bf16, xq, xs)
    st = load().fp8blk_act_quant(_dev(x_bf16, _bf16_dtypes(), "x_bf16"), M, cols, _dev(xq, (torch.uint8,), "xq"),
                                 _dev(xs, (torch.uint8,), "xs"), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp8blk_act_quant")
    return st


def _fp4_slab(fmt, codes, scales):
    """FP4 codes [rows, cols/2] and block scales [rows, cols/B]; returns (rows, cols)."""
    rows, half = _weights(codes)
    cols = 2 * half
    B = {FMT_MXFP4: 32, FMT_NVFP4: 16}.get(fmt)
    if B is not None:
        _numel(scales, rows * (cols // B), "scales", f"[rows={rows}, cols/{B}]")
    _one_device(codes, scales)
    return rows, cols


def fp4_load_check(fmt, codes, scales, ws, stream=None, check=True):
    """Validate an FP4 slab (codes [rows, cols/2], scales [rows, cols/B]).
    Waits on the stream. Returns (status, first_bad)."""
    import torch
    rows, cols = _fp4_slab(fmt, codes, scales)
    _one_device(codes, ws)
    wsp, wsb = _ws(ws)
    fb = ctypes.c_int64(-1)
    st = load().fp4_load_check(fmt, _dev(codes, (torch.uint8,), "codes"), _dev(scales, (torch.uint8,), "scales"),
                               rows, cols, wsp, wsb, ctypes.byref(fb), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp4_load_check", fb.value)
    return st, fb.value


def fp4_dequant_bf16(fmt, codes, scales, out_bf16, stream=None, check=True):
    """The bf16-dequant arm's exact slab [rows, cols]."""
    import torch
    rows, cols = _fp4_slab(fmt, codes, scales)
    _numel(out_bf16, rows * cols, "out_bf16", f"[rows={rows}, cols={cols}]")
    _one_device(codes, out_bf16)
    st = load().fp4_dequant_bf16(fmt, _dev(codes, (torch.uint8,), "codes"), _dev(scales, (torch.uint8,), "scales"),
                                 rows, cols, _dev(out_bf16, _bf16_dtypes(), "out_bf16"), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp4_dequant_bf16")
    return st


def fp4_expert_gemv(fmt, codes, scales, global_scale, xq, xs, y, stream=None, check=True):
    """Native expert GEMV: y[M, rows] = g * act(xq, xs) @ fp4(codes, scales)^T."""
    import torch
    rows, cols = _fp4_slab(fmt, codes, scales)
    M = _panel(xq, rows, cols, y, "xq")
    _numel(xs, M * (-(-cols // 128)), "xs", f"[M={M}, ceil(cols/128)]")
    _one_device(codes, xq, xs, y)
    st = load().fp4_expert_gemv(fmt, _dev(codes, (torch.uint8,), "codes"), _dev(scales, (torch.uint8,), "scales"),
                                float(global_scale), rows, cols, _dev(xq, (torch.uint8,), "xq"),
                                _dev(xs, (torch.uint8,), "xs"), xq.shape[0], _dev(y, (torch.float32,), "y"),
                                _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp4_expert_gemv")
    return st


def fp4_expert_sequence_init(fmt, linears, ws=None, stream=None, check=True):
    """Plan one launch over expert linears [(codes, scales, global_scale, xq, xs, y), ...]
    (the same M for all). ws: a device uint8 tensor of at least
    fp8blk_sequence_bytes(n) bytes, or None to allocate one here."""
    import torch
    n = len(linears)
    arr = (Fp4ExpertLinear * max(n, 1))()
    keep = []
    for k, (codes, scales, g, xq, xs, y) in enumerate(linears):
        try:
            rows, cols = _fp4_slab(fmt, codes, scales)
            M = _panel(xq, rows, cols, y, "xq")
            _numel(xs, M * (-(-cols // 128)), "xs", f"[M={M}, ceil(cols/128)]")
            _one_device(codes, xq, xs, y)
        except ValueError as e:
            raise ValueError(f"linear {k}: {e}") from None
        arr[k].codes = _dev(codes, (torch.uint8,), "codes")
        arr[k].scales = _dev(scales, (torch.uint8,), "scales")
        arr[k].global_scale = float(g)
        arr[k].rows, arr[k].cols, arr[k].M = rows, cols, M
        arr[k].xq = _dev(xq, (torch.uint8,), "xq")
        arr[k].xs = _dev(xs, (torch.uint8,), "xs")
        arr[k].y = _dev(y, (torch.float32,), "y")
        keep.append((codes, scales, xq, xs, y))
    if ws is None:
        nb = fp8blk_sequence_bytes(n) if 1 <= n <= MAX_SEQ else 64
        ws = torch.empty(max(nb, 64), dtype=torch.uint8, device=(linears[0][0].device if n else "cuda"))
    wsp, wsb = _ws(ws)
    h = SequenceHandle()
    st = load().fp4_expert_sequence_init(ctypes.byref(h), fmt, arr, n, wsp, wsb, _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp4_expert_sequence_init")
    return Sequence(h, ws, keep) if st == OK else st


def fp4_expert_sequence(seq, stream=None, check=True):
    """One persistent launch of every linear of an expert sequence."""
    st = load().fp4_expert_sequence(ctypes.byref(seq.handle), _stream(stream))
    if check and st != OK:
        raise Fp8BlkError(st, "fp4_expert_sequence")
    return st


def raw_call(name: str, *args):
    """Call an exported symbol with raw ctypes arguments (pointers as ints).
    Used by tests that exercise the C ABI's argument checks directly."""
    return getattr(load(), name)(*args)


def prepared(name: str, *tensors_and_sizes, stream=None):
    """Marshal an entry point's arguments once and return a zero-argument
    callable that enqueues it and returns its status. For launch-bound loops
    (benchmarks, graph capture), where per-call tensor inspection would
    dominate. Supported: "fp8blk_gemv" and "fp8blk_gemv_mfma" (codes,
    scales_f32, x_bf16, y), "bf16_gemv_twin" and "bf16_gemv_twin_mfma" (w_bf16,
    x_bf16, y), the grouped launches (members, x_bf16), the scaled-input
    launches (codes, scales_f32, src_f32, c, y) and (members, src_f32, c), the
    next-input launches (codes, scales_f32, x_bf16, y, c, x_next) and
    (members, x_bf16, k, c, x_next), the staged GEMMs (..., ws) and the sequence launches (a planned Sequence)."""
    import torch
    fn = getattr(load(), name)
    s = _stream(stream)
    if name == "fp8blk_gemv":
        codes, grid, x, y = tensors_and_sizes
        rows, cols, _M = _check_linear(codes, grid, x, y)
        args = (_dev(codes, (torch.uint8,), "codes"), _dev(grid, (torch.float32,), "scales_f32"), rows, cols,
                _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0], _dev(y, (torch.float32,), "y"), None, 0, s)
    elif name == "bf16_gemv_twin":
        w, x, y = tensors_and_sizes
        rows, cols, _M = _check_linear(w, None, x, y, "w_bf16")
        args = (_dev(w, _bf16_dtypes(), "w_bf16"), rows, cols, _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0],
                _dev(y, (torch.float32,), "y"), None, 0, s)
    elif name == "fp8blk_gemv_mfma":
        codes, grid, x, y = tensors_and_sizes
        rows, cols, _M = _check_linear(codes, grid, x, y)
        args = (_dev(codes, (torch.uint8,), "codes"), _dev(grid, (torch.float32,), "scales_f32"), rows, cols,
                _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0], _dev(y, (torch.float32,), "y"), s)
    elif name == "bf16_gemv_twin_mfma":
        w, x, y = tensors_and_sizes
        rows, cols, _M = _check_linear(w, None, x, y, "w_bf16")
        args = (_dev(w, _bf16_dtypes(), "w_bf16"), rows, cols, _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0],
                _dev(y, (torch.float32,), "y"), s)
    elif name in ("fp8blk_gemv_grouped", "bf16_gemv_twin_grouped"):
        members, x = tensors_and_sizes
        arr, cols = _group(members, name == "fp8blk_gemv_grouped", x)
        args = (arr, len(members), cols, _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0], s)
    elif name == "fp8blk_gemv_scaled_input":
        codes, grid, src, c, y = tensors_and_sizes
        arr, cols, srcp = _scaled([(codes, grid, y)], src)
        args = (arr[0].w, arr[0].scales_f32, arr[0].rows, cols, srcp, float(c), arr[0].y, s)
    elif name == "fp8blk_gemv_grouped_scaled_input":
        members, src, c = tensors_and_sizes
        arr, cols, srcp = _scaled(members, src)
        args = (arr, len(members), cols, srcp, float(c), s)
    elif name == "fp8blk_gemv_next_input":
        codes, grid, x, y, c, xn = tensors_and_sizes
        arr, cols, xnp = _next([(codes, grid, y)], x, 0, xn)
        args = (arr[0].w, arr[0].scales_f32, arr[0].rows, cols, _dev(x, _bf16_dtypes(), "x_bf16"), arr[0].y,
                float(c), xnp, s)
    elif name == "fp8blk_gemv_grouped_next_input":
        members, x, k, c, xn = tensors_and_sizes
        arr, cols, xnp = _next(members, x, k, xn)
        args = (arr, len(members), cols, _dev(x, _bf16_dtypes(), "x_bf16"), k, float(c), xnp, s)
    elif name == "fp8blk_gemm_staged":
        codes, grid, x, y, ws = tensors_and_sizes
        rows, cols, _N = _check_linear(codes, grid, x, y)
        _one_device(codes, ws)
        wsp, wsb = _ws(ws)
        args = (_dev(codes, (torch.uint8,), "codes"), _dev(grid, (torch.float32,), "scales_f32"), rows, cols,
                _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0], _dev(y, (torch.float32,), "y"), wsp, wsb, s)
    elif name == "bf16_gemm_twin":
        w, x, y, ws = tensors_and_sizes
        rows, cols, _N = _check_linear(w, None, x, y, "w_bf16")
        _one_device(w, ws)
        wsp, wsb = _ws(ws)
        args = (_dev(w, _bf16_dtypes(), "w_bf16"), rows, cols, _dev(x, _bf16_dtypes(), "x_bf16"), x.shape[0],
                _dev(y, (torch.float32,), "y"), wsp, wsb, s)
    elif name in ("fp8blk_gemv_sequence", "bf16_gemv_twin_sequence", "fp8blk_gemv_mfma_sequence",
                  "bf16_gemv_twin_mfma_sequence", "fp4_expert_sequence"):
        (seq,) = tensors_and_sizes
        args = (ctypes.byref(seq.handle), s)
    else:
        raise ValueError(f"prepared: unsupported entry point {name!r}")
    return lambda: fn(*args)
