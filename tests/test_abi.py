"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-only logic (status text, workspace sizes, argument
refusals that return before any device work) behaves as documented."""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_fp8blk_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_0-9]+)\s*\([^;{]*\)\s*;", text))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return fb.load()


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    assert {"fp8blk_load_check", "fp8blk_dequant_bf16", "fp8blk_gemv", "bf16_gemv_twin"} <= names
    assert names == set(fb.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # C linkage: the names are not mangled
    out = os.popen(f"nm -D --defined-only {fb.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_host_helpers(lib):
    assert fb.fp8blk_abi_version() == 1
    for st in range(9):
        assert fb.fp8blk_strerror(st) != "unknown status"
    assert fb.fp8blk_strerror(99) == "unknown status"
    assert fb.fp8blk_workspace_bytes(fb.OP_LOAD_CHECK, 4096, 4096) >= 24
    assert fb.fp8blk_workspace_bytes(fb.OP_GEMV, 4096, 4096, 16) == 0
    assert fb.fp8blk_workspace_bytes(77, 1, 16) == 0
    # the staged prefill GEMM: the bf16 slab (256-byte aligned size) plus 32 MB for the library GEMM
    lt = 32 << 20
    assert fb.fp8blk_workspace_bytes(fb.OP_BF16_GEMM, 4096, 4096, 2048) == lt
    assert fb.fp8blk_workspace_bytes(fb.OP_GEMM_STAGED, 4096, 4096, 2048) == 2 * 4096 * 4096 + lt
    assert fb.fp8blk_workspace_bytes(fb.OP_GEMM_STAGED, 3, 16, 1) == 256 + lt
    assert fb.fp8blk_workspace_bytes(fb.OP_GEMM_STAGED, 0, 16, 1) == 0


P = 1 << 12  # a fake, 4096-aligned address: never dereferenced, every call below refuses first


@pytest.mark.parametrize("rows,cols,M", [(0, 16, 1), (4, 8, 1), (4, 24, 1), (4, 65552, 1),
                                         (4, 16, 0), (4, 16, 17), (-1, 16, 1)])
def test_gemv_refuses_bad_shapes(lib, rows, cols, M):
    assert lib.fp8blk_gemv(P, P, rows, cols, P, M, P, None, 0, None) == fb.ERR_ARG
    assert lib.bf16_gemv_twin(P, rows, cols, P, M, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_mfma(P, P, rows, cols, P, M, P, None) == fb.ERR_ARG
    assert lib.bf16_gemv_twin_mfma(P, rows, cols, P, M, P, None) == fb.ERR_ARG


def test_refuses_null_and_misaligned_pointers(lib):
    assert lib.fp8blk_gemv(None, P, 4, 16, P, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(P, None, 4, 16, P, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(P, P, 4, 16, None, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(P, P, 4, 16, P, 1, None, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(P + 8, P, 4, 16, P, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(P, P, 4, 16, P + 2, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv(P, P + 2, 4, 16, P, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.bf16_gemv_twin(P + 4, 4, 16, P, 1, P, None, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_dequant_bf16(P, P, 4, 16, P + 8, None) == fb.ERR_ARG
    assert lib.fp8blk_dequant_bf16(None, P, 4, 16, P, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_mfma(None, P, 4, 16, P, 1, P, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_mfma(P, None, 4, 16, P, 1, P, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_mfma(P + 8, P, 4, 16, P, 1, P, None) == fb.ERR_ARG


def test_load_check_refuses_before_device_work(lib):
    fb_idx = ctypes.c_int64(123)
    assert lib.fp8blk_load_check(P, P, 4, 17, P, P, 256, ctypes.byref(fb_idx), None) == fb.ERR_ARG
    assert fb_idx.value == -1
    assert lib.fp8blk_load_check(P, P, 4, 16, P, None, 256, None, None) == fb.ERR_WORKSPACE
    assert lib.fp8blk_load_check(P, P, 4, 16, P, P, 8, None, None) == fb.ERR_WORKSPACE
    assert lib.fp8blk_load_check(P, P, 4, 16, P, P + 4, 256, None, None) == fb.ERR_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fb, "_lib", None)
    monkeypatch.setattr(fb, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fb.load()


def test_grouped_refusals(lib):
    L = fb.Linear
    good = (L * 2)(L(P, P, 4, P), L(P, P, 4, P))
    assert lib.fp8blk_gemv_grouped(good, 0, 16, P, 1, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_grouped(good, 9, 16, P, 1, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_grouped(None, 1, 16, P, 1, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_grouped(good, 2, 24, P, 1, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_grouped(good, 2, 16, P, 0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_grouped(good, 2, 16, P + 2, 1, None) == fb.ERR_ARG
    bad = (L * 2)(L(P, P, 4, P), L(P + 8, P, 4, P))
    assert lib.fp8blk_gemv_grouped(bad, 2, 16, P, 1, None) == fb.ERR_ARG
    bad = (L * 2)(L(P, P, 4, P), L(P, None, 4, P))
    assert lib.fp8blk_gemv_grouped(bad, 2, 16, P, 1, None) == fb.ERR_ARG
    bad = (L * 2)(L(P, P, 0, P), L(P, P, 4, P))
    assert lib.bf16_gemv_twin_grouped(bad, 2, 16, P, 1, None) == fb.ERR_ARG
    bad = (L * 1)(L(P, P, 4, None))
    assert lib.bf16_gemv_twin_grouped(bad, 1, 16, P, 1, None) == fb.ERR_ARG


def test_sequence_refusals(lib):
    S = fb.SeqLinear
    h = fb.SequenceHandle()
    good = (S * 2)(S(P, P, 4, 16, 1, P, P), S(P, P, 4, 32, 1, P, P))
    nb = fb.fp8blk_sequence_bytes(2)
    assert nb >= 2 * 64 + 2 * 3 * 8
    assert fb.fp8blk_sequence_bytes(0) == 0 and fb.fp8blk_sequence_bytes(fb.MAX_SEQ + 1) == 0
    init = lib.fp8blk_sequence_init
    assert init(ctypes.byref(h), fb.ARM_FP8, good, 0, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), fb.ARM_FP8, good, fb.MAX_SEQ + 1, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), 4, good, 2, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), -1, good, 2, P, nb, None) == fb.ERR_ARG
    assert init(None, fb.ARM_FP8, good, 2, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), fb.ARM_FP8, None, 2, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), fb.ARM_FP8, good, 2, None, nb, None) == fb.ERR_WORKSPACE
    assert init(ctypes.byref(h), fb.ARM_FP8, good, 2, P, nb - 1, None) == fb.ERR_WORKSPACE
    assert init(ctypes.byref(h), fb.ARM_FP8, good, 2, P + 32, nb, None) == fb.ERR_WORKSPACE
    for bad in (S(P, P, 0, 16, 1, P, P), S(P, P, 4, 24, 1, P, P), S(P, P, 4, 65552, 1, P, P),
                S(P + 8, P, 4, 16, 1, P, P), S(P, P, 4, 16, 1, P + 2, P), S(P, P, 4, 16, 1, P, P + 2),
                S(None, P, 4, 16, 1, P, P), S(P, P, 4, 16, 1, None, P), S(P, P, 4, 16, 1, P, None),
                S(P, P, 4, 16, 2, P, P), S(P, P, 4, 16, 0, P, P)):
        arr = (S * 2)(good[0], bad)
        for arm in (fb.ARM_FP8, fb.ARM_BF16, fb.ARM_FP8_MFMA, fb.ARM_BF16_MFMA):
            assert init(ctypes.byref(h), arm, arr, 2, P, nb, None) == fb.ERR_ARG, (arm, bad.M)
    # the vector arms take M = 1 only; the matrix-core arms M <= 16, the same for all
    for M in (2, 16):
        arr = (S * 1)(S(P, P, 4, 16, M, P, P))
        assert init(ctypes.byref(h), fb.ARM_FP8, arr, 1, P, nb, None) == fb.ERR_ARG
        assert init(ctypes.byref(h), fb.ARM_BF16, arr, 1, P, nb, None) == fb.ERR_ARG
    arr = (S * 1)(S(P, P, 4, 16, 17, P, P))
    assert init(ctypes.byref(h), fb.ARM_FP8_MFMA, arr, 1, P, nb, None) == fb.ERR_ARG
    arr = (S * 2)(S(P, P, 4, 16, 4, P, P), S(P, P, 4, 16, 8, P, P))
    assert init(ctypes.byref(h), fb.ARM_FP8_MFMA, arr, 2, P, nb, None) == fb.ERR_ARG
    # the FP8 arms need the scale grid, the twin arms ignore it
    arr = (S * 1)(S(P, None, 4, 16, 1, P, P))
    assert init(ctypes.byref(h), fb.ARM_FP8, arr, 1, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), fb.ARM_FP8_MFMA, arr, 1, P, nb, None) == fb.ERR_ARG
    # a launch checks its handle before any device work
    h.plan, h.units_dense, h.units_general, h.n, h.arm, h.grid_dense, h.grid_general, h.M = \
        P, 10, 0, 2, fb.ARM_FP8, 4, 0, 1
    assert lib.bf16_gemv_twin_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_sequence(None, None) == fb.ERR_ARG
    h.arm = fb.ARM_BF16
    assert lib.fp8blk_gemv_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    h.arm, h.plan = fb.ARM_FP8, None
    assert lib.fp8blk_gemv_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    h.plan, h.units_dense, h.units_general = P, 0, 0
    assert lib.fp8blk_gemv_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    h.units_general, h.grid_general = 5, 0
    assert lib.fp8blk_gemv_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    # matrix-core launches check the arm and M
    h.plan, h.units_dense, h.units_general, h.grid_dense, h.grid_general, h.M = P, 10, 0, 4, 0, 16
    assert lib.fp8blk_gemv_mfma_sequence(ctypes.byref(h), None) == fb.ERR_ARG  # arm is ARM_FP8
    h.arm = fb.ARM_FP8_MFMA
    assert lib.bf16_gemv_twin_mfma_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    h.M = 17
    assert lib.fp8blk_gemv_mfma_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    h.M, h.units_dense = 16, 0
    assert lib.fp8blk_gemv_mfma_sequence(ctypes.byref(h), None) == fb.ERR_ARG


def test_gemm_refusals(lib):
    big = 1 << 40
    ws = fb.fp8blk_workspace_bytes(fb.OP_GEMM_STAGED, 4, 16, 1)
    assert lib.fp8blk_gemm_staged(P, P, 4, 16, P, 1, P, P, ws - 1, None) == fb.ERR_WORKSPACE
    assert lib.fp8blk_gemm_staged(P, P, 4, 16, P, 1, P, None, ws, None) == fb.ERR_WORKSPACE
    assert lib.fp8blk_gemm_staged(P, P, 4, 16, P, 1, P, P + 16, ws, None) == fb.ERR_WORKSPACE
    for bad in ((P, P, 4, 16, P, 0, P), (P, P, 4, 16, P, fb.MAX_PANEL + 1, P), (P, P, 4, 24, P, 1, P),
                (P + 8, P, 4, 16, P, 1, P), (P, None, 4, 16, P, 1, P), (P, P + 2, 4, 16, P, 1, P),
                (P, P, 4, 16, P + 8, 1, P), (P, P, 4, 16, P, 1, P + 4), (None, P, 4, 16, P, 1, P)):
        assert lib.fp8blk_gemm_staged(*bad, P, big, None) == fb.ERR_ARG, bad
    wt = fb.fp8blk_workspace_bytes(fb.OP_BF16_GEMM, 4, 16, 1)
    assert lib.bf16_gemm_twin(P, 4, 16, P, 1, P, P, wt - 1, None) == fb.ERR_WORKSPACE
    assert lib.bf16_gemm_twin(P, 4, 16, P, 0, P, P, wt, None) == fb.ERR_ARG
    assert lib.bf16_gemm_twin(P + 2, 4, 16, P, 1, P, P, wt, None) == fb.ERR_ARG


def test_expert_arm_refusals(lib):
    """The native expert arm's entry points refuse bad formats, shapes, M,
    pointers and global scales before any device work."""
    MX, NV = fb.FMT_MXFP4, fb.FMT_NVFP4
    g = lib.fp4_expert_gemv
    for bad in ((2, P, P, 1.0, 4, 128, P, P, 1, P), (-1, P, P, 1.0, 4, 128, P, P, 1, P),
                (MX, P, P, 1.0, 0, 128, P, P, 1, P), (MX, P, P, 1.0, 4, 64, P, P, 1, P),
                (MX, P, P, 1.0, 4, 192, P, P, 1, P), (MX, P, P, 1.0, 4, 65536 + 128, P, P, 1, P),
                (MX, P, P, 1.0, 4, 128, P, P, 0, P), (MX, P, P, 1.0, 4, 128, P, P, 17, P),
                (MX, P, P, float("inf"), 4, 128, P, P, 1, P), (NV, P, P, float("nan"), 4, 128, P, P, 1, P),
                (MX, None, P, 1.0, 4, 128, P, P, 1, P), (MX, P, None, 1.0, 4, 128, P, P, 1, P),
                (MX, P, P, 1.0, 4, 128, None, P, 1, P), (MX, P, P, 1.0, 4, 128, P, None, 1, P),
                (MX, P, P, 1.0, 4, 128, P, P, 1, None), (MX, P + 8, P, 1.0, 4, 128, P, P, 1, P),
                (MX, P, P, 1.0, 4, 128, P + 8, P, 1, P), (MX, P, P, 1.0, 4, 128, P, P, 1, P + 2),
                (NV, P, P + 2, 1.0, 4, 128, P, P, 1, P)):
        assert g(*bad, None) == fb.ERR_ARG, bad
    # act_quant: M in [1, 16], cols a multiple of 16, 16-byte aligned x and xq
    q = lib.fp8blk_act_quant
    for bad in ((P, 0, 128, P, P), (P, 17, 128, P, P), (P, 1, 24, P, P), (P, 1, 8, P, P),
                (P + 2, 1, 128, P, P), (P, 1, 128, P + 4, P), (None, 1, 128, P, P), (P, 1, 128, P, None)):
        assert q(*bad, None) == fb.ERR_ARG, bad
    # load check and dequant: cols a multiple of 32
    fbi = ctypes.c_int64(5)
    assert lib.fp4_load_check(MX, P, P, 4, 48, P, 256, ctypes.byref(fbi), None) == fb.ERR_ARG and fbi.value == -1
    assert lib.fp4_load_check(2, P, P, 4, 64, P, 256, None, None) == fb.ERR_ARG
    assert lib.fp4_load_check(NV, P, P, 0, 64, P, 256, None, None) == fb.ERR_ARG
    assert lib.fp4_load_check(NV, P, P, 4, 64, None, 256, None, None) == fb.ERR_WORKSPACE
    assert lib.fp4_load_check(NV, P, P, 4, 64, P, 8, None, None) == fb.ERR_WORKSPACE
    assert lib.fp4_dequant_bf16(MX, P, P, 4, 48, P, None) == fb.ERR_ARG
    assert lib.fp4_dequant_bf16(MX, P, P, 4, 64, P + 8, None) == fb.ERR_ARG
    assert lib.fp4_dequant_bf16(NV, P, P + 1, 4, 64, P, None) == fb.ERR_ARG
    assert lib.fp4_dequant_bf16(3, P, P, 4, 64, P, None) == fb.ERR_ARG
    # the expert sequence: same M for every linear, valid descriptors, workspace
    E = fb.Fp4ExpertLinear
    h = fb.SequenceHandle()
    nb = fb.fp8blk_sequence_bytes(2)
    init = lib.fp4_expert_sequence_init
    good = E(P, P, 1.0, 4, 128, 1, P, P, P)
    arr = (E * 2)(good, good)
    assert init(ctypes.byref(h), MX, arr, 0, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), 7, arr, 2, P, nb, None) == fb.ERR_ARG
    assert init(None, MX, arr, 2, P, nb, None) == fb.ERR_ARG
    assert init(ctypes.byref(h), MX, arr, 2, None, nb, None) == fb.ERR_WORKSPACE
    assert init(ctypes.byref(h), MX, arr, 2, P, nb - 1, None) == fb.ERR_WORKSPACE
    assert init(ctypes.byref(h), MX, arr, 2, P + 32, nb, None) == fb.ERR_WORKSPACE
    for bad in (E(P, P, 1.0, 4, 128, 2, P, P, P), E(P, P, 1.0, 4, 96, 1, P, P, P), E(P, P, 1.0, 0, 128, 1, P, P, P),
                E(P, P, float("inf"), 4, 128, 1, P, P, P), E(P + 8, P, 1.0, 4, 128, 1, P, P, P),
                E(P, P, 1.0, 4, 128, 1, None, P, P)):
        assert init(ctypes.byref(h), NV, (E * 2)(good, bad), 2, P, nb, None) == fb.ERR_ARG
    h.plan, h.units_dense, h.n, h.arm, h.grid_dense, h.M = P, 10, 2, fb.ARM_FP8, 4, 1
    assert lib.fp4_expert_sequence(ctypes.byref(h), None) == fb.ERR_ARG  # not an expert plan
    h.arm, h.M = fb.ARM_NVFP4, 17
    assert lib.fp4_expert_sequence(ctypes.byref(h), None) == fb.ERR_ARG
    assert lib.fp4_expert_sequence(None, None) == fb.ERR_ARG


def _chain_arrays(specs, groups):
    """C arrays for the chained-launch host checks: specs [(rows, cols)] with
    fake, aligned device addresses (the checks never dereference them)."""
    la = (fb.Linear * len(specs))()
    for k, (rows, _cols) in enumerate(specs):
        la[k].w, la[k].scales_f32, la[k].rows, la[k].y = 0x100000 * (k + 1), 0x7000000 + 0x10000 * k, rows, \
            0x9000000 + 0x10000 * k
    ga = (fb.ChainGroup * len(groups))()
    for k, (first, n, cols, src, c) in enumerate(groups):
        ga[k].first, ga[k].n, ga[k].cols, ga[k].src, ga[k].c = first, n, cols, src, c
    return la, len(specs), ga, len(groups)


def test_chain_plan_checks(lib):
    """The chained launch's list checks run on the host, before any device
    work: a valid list has a workspace size (descriptors + control words + one
    8-byte word per output row of every linear that feeds a later group), and
    each malformed list is refused (size 0, init FP8BLK_ERR_ARG)."""
    specs = [(4096, 4096), (1024, 4096), (4096, 4096), (2048, 4096), (4096, 2048)]
    good = [(0, 2, 4096, -1, 1.0), (2, 1, 4096, 0, 0.5), (3, 1, 4096, 2, 2.0), (4, 1, 2048, 3, 1.0)]
    n = lib.fp8blk_chain_bytes(*_chain_arrays(specs, good))
    # 256 control bytes, 4 x 16-byte groups, one 48-byte record per work unit (2 rows of a 4096-column linear,
    # 4 rows of a 2048-column one), then one 8-byte word per output row of linears 0, 2 and 3 (the inputs of
    # groups 1, 2 and 3)
    units = 4096 // 2 + 1024 // 2 + 4096 // 2 + 2048 // 2 + 4096 // 4
    recs_end = 256 + 64 + 48 * units
    assert n == -(-recs_end // 64) * 64 + 8 * (4096 + 4096 + 2048)
    bad = {
        "a gap between groups": [(0, 2, 4096, -1, 1.0), (3, 1, 4096, 0, 0.5), (4, 1, 2048, 3, 1.0)],
        "groups not covering the list": good[:3],
        "src in the same group": [(0, 2, 4096, 1, 1.0)] + good[1:],
        "src in a later group": [(0, 2, 4096, 2, 1.0)] + good[1:],
        "src rows != cols": [good[0], (2, 1, 4096, 1, 0.5)] + good[2:],
        "cols 8192": [good[0], good[1], good[2], (4, 1, 8192, 3, 1.0)],
        "cols 1536": [good[0], good[1], good[2], (4, 1, 1536, 3, 1.0)],
        "NaN scale": [good[0], (2, 1, 4096, 0, float("nan"))] + good[2:],
        "src -2": [good[0], (2, 1, 4096, -2, 1.0)] + good[2:],
        "empty group": [good[0], (2, 0, 4096, 0, 1.0), (2, 1, 4096, 0, 1.0)] + good[2:],
    }
    for what, groups in bad.items():
        assert lib.fp8blk_chain_bytes(*_chain_arrays(specs, groups)) == 0, what
        h = fb.ChainHandle()
        la, nl, ga, ng = _chain_arrays(specs, groups)
        st = lib.fp8blk_chain_init(ctypes.byref(h), la, nl, ga, ng, ctypes.c_void_p(0x10000000), 1 << 30, None)
        assert st == fb.ERR_ARG, what
    # a list whose cols do not match its linears' rows where it says so, with a
    # misaligned code pointer
    la, nl, ga, ng = _chain_arrays(specs, good)
    la[1].w = 0x100008
    assert lib.fp8blk_chain_bytes(la, nl, ga, ng) == 0
    # a launch without a planned chain, or with a misaligned x0, is refused
    assert lib.fp8blk_gemv_chain(None, ctypes.c_void_p(0x1000), None) == fb.ERR_ARG
    h = fb.ChainHandle()
    assert lib.fp8blk_gemv_chain(ctypes.byref(h), ctypes.c_void_p(0x1000), None) == fb.ERR_ARG
    assert lib.fp8blk_chain_status(ctypes.byref(h), None) == fb.ERR_ARG


def test_scaled_input_refusals(lib):
    """The scaled-input launches check their arguments on the host before any
    device work: more than 16 segments of columns, a NULL or misaligned src, a
    bad group size, no rows or no scale grid are refused with FP8BLK_ERR_ARG
    (the pointers here are never dereferenced)."""
    P = ctypes.c_void_p
    codes, grid, src, y = P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000)
    one = lambda rows, cols, g, s: lib.fp8blk_gemv_scaled_input(codes, g, rows, cols, s, 1.0, y, None)
    assert one(4096, 17 * 1024, grid, src) == fb.ERR_ARG
    assert one(4096, 16 * 1024 + 16, grid, src) == fb.ERR_ARG
    assert one(4096, 4096, grid, P(0x30000008)) == fb.ERR_ARG
    assert one(4096, 4096, grid, None) == fb.ERR_ARG
    assert one(0, 4096, grid, src) == fb.ERR_ARG
    assert one(4096, 4100, grid, src) == fb.ERR_ARG
    assert one(4096, 4096, None, src) == fb.ERR_ARG
    arr = (fb.Linear * 9)()
    for k in range(9):
        arr[k].w, arr[k].scales_f32, arr[k].rows, arr[k].y = 0x10000000, 0x20000000, 128, 0x40000000
    assert lib.fp8blk_gemv_grouped_scaled_input(arr, 0, 4096, src, 1.0, None) == fb.ERR_ARG
    assert lib.fp8blk_gemv_grouped_scaled_input(arr, 9, 4096, src, 1.0, None) == fb.ERR_ARG
    arr[1].rows = 0
    assert lib.fp8blk_gemv_grouped_scaled_input(arr, 2, 4096, src, 1.0, None) == fb.ERR_ARG


def test_next_input_refusals(lib):
    """The next-input launches refuse, on the host: more than 16 segments of
    columns, a NULL or odd x_next, k outside the group, a bad group size."""
    P = ctypes.c_void_p
    codes, grid, x, y, xn = P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000)
    one = lambda cols, n: lib.fp8blk_gemv_next_input(codes, grid, 4096, cols, x, y, 1.0, n, None)
    assert one(17 * 1024, xn) == fb.ERR_ARG
    assert one(4096, None) == fb.ERR_ARG
    assert one(4096, P(0x50000001)) == fb.ERR_ARG
    assert one(4100, xn) == fb.ERR_ARG
    arr = (fb.Linear * 9)()
    for k in range(9):
        arr[k].w, arr[k].scales_f32, arr[k].rows, arr[k].y = 0x10000000, 0x20000000, 128, 0x40000000
    grp = lambda n, k: lib.fp8blk_gemv_grouped_next_input(arr, n, 4096, x, k, 1.0, xn, None)
    assert grp(2, 2) == fb.ERR_ARG
    assert grp(2, -1) == fb.ERR_ARG
    assert grp(0, 0) == fb.ERR_ARG
    assert grp(9, 0) == fb.ERR_ARG


def test_glue_launch_overlap_refusals(lib):
    """An output range that overlaps the input it is formed from is refused on
    the host: a scaled-input src overlapping an output, a next-input x_next
    overlapping x or an output (the pointers are never dereferenced)."""
    P = ctypes.c_void_p
    codes, grid = P(0x10000000), P(0x20000000)
    # scaled input: src (4096 f32 = 16 KB at 0x30000000) against y (4096 f32)
    sc = lambda y: lib.fp8blk_gemv_scaled_input(codes, grid, 4096, 4096, P(0x30000000), 1.0, P(y), None)
    assert sc(0x30000000) == fb.ERR_ARG
    assert sc(0x30000000 + 16384 - 4) == fb.ERR_ARG
    assert sc(0x30000000 - 16384 + 4) == fb.ERR_ARG
    # next input: x (4096 bf16 = 8 KB at 0x30000000), y (4096 f32 at 0x40000000), x_next (4096 bf16)
    nx = lambda xn: lib.fp8blk_gemv_next_input(codes, grid, 4096, 4096, P(0x30000000), P(0x40000000), 1.0, P(xn), None)
    assert nx(0x30000000 + 8192 - 2) == fb.ERR_ARG
    assert nx(0x30000000 - 8192 + 2) == fb.ERR_ARG
    assert nx(0x40000000 + 16384 - 2) == fb.ERR_ARG
    assert nx(0x40000000 - 8192 + 2) == fb.ERR_ARG
