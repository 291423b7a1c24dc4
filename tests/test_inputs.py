"""The seeded input generator: determinism and the stated distributions."""
import numpy as np

from block_scaled_fp8_fp8blk_amd import inputs


def test_same_seed_same_bytes_and_seeds_differ():
    a = inputs.host_linear(300, 528, 3, 42)
    b = inputs.host_linear(300, 528, 3, 42)
    c = inputs.host_linear(300, 528, 3, 43)
    for k in ("codes", "scales", "x"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert not np.array_equal(a.codes, c.codes)


def test_tiny_distribution():
    L = inputs.tiny()
    assert L.codes.shape == (256, 512) and L.scales.shape == (2, 4) and L.x.shape == (1, 512)
    assert not np.any((L.codes & 0x7F) == 0x7F)
    assert len(np.unique(L.codes)) == 254
    assert L.scales.min() >= 120 and L.scales.max() <= 134


def test_normal_code_distribution():
    L = inputs.host_linear(1024, 1024, 1, 1)
    assert not np.any((L.codes & 0x7F) == 0x7F)
    E = (L.codes >> 3) & 15
    frac_sub = np.mean(E == 0)  # zero or subnormal codes
    assert 0.2 < frac_sub < 0.3
    assert L.scales.min() >= 124 and L.scales.max() <= 130
    xe = (L.x >> 7) & 0xFF
    assert not np.any(xe == 0xFF)  # finite activations


def test_sweep_plan():
    sw = inputs.sweep_plan()
    assert len(sw.linears) == 43 * 6 + 1 == 259
    assert sw.linears[-1].rows == 129280 and sw.linears[-1].cols == 4096
    assert [l.seed for l in sw.linears] == list(range(100, 359))
    codes = sum(l.rows * l.cols for l in sw.linears)
    assert codes == 3_234_856_960
    assert sw.weight_bytes() == 3_234_856_960 + 4 * 197_440


def test_verify_panel_specs():
    assert inputs.VERIFY_SPECS == ((12288, 4096, 16, 5), (4096, 4096, 16, 6))
    assert inputs.VERIFY_M == (2, 4, 8, 16)
