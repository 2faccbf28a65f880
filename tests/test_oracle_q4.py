"""Pins of the 4-bit group-64 quantiser (input preparation) and the oracle's dequantiser."""
import numpy as np

from block_verify_amd.synth import bf16_bits_to_f32, f32_to_bf16_bits, quantize_q4g64
from oracle import q4


def _rand_bf16(n, k, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((n, k)).astype(np.float32) * 0.02)


def test_unpack_nibble_order():
    packed = np.array([[0x21, 0xF0]], dtype=np.uint8)
    assert q4.unpack_codes(packed).tolist() == [[1, 2, 0, 15]]


def test_dequant_error_bound():
    w = _rand_bf16(32, 256, 0)
    packed, s, z = quantize_q4g64(w)
    wd = q4.dequantize(packed, s, z)
    wf = bf16_bits_to_f32(w).astype(np.float64)
    sf = s.astype(np.float64).repeat(64, axis=1)
    zf = z.astype(np.float64).repeat(64, axis=1)
    # rounding to the nearest code costs s/2; fp16 rounding of the zero shifts the grid by |z - z_h| s
    mn = wf.reshape(32, 4, 64).min(axis=2).repeat(64, axis=1)
    z_exact = -mn / sf
    bound = sf / 2 + np.abs(z_exact - zf) * sf + 1e-12
    assert np.all(np.abs(wd - wf) <= bound + 1e-9)
    assert np.abs(wd - wf).max() > 0


def test_values_on_the_grid_are_exact():
    s, lo = 2.0 ** -7, -3 * 2.0 ** -7
    codes = np.tile(np.arange(16), 4)[None, :64].repeat(2, axis=0)
    w = (lo + codes * s).astype(np.float32)
    packed, s_h, z_h = quantize_q4g64(f32_to_bf16_bits(w))
    np.testing.assert_array_equal(q4.dequantize(packed, s_h, z_h), w.astype(np.float64))


def test_degenerate_group():
    wb = f32_to_bf16_bits(np.full((1, 64), 0.0125, dtype=np.float32))
    packed, s_h, z_h = quantize_q4g64(wb)
    assert float(s_h[0, 0]) == 1.0
    assert np.all(q4.unpack_codes(packed) == 0)
    expect = float(np.float16(bf16_bits_to_f32(wb)[0, 0]))
    np.testing.assert_array_equal(q4.dequantize(packed, s_h, z_h), np.full((1, 64), expect))


def test_codes_monotone_in_weight():
    rng = np.random.default_rng(3)
    w = np.sort(rng.standard_normal((4, 64)).astype(np.float32) * 0.02, axis=1)
    packed, _, _ = quantize_q4g64(f32_to_bf16_bits(w))
    codes = q4.unpack_codes(packed).astype(int)
    assert np.all(np.diff(codes, axis=1) >= 0)
    assert np.all(codes[:, 0] == 0) and np.all(codes[:, -1] == 15)
