"""Pins for the FP8 E4M3 encoder of the oracle (OCP "fn" format, RNE, clamped
to +-448, one fp32 scale per tensor): values fixed by the format's
definition, brute force against every finite code, and the bf16 table."""

import math

import numpy as np

from oracle import fp8

FINITE = [b for b in range(256) if not math.isnan(fp8.decode_value(b))]


def test_format_constants():
    assert len(FINITE) == 254                      # 0x7F and 0xFF are the only NaNs
    assert fp8.decode_value(0x7E) == 448.0 and fp8.decode_value(0xFE) == -448.0
    assert fp8.decode_value(0x38) == 1.0           # exponent 7 = bias
    assert fp8.decode_value(0x08) == 2.0 ** -6     # smallest normal
    assert fp8.decode_value(0x01) == 2.0 ** -9     # smallest subnormal
    assert fp8.decode_value(0x77) == 240.0         # 1.875 * 2^7
    assert fp8.encode_value(1.0) == 0x38 and fp8.encode_value(-1.0) == 0xB8
    assert fp8.encode_value(0.0) == 0x00 and fp8.encode_value(-0.0) == 0x80


def test_round_half_even_and_saturation():
    # ties between neighbours go to the even mantissa
    assert fp8.encode_value(0.5 * 2.0 ** -9) == 0x00          # 0 and 1 subnormal units: even is 0
    assert fp8.encode_value(1.5 * 2.0 ** -9) == 0x02          # 1 and 2: even is 2
    assert fp8.encode_value(1.0 + 1.0 / 16) == 0x38           # 1.0 and 1.125: even mantissa 0
    assert fp8.encode_value(1.0 + 3.0 / 16) == 0x3A           # 1.125 and 1.25: even mantissa 2
    # clamped to the largest finite value
    for x in (448.0, 449.0, 464.0, 1e6):
        assert fp8.encode_value(x) == 0x7E and fp8.encode_value(-x) == 0xFE


def test_every_code_round_trips():
    for b in FINITE:
        assert fp8.encode_value(fp8.decode_value(b)) == (b if b != 0x80 else 0x80)


def test_nearest_code_by_brute_force():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 60, 3000), rng.uniform(-0.02, 0.02, 2000)])
    codes = np.array(FINITE)
    dec = np.array([fp8.decode_value(int(b)) for b in codes])
    for x in vals.astype(np.float32).astype(np.float64):
        got = fp8.encode_value(x)
        xc = min(max(x, -448.0), 448.0)
        err = np.abs(dec - xc)
        best = err.min()
        assert abs(fp8.decode_value(got) - xc) == best
        ties = codes[err == best]
        if len(ties) > 1:                           # a tie: the even mantissa (or the zero of x's sign)
            assert got & 1 == 0 or fp8.decode_value(got) == 0


def test_bf16_table_matches_scalar_encoder():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, 4000).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    bits, f = bits[np.isfinite(f)], f[np.isfinite(f)]
    for scale in (1.0, 0.05, 3.0):
        tab = fp8.quantize_bf16(bits, scale)
        inv = np.float32(np.float32(1.0) / np.float32(scale))
        ref = np.array([fp8.encode_value(float(np.float32(v) * inv)) for v in f], np.uint8)
        assert np.array_equal(tab, ref)


def test_every_bf16_input_matches_torch_cast():
    """torch's float8_e4m3fn cast (round to nearest even, no saturation) of the clamped fp32 product gives
    the same code for every finite bf16 input, at several scales."""
    import torch
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    fin = np.isfinite(f)
    for scale in (1.0, 0.05, 3.0, 0.013, 1.0 / 448):
        inv = fp8.inverse_scale(scale)
        with np.errstate(over="ignore"):
            prod = np.clip((f[fin] * inv).astype(np.float32), -448, 448)
        ref = torch.from_numpy(prod).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(fp8.quantize_bf16(bits[fin].astype(np.uint16), scale), ref)
