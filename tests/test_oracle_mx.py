"""Pins of the oracle's MX (E4M3 + E8M0) quantizer: hand-worked cases, an
exhaustive sweep over bf16 bit patterns against torch's float8_e4m3fn cast,
and the decode table against torch."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def block(vals):
    v = np.zeros(32)
    v[:len(vals)] = vals
    return v


def test_hand_cases():
    # all-zero block: scale code 0, zero elements
    c, s = O.mx_quantize(np.zeros((1, 32)))
    assert s.tolist() == [[0]] and np.all(c == 0)
    # amax 1.0: 1.0 / 2^-8 = 256 <= 448 and 1.0 / 2^-9 = 512 > 448, so e_s = -8
    # (code 119); 1.0 -> 256 = 2^8 (field 15, mant 0) = 0x78
    c, s = O.mx_quantize(block([1.0, 0.5, -1.0])[None])
    assert s[0, 0] == 119 and c[0, 0] == 0x78 and c[0, 1] == 0x70 and c[0, 2] == 0xF8
    # amax 1.75 is exactly 448 at e_s = -8: kept at code 119, element 0x7E
    c, s = O.mx_quantize(block([1.75, -1.75])[None])
    assert s[0, 0] == 119 and c[0, 0] == 0x7E and c[0, 1] == 0xFE
    # amax 1.9375: 1.9375 * 256 = 496 > 448, so e_s = -7 (code 120) and nothing
    # clips: 1.9375 * 128 = 248 is halfway between 240 (0x77, mant 7) and 256
    # (0x78, mant 0) -> 256; 1.8125 * 128 = 232 halfway between 224 (0x76) and
    # 240 (0x77) -> 224; 1.0625 * 128 = 136 halfway between 128 (0x70) and 144
    # (0x71) -> 128
    c, s = O.mx_quantize(block([1.9375, 1.8125, 1.0625])[None])
    assert s[0, 0] == 120 and c[0, 0] == 0x78 and c[0, 1] == 0x76 and c[0, 2] == 0x70
    # just above 1.75: one step coarser
    c, s = O.mx_quantize(block([1.75 * (1 + 2.0 ** -20)])[None])
    assert s[0, 0] == 120
    # 1.0625 * 256 = 272 at e_s = -8: halfway between 256 (m=0) and 288 (m=1) -> 256
    c, s = O.mx_quantize(block([1.0, 1.0625])[None])
    assert s[0, 0] == 119 and c[0, 1] == 0x78
    # subnormal: 2^-16 relative to 2^-8 is 2^-8 = 2 * 2^-9 -> code 0x02
    c, s = O.mx_quantize(block([1.0, 2.0 ** -16])[None])
    assert c[0, 1] == 0x02
    # scale clamp at the bottom of E8M0
    c, s = O.mx_quantize(block([2.0 ** -130])[None])
    assert s[0, 0] == 0
    # scale clamp at the top of E8M0 (code 254): 2^140 / 2^127 = 8192 saturates at 448
    c, s = O.mx_quantize(block([2.0 ** 140, -(2.0 ** 140)])[None])
    assert s[0, 0] == 254 and c[0, 0] == 0x7E and c[0, 1] == 0xFE


def test_scale_is_smallest_unclipped_power_of_two():
    """The block exponent is the smallest integer e with amax / 2^e <= 448,
    found here by a search over e, on magnitudes spread over the whole range,
    exact powers of two, 448 times powers of two and their neighbours."""
    rng = np.random.default_rng(3)
    a = np.exp(rng.uniform(-80, 80, size=4000))
    pw = np.ldexp(1.0, np.arange(-100, 100))
    edge = np.concatenate([pw, 448 * pw, 1.75 * pw])
    a = np.concatenate([a, edge, np.nextafter(edge, 0), np.nextafter(edge, np.inf)])
    got = O.mx_scale_exponent(a)
    for v, e in zip(a, got):
        want = -200
        while v / 2.0 ** want > 448.0:
            want += 1
        assert e == want, (v, e, want)
        assert v / 2.0 ** e <= 448.0 and v / 2.0 ** (e - 1) > 448.0


def test_exhaustive_bf16_against_torch_cast():
    bits = np.arange(65536, dtype=np.uint32)
    v = (bits << 16).view(np.float32).astype(np.float64)
    v = v[np.isfinite(v)]
    ours = O.e4m3_round(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    inr = np.abs(v) <= 464.0            # torch does not saturate beyond this
    assert np.array_equal(ours[inr], ref[inr])
    assert np.all(np.abs(ours[~inr]) == 448.0)
    assert np.array_equal(np.signbit(ours[v != 0]), np.signbit(v[v != 0]))
    enc = O.e4m3_encode(ours[inr])
    ref_bits = torch.from_numpy(v[inr].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc, ref_bits)


def test_decode_table_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


@pytest.mark.parametrize("axis", [0, 1])
def test_round_trip_error_bound(axis):
    rng = np.random.default_rng(11)
    v = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-8, 8, size=(64, 96)))
    v = v.astype(np.float32).astype(np.float64)
    c, s = O.mx_quantize(v, axis=axis)
    back = O.mx_dequantize(c, s, axis=axis)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=axis)
    scaled = np.abs(v) / sc
    _, ex = np.frexp(np.maximum(scaled, 2.0 ** -6))
    half_q = np.ldexp(1.0, np.maximum(ex - 1, -6) - 4) * sc
    assert np.all(scaled <= 448)           # the block scale never clips
    assert np.all(np.abs(back - v) <= half_q)


def test_round_trip_from_primitives_matches_codes():
    """The parity tests' fast MX round trip (block exponent + E4M3 rounding,
    no bit encoding) gives exactly dequantize(quantize(v))."""
    from tests.moe_parity import qd
    rng = np.random.default_rng(5)
    for shape, axis in (((64, 96), -1), ((96, 40), 0), ((3, 32, 64), 1)):
        v = (rng.standard_normal(shape) * rng.choice([1e-3, 1.0, 300.0])).astype(np.float32).astype(np.float64)
        v.flat[::17] = 0.0
        q, s = O.mx_quantize(v, axis=axis)
        assert np.array_equal(qd(v, axis), O.mx_dequantize(q, s, axis=axis))
