"""Pins for the oracle's bf16 and OCP E4M3 codecs.

Each codec is checked exhaustively against what the formats fix (every bit
pattern, every rounding midpoint) and against torch's independent CPU
conversions (``Tensor.to(torch.bfloat16)`` and ``torch.float8_e4m3fn``), so a
wrong exponent bias, a dropped subnormal branch or a wrong tie rule fails here.
"""
import numpy as np
import pytest
import torch

import oracle


def _bf16_bits_to_f64_torch(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ----------------------------------------------------------------------------- bf16

def test_bf16_decode_matches_torch_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = _bf16_bits_to_f64_torch(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0x0000])


def test_bf16_encode_roundtrip_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_decode(bits)
    finite = np.isfinite(vals)
    back = oracle.bf16_encode(vals[finite])
    assert np.array_equal(back, bits[finite])
    # infinities map to themselves; NaN to the canonical quiet NaN
    assert oracle.bf16_encode(np.array([np.inf, -np.inf]))[0] == 0x7F80
    assert oracle.bf16_encode(np.array([np.inf, -np.inf]))[1] == 0xFF80
    assert oracle.bf16_encode(np.array([np.nan]))[0] == 0x7FC0


def test_bf16_midpoints_tie_to_even_exhaustive():
    # every pair of adjacent finite positive bf16 values (subnormals included)
    lo_bits = np.arange(0x0000, 0x7F7F, dtype=np.uint16)
    lo = oracle.bf16_decode(lo_bits)
    hi = oracle.bf16_decode(lo_bits + 1)
    mid = 0.5 * (lo + hi)                        # exact in fp64 (9 significant bits)
    even = np.where(lo_bits % 2 == 0, lo_bits, lo_bits + 1).astype(np.uint16)
    assert np.array_equal(oracle.bf16_encode(mid), even)
    assert np.array_equal(oracle.bf16_encode(np.nextafter(mid, 0.0)), lo_bits)
    assert np.array_equal(oracle.bf16_encode(np.nextafter(mid, np.inf)), lo_bits + 1)
    # negative side mirrors
    assert np.array_equal(oracle.bf16_encode(-mid), even | 0x8000)


def test_bf16_hand_values():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to 1.0 (even mantissa);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6.
    got = oracle.bf16_encode(np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -2.0, 2.0**-133,
                                       2.0**-134, 3 * 2.0**-135]))
    assert list(got) == [0x3F80, 0x3F82, 0xC000, 0x0001, 0x0000, 0x0001]


def test_bf16_encode_matches_torch_on_random_fp32():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(200000, generator=g) * torch.exp2(torch.randint(-140, 120, (200000,),
                                                                     generator=g).float())
    x = x[torch.isfinite(x)]
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.bf16_encode(x.to(torch.float64).numpy())
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------- e4m3

def test_e4m3_decode_matches_torch_exhaustive():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_format_landmarks():
    # OCP E4M3: bias 7, 3 mantissa bits, largest finite S.1111.110 = 448,
    # smallest normal 2^-6, smallest subnormal 2^-9, no infinities.
    d = oracle.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x38, 0x07, 0xFE, 0x80], np.uint8))
    assert list(d[:6]) == [448.0, 2.0**-6, 2.0**-9, 1.0, 7 * 2.0**-9, -448.0]
    assert d[6] == 0.0 and np.signbit(d[6])
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)              # strictly increasing finite codes


def test_e4m3_encode_roundtrip_and_midpoints():
    codes = np.arange(127, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    assert np.array_equal(oracle.e4m3_encode(-vals[1:]), codes[1:] | 0x80)
    mid = 0.5 * (vals[:-1] + vals[1:])
    even = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:]).astype(np.uint8)
    enc, tie = oracle.e4m3_encode(mid, with_near_tie=True)
    assert np.array_equal(enc, even)
    assert tie.all()
    below = mid * (1 - 2.0**-17)
    above = mid * (1 + 2.0**-17)
    enc_b, tie_b = oracle.e4m3_encode(below, with_near_tie=True)
    enc_a, tie_a = oracle.e4m3_encode(above, with_near_tie=True)
    assert np.array_equal(enc_b, codes[:-1]) and np.array_equal(enc_a, codes[1:])
    assert not tie_b.any() and not tie_a.any()
    _, tie_in = oracle.e4m3_encode(mid * (1 + 2.0**-20), with_near_tie=True)
    assert tie_in.all()


def test_e4m3_saturation_and_signed_zero():
    enc = oracle.e4m3_encode(np.array([448.0, 449.0, 464.0, 1e9, -1e9, -1e-5, 0.0, 2.0**-10,
                                       3 * 2.0**-11]))
    # clamp to 448 before rounding; 2^-10 is the tie between 0 and 2^-9 -> 0;
    # 3*2^-11 lies nearer 2^-9
    assert list(enc) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x01]


def test_e4m3_encode_matches_torch_in_range():
    g = torch.Generator().manual_seed(2)
    x = (torch.rand(300000, generator=g) * 2 - 1) * torch.exp2(
        torch.randint(-14, 9, (300000,), generator=g).float())
    x = x.clamp(-448, 448)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3_encode(x.to(torch.float64).numpy())
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("v", [1.0625, 0.0009765625, 432.0])
def test_e4m3_near_tie_flags_exact_midpoints(v):
    # 1.0625 lies halfway between 1 and 1.125; 2^-10 between 0 and 2^-9;
    # 432 between 416 and 448.
    _, tie = oracle.e4m3_encode(np.array([v, -v]), with_near_tie=True)
    assert tie.all()
