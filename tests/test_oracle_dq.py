"""Pins for the oracle's double quantization and two-level constant decode.

"Double quantization" (zerotofrontier.app PEFT page): the fp32 absmax values
c1 are treated as data, their mean is subtracted, and they are quantized to
8-bit floats in blocks of 256, each block with its own fp32 constant c2.  The
cost per parameter falls from 32/64 = 0.5 bits to 8/64 + 32/(64*256) ~ 0.127
bits (a saving of 0.373 bits, ~3 GB at 65B), 4.127 bits or ~0.516 bytes per
weight in total, and 65e9 * 4.127 / 8 ~ 33.5 GB for a 65B base ("Paged
optimizers, and QLoRA end to end").
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

E4M3_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
              0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0,
              0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}


def test_e4m3_decode_known_values(orc):
    for code, val in E4M3_KNOWN.items():
        assert orc.e4m3_decode(code) == val
    assert math.copysign(1.0, orc.e4m3_decode(0x80)) == -1.0


def _torch_e4m3(v):
    t = torch.tensor(np.asarray(v, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_matches_library_conversion(orc):
    # every finite value, every midpoint, and points just around the midpoints
    vals = np.array([orc.e4m3_decode(c) for c in range(0x7F)])
    mids = (vals[1:] + vals[:-1]) / 2
    probe = [vals, mids]
    for m in mids:
        f = np.float32(m)
        probe.append(np.array([np.nextafter(f, np.float32(-1)), np.nextafter(f, np.float32(1e9))],
                              np.float64))
    rng = np.random.Generator(np.random.PCG64(0))
    probe.append(rng.uniform(0, 448, 20000))
    probe.append(np.exp2(rng.uniform(-14, 8.8, 20000)))
    v = np.concatenate(probe).astype(np.float32)
    v = v[v <= 448]
    v = np.concatenate([v, -v])
    ref = _torch_e4m3(v)
    got = np.array([orc.e4m3_encode(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_ties_to_even(orc):
    assert orc.e4m3_encode(1.0625) == 0x38      # halfway 1.0 / 1.125 -> even mantissa
    assert orc.e4m3_encode(1.1875) == 0x3A      # halfway 1.125 / 1.25 -> even mantissa
    assert orc.e4m3_encode(2.0 ** -10) == 0x00  # halfway 0 / 2^-9 -> zero
    assert orc.e4m3_encode(-(2.0 ** -11)) == 0x80


def test_pairwise_sum_order(orc):
    # aligned pairwise tree: (2^53 + 1) + (1 + 1) = 2^53 + 2, whereas a left-to-right
    # float64 sum loses each 1 and returns 2^53
    x = np.array([2.0 ** 53, 1.0, 1.0, 1.0], np.float32)
    assert orc.pairwise_sum(x) == 2.0 ** 53 + 2
    assert orc.pairwise_sum(np.array([1, 2, 3, 4, 5], np.float32)) == 15.0
    assert orc.pairwise_sum(np.zeros(0, np.float32)) == 0.0


def test_mean_is_exact_for_realistic_constants(orc):
    rng = np.random.Generator(np.random.PCG64(1))
    c1 = np.abs(rng.standard_normal(100_003) * 0.02).astype(np.float32) + np.float32(0.03)
    q, c2, mean = orc.double_quantize(c1)
    exact = math.fsum(c1.astype(np.float64).tolist())   # correctly rounded library sum
    assert mean[0] == np.float32(exact / c1.size)
    assert c2.size == (c1.size + 255) // 256


def test_constant_block_decodes_to_mean(orc):
    c1 = np.full(700, 0.125, np.float32)
    q, c2, mean = orc.double_quantize(c1)
    assert mean[0] == np.float32(0.125)
    assert np.all(c2 == 0) and np.all(q == 0)
    assert np.all(orc.double_dequantize(q, c2, mean) == np.float32(0.125))


def test_block_extreme_maps_to_448(orc):
    rng = np.random.Generator(np.random.PCG64(2))
    c1 = np.abs(rng.standard_normal(256 * 6 + 100)).astype(np.float32)
    q, c2, mean = orc.double_quantize(c1)
    d = c1 - mean[0]
    for b in range(c2.size):
        blk = d[256 * b: 256 * b + 256]
        i = int(np.argmax(np.abs(blk)))
        assert c2[b] == np.abs(blk[i])
        assert q[256 * b + i] == (0xFE if blk[i] < 0 else 0x7E)


def _round_fraction_to_f32(x: Fraction) -> np.float32:
    """Round an exact rational to fp32, nearest, ties to even."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_decode_is_single_rounding(orc):
    rng = np.random.Generator(np.random.PCG64(3))
    n1 = 256 * 8
    q = rng.integers(0, 256, n1).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10                       # no NaN codes
    c2 = (np.abs(rng.standard_normal(8)) * 0.05).astype(np.float32)
    mean = np.array([0.0312], np.float32)
    got = orc.double_dequantize(q, c2, mean)
    for i in range(0, n1, 7):
        step = np.float32(c2[i // 256]) / np.float32(448.0)      # IEEE fp32 division
        exact = (Fraction(orc.e4m3_decode(int(q[i]))) * Fraction(float(step))
                 + Fraction(float(mean[0])))
        assert got[i] == _round_fraction_to_f32(exact), i


def test_dq_error_on_gaussian_weights(orc):
    # context, not a page figure: the decoded constants stay close to the originals
    rng = np.random.Generator(np.random.PCG64(4))
    w = (rng.standard_normal(64 * 256 * 40) * 0.02).astype(np.float32)
    _, absmax = orc.nf4_quantize(w)
    q, c2, mean = orc.double_quantize(absmax)
    c1p = orc.double_dequantize(q, c2, mean)
    rel = np.abs(c1p - absmax) / absmax
    assert np.median(rel) < 0.005 and rel.max() < 0.05


def test_encode_decode_roundtrip_within_half_step(orc):
    rng = np.random.Generator(np.random.PCG64(5))
    c1 = np.abs(rng.standard_normal(256 * 20)).astype(np.float32) * 0.05
    q, c2, mean = orc.double_quantize(c1)
    c1p = orc.double_dequantize(q, c2, mean)
    d = c1.astype(np.float64) - mean[0]
    s = d / np.repeat(c2, 256)[: c1.size].astype(np.float64)
    # E4M3 relative spacing is 1/8 in the normal range, so |error| <= c2/448 * ulp/2
    ulp = np.where(np.abs(s * 448) >= 2.0 ** -6,
                   2.0 ** (np.floor(np.log2(np.maximum(np.abs(s * 448), 1e-30))) - 3), 2.0 ** -9)
    bound = ulp / 2 * np.repeat(c2, 256)[: c1.size] / 448 * 1.0001 + 1e-9
    assert np.all(np.abs(c1p - c1) <= bound + np.abs(c1) * 2.0 ** -23)


@pytest.mark.parametrize("n", [0, 1, 63, 64, 65, 64 * 256, 64 * 256 + 1])
def test_tuple_sizes(orc, n):
    rng = np.random.Generator(np.random.PCG64(6))
    w = rng.standard_normal(n).astype(np.float32)
    codes, absmax = orc.nf4_quantize(w)
    q, c2, mean = orc.double_quantize(absmax)
    assert codes.size == (n + 1) // 2
    assert absmax.size == q.size == (n + 63) // 64
    assert c2.size == ((n + 63) // 64 + 255) // 256
    if n == 0:
        assert mean[0] == 0.0


def test_plain_constants_dequantize_round_trip(orc):
    # double quantization off ("Double quantization": the 0.5-bit plain constants): w' =
    # level * absmax.  Each block's absmax element comes back as +-absmax exactly and
    # every other value stays nearest its level, so re-encoding w' returns the same codes
    # and the same constants; code 7 is an exact zero
    rng = np.random.Generator(np.random.PCG64(11))
    w = rng.normal(0, 0.02, 64 * 300 + 17).astype(np.float32)
    w[64:128] = 0.0
    codes, absmax = orc.nf4_quantize(w)
    wd = orc.nf4_dequantize_plain(codes, absmax, (w.size,))
    codes2, absmax2 = orc.nf4_quantize(wd)
    assert np.array_equal(codes2, codes)
    assert np.array_equal(absmax2.view(np.uint32), absmax.view(np.uint32))
    c = np.concatenate([codes & 15, codes >> 4], axis=0).reshape(2, -1).T.reshape(-1)[:w.size]
    assert np.all(wd[c == 7] == 0.0)
    blk = np.repeat(absmax, 64)[:w.size]
    assert np.array_equal(wd[c == 15], blk[c == 15]) and np.array_equal(wd[c == 0], -blk[c == 0])
