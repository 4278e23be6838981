"""Pins for the oracle's NF4 encoder and dequantizer.

"Block-wise quantization in one page" (zerotofrontier.app PEFT page): per
block of 64 consecutive values store c = max|w|, divide the block by c and
replace each value by the index of the nearest codebook level; to use a weight
multiply its level by c.  "NF4, derived from normal quantiles": exact zeros
must stay zero.  "The real way": two codes per byte.
"""
from fractions import Fraction

import numpy as np
import pytest


def _unpack(codes, n):
    out = np.empty(codes.size * 2, np.uint8)
    out[0::2] = codes & 0xF
    out[1::2] = codes >> 4
    return out[:n]


def _brute_codes(w32, levels):
    """Nearest level by exact rational distance; a tie takes the lower index."""
    w32 = np.asarray(w32, np.float32).reshape(-1)
    n = w32.size
    L = [Fraction(float(v)) for v in levels]
    out = np.zeros(n, np.uint8)
    amax = np.zeros((n + 63) // 64, np.float32)
    for b in range(amax.size):
        blk = w32[64 * b: 64 * b + 64]
        c = np.float32(np.max(np.abs(blk)))
        amax[b] = c
        for i, v in enumerate(blk):
            if c == 0:
                out[64 * b + i] = 7
                continue
            x = Fraction(float(np.float32(v) / c))       # IEEE fp32 division
            d = [abs(x - l) for l in L]
            out[64 * b + i] = int(min(range(16), key=lambda j: (d[j], j)))
    return out, amax


@pytest.mark.parametrize("n,scale,seed", [(64, 1.0, 0), (200, 0.02, 1), (321, 3.0, 2),
                                          (1000, 1e-30, 3), (127, 1e20, 4)])
def test_brute_force_tiny(orc, nf4_levels, n, scale, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = (rng.standard_normal(n) * scale).astype(np.float32)
    w[rng.integers(0, n, size=n // 7)] = 0.0                 # exact zeros
    codes, absmax = orc.nf4_quantize(w)
    ref, amax = _brute_codes(w, nf4_levels)
    assert np.array_equal(absmax, amax)
    assert np.array_equal(_unpack(codes, n), ref)
    # exact zeros stay exactly zero after dequantization (level 7 is 0.0)
    assert np.all(_unpack(codes, n)[w == 0] == 7)


def test_packing_layout_and_odd_tail(orc):
    rng = np.random.Generator(np.random.PCG64(5))
    n = 64 * 3 + 37                                          # partial last block, odd n
    w = rng.standard_normal(n).astype(np.float32)
    codes, absmax = orc.nf4_quantize(w)
    assert codes.size == (n + 1) // 2 and absmax.size == 4
    full = _unpack(codes, codes.size * 2)
    assert full[-1] == 0, "high nibble past an odd tail is 0"
    # element 2i is the low nibble of byte i
    assert np.array_equal(codes[:5] & 0xF, full[0:10:2])
    assert np.array_equal(codes[:5] >> 4, full[1:10:2])


def test_thresholds_neighbourhood_sweep(orc, nf4_levels):
    """Every fp32 within +-3000 ulps of each midpoint, against exact nearest-level search."""
    lv = nf4_levels.astype(np.float64)
    xs = []
    for j in range(15):
        m = np.float32((lv[j] + lv[j + 1]) / 2)
        bits = m.view(np.int32) + np.arange(-3000, 3001, dtype=np.int32) * (1 if m > 0 else -1)
        xs.append(bits.view(np.float32))
    x = np.concatenate(xs)
    x = x[np.abs(x) <= 1.0]
    # blocks of 63 probe values plus the constant 1.0 so that c == 1 and w/c == w exactly
    pad = (-x.size) % 63
    x = np.concatenate([x, np.zeros(pad, np.float32)]).reshape(-1, 63)
    w = np.concatenate([x, np.ones((x.shape[0], 1), np.float32)], axis=1).reshape(-1)
    codes, absmax = orc.nf4_quantize(w)
    assert np.all(absmax == 1.0)
    got = _unpack(codes, w.size)
    # nearest level: x - level is exact in float64 for these magnitudes
    d = np.abs(w.astype(np.float64)[:, None] - lv[None, :])
    dmin = d.min(axis=1, keepdims=True)
    ref = np.argmax(d == dmin, axis=1)                      # first (lower) index on a tie
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("j", [2, 6, 7, 14])
def test_exact_ties_take_lower_level(orc, nf4_levels, j):
    lv = nf4_levels.astype(np.float64)
    m = (lv[j] + lv[j + 1]) / 2
    assert float(np.float32(m)) == m, "this midpoint is an fp32 value, so ties are reachable"
    w = np.array([m, 1.0] + [0.0] * 62, np.float32)
    codes, _ = orc.nf4_quantize(w)
    assert _unpack(codes, 2)[0] == j


def test_zero_block_and_extremes(orc):
    w = np.zeros(128, np.float32)
    w[64:] = np.linspace(-2.0, 1.0, 64, dtype=np.float32)
    codes, absmax = orc.nf4_quantize(w)
    u = _unpack(codes, 128)
    assert absmax[0] == 0.0 and np.all(u[:64] == 7)
    assert absmax[1] == 2.0 and u[64] == 0                   # -absmax -> level -1
    w2 = np.zeros(64, np.float32)
    w2[10] = 5.0
    w2[11] = -0.0
    codes2, _ = orc.nf4_quantize(w2)
    u2 = _unpack(codes2, 64)
    assert u2[10] == 15 and u2[11] == 7


def test_bf16_input_equals_widened_fp32(orc):
    rng = np.random.Generator(np.random.PCG64(6))
    f = rng.standard_normal(64 * 50 + 10).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)        # truncation gives some bf16 values
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    c_b, a_b = orc.nf4_quantize(bits)
    c_f, a_f = orc.nf4_quantize(widened)
    assert np.array_equal(c_b, c_f) and np.array_equal(a_b, a_f)


def test_requantize_is_idempotent(orc, nf4_levels):
    rng = np.random.Generator(np.random.PCG64(7))
    w = (rng.standard_normal(64 * 200) * 0.02).astype(np.float32)
    codes, absmax = orc.nf4_quantize(w)
    u = _unpack(codes, w.size)
    wq = nf4_levels[u] * np.repeat(absmax, 64)                # fp32 level * c
    codes2, absmax2 = orc.nf4_quantize(wq.astype(np.float32))
    assert np.array_equal(absmax, absmax2) and np.array_equal(codes, codes2)


def test_dequantize_fixed_points(orc):
    # Pins of the double-quantized dequantize that do not restate level x c1':
    #  - code 7 is the exact zero level, so it decodes to +0 or -0 whatever c1' is;
    #  - codes 0 and 15 are the levels -1 and +1 exactly, so they decode to -c1' and +c1'
    #    bit for bit, and c1' comes from the oracle's constant decode alone;
    #  - a block whose 64 values are +-v (v a power of two, so every quotient is exact)
    #    has absmax v; codes 15/0 for +v/-v; dequantized back to +-c1' (the decoded
    #    constant), and with every absmax equal, double quantization keeps c1' == v exactly
    #    (c2 = 0, q = 0, c1' = mean): the weight comes back unchanged;
    #  - re-encoding the dequantized weight with its decoded constants c1' as absmax
    #    (those are the block maxima of w' whenever a block holds a code 0 or 15) gives the
    #    same codes.
    rng = np.random.Generator(np.random.PCG64(81))
    n = 64 * 40
    signs = np.where(rng.standard_normal(n) >= 0, 1.0, -1.0)
    w = (signs * 0.03125).astype(np.float32)
    codes, absmax = orc.nf4_quantize(w)
    assert np.all(absmax == np.float32(0.03125))
    c = _unpack(codes, n)
    assert np.array_equal(c, np.where(signs > 0, 15, 0))
    q, c2, mean = orc.double_quantize(absmax)
    assert np.all(c2 == 0) and np.all(q == 0) and mean[0] == np.float32(0.03125)
    out = orc.nf4_dequantize(codes, q, c2, mean, (n,))
    assert np.array_equal(out.view(np.uint32), w.view(np.uint32))

    # random weights: zero level exact, extremes at +-c1' bit for bit
    w = (rng.standard_normal(64 * 500) * 0.02).astype(np.float32)
    w[64 * 7: 64 * 8] = 0.0                                   # a zero block
    n = w.size
    codes, absmax = orc.nf4_quantize(w)
    q, c2, mean = orc.double_quantize(absmax)
    c1p = np.repeat(orc.double_dequantize(q, c2, mean), 64)
    out = orc.nf4_dequantize(codes, q, c2, mean, (n,))
    c = _unpack(codes, n)
    assert np.all(out[c == 7] == 0.0)
    assert np.array_equal(out[c == 15].view(np.uint32), c1p[c == 15].view(np.uint32))
    assert np.array_equal(out[c == 0].view(np.uint32), (-c1p[c == 0]).view(np.uint32))
    assert np.all(c[64 * 7: 64 * 8] == 7)
    # every block holds its absmax element, code 0 or 15 (zero block aside)
    has_ext = np.array([np.any((c[b * 64:(b + 1) * 64] == 0) | (c[b * 64:(b + 1) * 64] == 15))
                        for b in range(n // 64)])
    assert np.all(has_ext | (absmax == 0))
    # re-encode with the decoded constants as absmax: the same codes
    blocks = out.reshape(-1, 64)
    bm = np.max(np.abs(blocks), axis=1)
    ok = bm > 0
    assert np.array_equal(bm[ok].view(np.uint32), np.abs(c1p.reshape(-1, 64)[ok, 0]).view(np.uint32))
    codes2, absmax2 = orc.nf4_quantize(out)
    ok_vals = np.repeat(ok & (c1p.reshape(-1, 64)[:, 0] > 0), 64)
    assert np.array_equal(_unpack(codes2, n)[ok_vals], c[ok_vals])


def test_dequantize_matches_definition(orc, nf4_levels):
    rng = np.random.Generator(np.random.PCG64(8))
    n = 64 * 300 + 17
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    codes, absmax = orc.nf4_quantize(w)
    q, c2, mean = orc.double_quantize(absmax)
    c1p = orc.double_dequantize(q, c2, mean)
    out = orc.nf4_dequantize(codes, q, c2, mean, (n,))
    ref = nf4_levels[_unpack(codes, n)] * np.repeat(c1p, 64)[:n]   # one fp32 product each
    assert np.array_equal(out.view(np.uint32), ref.astype(np.float32).view(np.uint32))
    # the dequantized weight tracks the original within the 4-bit grid's reach
    err = np.abs(out - w) / np.repeat(absmax, 64)[:n]
    assert np.max(err) < 0.2
