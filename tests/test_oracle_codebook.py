"""Pins for the oracle's NF4 codebook and quantizer statistics.

What the pages fix ("NF4, derived from normal quantiles", zerotofrontier.app
PEFT page): 16 levels, an exact zero, 8 positive and 7 negative quantile
levels, extremes +-1, probabilities from p = 0.9677 (the average of 1-1/30 and
1-1/32) down to 1/2, finer steps on the positive side, and the page's own
experiment on Gaussian blocks of 64: NF4 uses 3.88 of 4 bits of code entropy
against 3.50 for the symmetric int4 grid {-7..7}/7, cuts RMS error by about
15%, and the MSE-optimal (Lloyd) codebook is only about 5% better still.
"""
import numpy as np
import pytest
from scipy.special import ndtri

PMAX = ((1 - 1 / 30) + (1 - 1 / 32)) / 2


def test_ppf_matches_library_routine(orc):
    # AS 241 against scipy's ndtri (a different implementation) over a dense grid;
    # a wrong coefficient would show up far above a few float64 ulps
    ps = np.concatenate([np.linspace(1e-12, 1 - 1e-12, 20001),
                         PMAX - np.arange(9) * (PMAX - 0.5) / 8,
                         PMAX - np.arange(8) * (PMAX - 0.5) / 7])
    for p in ps:
        a, b = orc.norm_ppf(p), ndtri(p)
        assert abs(a - b) <= 2e-15 * max(1.0, abs(b)), (p, a, b)


def test_codebook_invariants(nf4_levels):
    lv = nf4_levels
    assert lv.dtype == np.float32 and lv.shape == (16,)
    assert np.all(np.diff(lv.astype(np.float64)) > 0), "strictly ascending"
    assert lv[7] == 0.0 and not np.signbit(lv[7]), "exact zero at code 7"
    assert lv[0] == -1.0 and lv[15] == 1.0, "extremes +-1"
    assert (lv > 0).sum() == 8 and (lv < 0).sum() == 7
    # the positive side has one more level, so its steps are finer
    pos_steps = np.diff(lv[7:].astype(np.float64))     # 8 steps from 0 to +1
    neg_steps = np.diff(lv[:8].astype(np.float64))     # 7 steps from -1 to 0
    assert pos_steps.mean() < neg_steps.mean()
    assert pos_steps.max() < neg_steps.max()


def test_codebook_matches_library_quantiles(nf4_levels):
    # the same construction with the library's inverse CDF gives the same fp32 table
    top = ndtri(PMAX)
    pos = [ndtri(PMAX - i * (PMAX - 0.5) / 8) for i in range(8)]
    neg = [-ndtri(PMAX - i * (PMAX - 0.5) / 7) for i in range(7)]
    ref = (np.array(sorted(pos + neg + [0.0])) / top).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), nf4_levels.view(np.uint32))


def test_offset_reading(nf4_levels):
    # the page quotes p = 0.9677; the exact average of 1-1/30 and 1-1/32 rounds to it
    assert round(PMAX, 4) == 0.9677
    # the rounded print would shift the levels by ~1e-5 only
    top = ndtri(0.9677)
    alt = np.array(sorted([ndtri(0.9677 - i * (0.9677 - 0.5) / 8) for i in range(8)]
                          + [-ndtri(0.9677 - i * (0.9677 - 0.5) / 7) for i in range(7)] + [0.0])) / top
    assert np.max(np.abs(alt - nf4_levels)) < 5e-5


def _entropy(codes_u4):
    h = np.bincount(codes_u4, minlength=16).astype(np.float64)
    p = h[h > 0] / h.sum()
    return float(-(p * np.log2(p)).sum())


def _unpack(codes, n):
    out = np.empty(codes.size * 2, np.uint8)
    out[0::2] = codes & 0xF
    out[1::2] = codes >> 4
    return out[:n]


@pytest.fixture(scope="module")
def gaussian_blocks(orc):
    rng = np.random.Generator(np.random.PCG64(0))
    w = rng.standard_normal(1 << 22).astype(np.float32)
    codes, absmax = orc.nf4_quantize(w)
    return w, _unpack(codes, w.size), absmax


def test_page_statistics_entropy(gaussian_blocks):
    # "3.88 of 4 possible bits of entropy, against 3.50" (page experiment, blocks of 64)
    w, codes, absmax = gaussian_blocks
    assert abs(_entropy(codes) - 3.88) < 0.01
    c = np.repeat(absmax, 64)[: w.size]
    int4 = np.rint(w / c * 7).astype(np.int64) + 7          # symmetric grid {-7..7}/7
    assert abs(_entropy(int4) - 3.50) < 0.01


def test_page_statistics_rms(gaussian_blocks, nf4_levels):
    # "NF4 cuts the RMS error by about 15% relative to symmetric int4"
    w, codes, absmax = gaussian_blocks
    c = np.repeat(absmax, 64)[: w.size].astype(np.float64)
    x = w.astype(np.float64) / c
    nf4 = nf4_levels.astype(np.float64)[codes]
    rms_nf4 = np.sqrt(np.mean(((nf4 - x) * c) ** 2))
    rms_int4 = np.sqrt(np.mean(((np.rint(x * 7) / 7 - x) * c) ** 2))
    gain = 1 - rms_nf4 / rms_int4
    assert 0.12 < gain < 0.18, gain
    # "The MSE-optimal codebook is only about 5% better still" (Lloyd, 1-D k-means
    # on the normalised values, weighted by c^2 so that it minimises weight-space MSE)
    cb = nf4_levels.astype(np.float64).copy()
    wgt = c * c
    for _ in range(40):
        idx = np.searchsorted((cb[1:] + cb[:-1]) / 2, x)
        num = np.bincount(idx, weights=x * wgt, minlength=16)
        den = np.bincount(idx, weights=wgt, minlength=16)
        cb = np.where(den > 0, num / np.maximum(den, 1e-300), cb)
    idx = np.searchsorted((cb[1:] + cb[:-1]) / 2, x)
    rms_lloyd = np.sqrt(np.mean(((cb[idx] - x) * c) ** 2))
    lloyd_gain = 1 - rms_lloyd / rms_nf4
    assert 0.03 < lloyd_gain < 0.07, lloyd_gain


def test_equal_mass_levels(orc):
    # NF4 places its levels at equal-probability quantiles: N(0,1) data normalised
    # by the top quantile uses every level at near-equal frequency.
    rng = np.random.Generator(np.random.PCG64(1))
    top = np.float32(ndtri(PMAX))
    nblk = 1 << 15
    v = rng.standard_normal((nblk, 63)).astype(np.float32)
    v = np.clip(v, -top, top)
    w = np.concatenate([v, np.full((nblk, 1), top, np.float32)], axis=1)  # absmax == top
    codes, absmax = orc.nf4_quantize(w.reshape(-1))
    assert np.all(absmax == top)
    cu = _unpack(codes, w.size).reshape(nblk, 64)[:, :63].reshape(-1)
    freq = np.bincount(cu, minlength=16) / cu.size
    assert freq.min() > 0.05 and freq.max() < 0.08, freq
    assert _entropy(cu) > 3.98
