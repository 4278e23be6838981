"""Pins of the oracle's rank-r truncated SVD and its LoftQ-style initialisation.

"Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft", closing remark on
LoftQ, Li et al. 2023): the adapter of a quantized base is started so that
dequant(W^NF4) + gamma B A is close to W.  The oracle alternates NF4 + double quantization
of the residual W - gamma B A with a rank-r truncated SVD (one-sided Jacobi) of the
quantization error.

The SVD is pinned to numpy's LAPACK SVD (a different algorithm: bidiagonalisation and
QR sweeps) and to the Eckart-Young identity ||E - E_r||_F^2 = sum_{i > r} s_i^2; the
alternation is pinned step by step to numpy evaluations of its definition.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("m,n,r", [(96, 64, 8), (64, 96, 8), (80, 80, 16), (33, 57, 5), (128, 40, 40)])
def test_svd_topr_matches_lapack(m, n, r):
    rng = np.random.Generator(np.random.PCG64(m * 1000 + n))
    E = rng.standard_normal((m, n))
    S, U, Vt = oracle.svd_topr(E, r)
    Ul, Sl, Vtl = np.linalg.svd(E, full_matrices=False)
    np.testing.assert_allclose(S, Sl[:r], rtol=1e-12)
    assert np.all(np.diff(S) <= 0)
    np.testing.assert_allclose(U.T @ U, np.eye(r), atol=1e-12)
    np.testing.assert_allclose(Vt @ Vt.T, np.eye(r), atol=1e-12)
    P = (U * S) @ Vt
    Pl = (Ul[:, :r] * Sl[:r]) @ Vtl[:r]
    np.testing.assert_allclose(P, Pl, atol=1e-10 * np.abs(E).max())
    # Eckart-Young: the residual of the best rank-r approximation
    assert abs(np.linalg.norm(E - P) ** 2 - np.sum(Sl[r:] ** 2)) <= 1e-9 * np.sum(Sl ** 2)


def test_svd_topr_planted_spectrum_and_rank_deficiency():
    rng = np.random.Generator(np.random.PCG64(5))
    m, n = 70, 50
    Qa, _ = np.linalg.qr(rng.standard_normal((m, m)))
    Qb, _ = np.linalg.qr(rng.standard_normal((n, n)))
    s = np.array([10.0, 10.0, 7.0, 3.0, 1e-3] + [0.0] * (n - 5))      # a repeated value, then rank 5
    E = (Qa[:, :n] * s) @ Qb.T
    S, U, Vt = oracle.svd_topr(E, 4)
    np.testing.assert_allclose(S, s[:4], rtol=1e-12)
    # the rank-4 approximation is unique (s_4 > s_5) even though s_1 = s_2
    P = (U * S) @ Vt
    np.testing.assert_allclose(P, (Qa[:, :4] * s[:4]) @ Qb[:, :4].T, atol=1e-11)
    S6, _, _ = oracle.svd_topr(E, 6)
    np.testing.assert_allclose(S6[:5], s[:5], rtol=1e-9, atol=1e-13)
    assert abs(S6[5]) < 1e-12


def _quant_error(W):
    codes, absmax = oracle.nf4_quantize(W.reshape(-1))
    q, c2, mean = oracle.double_quantize(absmax)
    Wd = oracle.nf4_dequantize(codes, q, c2, mean, W.shape)
    return (W - Wd).astype(np.float64), codes


def test_loftq_first_alternation_is_the_truncated_svd_of_the_quantization_error():
    rng = np.random.Generator(np.random.PCG64(21))
    N, K, r, gamma = 64, 128, 8, 2.0
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    out = oracle.loftq(W, r, gamma, 1)
    E, codes = _quant_error(W)
    assert np.array_equal(out["codes"], codes)                      # B A = 0: W itself is quantized
    Ul, Sl, Vtl = np.linalg.svd(E, full_matrices=False)
    np.testing.assert_allclose(gamma * out["B"] @ out["A"], (Ul[:, :r] * Sl[:r]) @ Vtl[:r], atol=1e-12)
    np.testing.assert_allclose(out["err"][0], np.sqrt(np.sum(Sl[r:] ** 2)), rtol=1e-10)
    # the scale is split evenly: column j of B and row j of A both have norm sqrt(s_j / gamma)
    np.testing.assert_allclose(np.linalg.norm(out["B"], axis=0), np.sqrt(Sl[:r] / gamma), rtol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(out["A"], axis=1), np.sqrt(Sl[:r] / gamma), rtol=1e-10)


def test_loftq_second_alternation_quantizes_the_residual():
    rng = np.random.Generator(np.random.PCG64(22))
    N, K, r, gamma = 48, 192, 6, 0.25
    # a weight with a strong low-rank part, so that the adapter moves the residual visibly
    W = (rng.standard_normal((N, K)) * 0.02 + 0.05 * np.outer(rng.standard_normal(N), rng.standard_normal(K)) / 8
         ).astype(np.float32)
    one = oracle.loftq(W, r, gamma, 1)
    two = oracle.loftq(W, r, gamma, 2)
    # the same first alternation in both calls (threaded float64 LAPACK may round its last
    # bit differently from call to call)
    np.testing.assert_allclose(two["err"][0], one["err"][0], rtol=1e-12, atol=0)
    R = (W.astype(np.float64) - gamma * one["B"] @ one["A"]).astype(np.float32)
    codes, absmax = oracle.nf4_quantize(R.reshape(-1))
    # a last-bit difference of the residual can move a code across a threshold: nearly all agree
    assert np.mean(codes == two["codes"]) > 0.999
    q, c2, mean = oracle.double_quantize(absmax)
    E = (W - oracle.nf4_dequantize(two["codes"], two["q"], two["c2"], two["mean"], W.shape)).astype(np.float64)
    Ul, Sl, Vtl = np.linalg.svd(E, full_matrices=False)
    np.testing.assert_allclose(two["err"][1], np.sqrt(np.sum(Sl[r:] ** 2)), rtol=1e-10)
    np.testing.assert_allclose(gamma * two["B"] @ two["A"], (Ul[:, :r] * Sl[:r]) @ Vtl[:r], atol=1e-12)
    # the adapter absorbs part of the quantization error: below plain NF4's
    E0, _ = _quant_error(W)
    assert two["err"][1] < np.linalg.norm(E0)


def test_loftq_zero_weight():
    # an all-zero weight quantizes exactly: zero error, zero adapter
    out = oracle.loftq(np.zeros((16, 64), np.float32), 4, 1.0, 2)
    assert np.all(out["err"] == 0) and np.all(out["B"] == 0) and np.all(out["A"] == 0)
    assert np.all(out["codes"] == 0x77)
