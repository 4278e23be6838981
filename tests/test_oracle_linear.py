"""Pins for the oracle's QLoRA linear forward and backward.

Forward ("Putting it together", prism.theerrors.in QLoRA explainer, and "Paged
optimizers, and QLoRA end to end", zerotofrontier.app PEFT page):
Y = X dequant(W)^T + (alpha/r) (X A^T) B^T.  Backward: gradients flow through
the dequantized frozen weight to X and into the adapters A and B only.
"""
import numpy as np
import pytest


def _rand(rng, *shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


@pytest.fixture(scope="module")
def small():
    rng = np.random.Generator(np.random.PCG64(11))
    M, N, K, r = 9, 40, 128, 8
    return dict(Wd=_rand(rng, N, K, scale=0.02), X=_rand(rng, M, K), A=_rand(rng, r, K, scale=0.1),
                B=_rand(rng, N, r, scale=0.05), dY=_rand(rng, M, N), alpha=16.0)


def test_forward_matches_library_gemm(orc, small):
    s = small
    Y, T = orc.qlora_linear_fwd(s["Wd"], s["X"], s["A"], s["B"], s["alpha"])
    X, W, A, B = (s[k].astype(np.float64) for k in ("X", "Wd", "A", "B"))
    sc = s["alpha"] / A.shape[0]
    assert np.allclose(T, X @ A.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(Y, X @ W.T + sc * (X @ A.T) @ B.T, rtol=1e-12, atol=1e-12)


def test_forward_special_cases(orc, small):
    s = small
    X, W = s["X"].astype(np.float64), s["Wd"].astype(np.float64)
    Y0, _ = orc.qlora_linear_fwd(s["Wd"], s["X"], s["A"], np.zeros_like(s["B"]), s["alpha"])
    assert np.allclose(Y0, X @ W.T, rtol=1e-12, atol=1e-12)          # B = 0: plain GEMM
    Yl, T = orc.qlora_linear_fwd(np.zeros_like(s["Wd"]), s["X"], s["A"], s["B"], s["alpha"])
    sc = s["alpha"] / s["A"].shape[0]
    assert np.allclose(Yl, sc * T @ s["B"].astype(np.float64).T, rtol=1e-12)  # W = 0: pure LoRA
    rows = np.array([4, 0, 8])
    Yr, _ = orc.qlora_linear_fwd(s["Wd"], s["X"], s["A"], s["B"], s["alpha"], rows=rows)
    Yf, _ = orc.qlora_linear_fwd(s["Wd"], s["X"], s["A"], s["B"], s["alpha"])
    assert np.array_equal(Yr, Yf[rows])


def test_backward_matches_library_gemm(orc, small):
    s = small
    dX, dA, dB = orc.qlora_linear_bwd(s["Wd"], s["X"], s["dY"], s["A"], s["B"], s["alpha"])
    X, W, A, B, G = (s[k].astype(np.float64) for k in ("X", "Wd", "A", "B", "dY"))
    sc = s["alpha"] / A.shape[0]
    U = G @ B
    assert np.allclose(dX, G @ W + sc * U @ A, rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, sc * U.T @ X, rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, sc * G.T @ (X @ A.T), rtol=1e-12, atol=1e-12)
    rows = np.array([1, 7])
    dXr, _, _ = orc.qlora_linear_bwd(s["Wd"], s["X"], s["dY"], s["A"], s["B"], s["alpha"],
                                     rows=rows, want_da=False, want_db=False)
    assert np.array_equal(dXr, dX[rows])


def test_backward_finite_differences(orc, small):
    """Central differences of L = <dY, Y(X, A, B)> in float64."""
    s = small
    X = s["X"].astype(np.float64)
    A = s["A"].astype(np.float64)
    B = s["B"].astype(np.float64)

    def loss(X_, A_, B_):
        Y, _ = orc.qlora_linear_fwd(s["Wd"], X_, A_, B_, s["alpha"])
        return float(np.sum(Y * s["dY"].astype(np.float64)))

    dX, dA, dB = orc.qlora_linear_bwd(s["Wd"], s["X"], s["dY"], s["A"], s["B"], s["alpha"])
    rng = np.random.Generator(np.random.PCG64(3))
    h = 0.25          # L is linear in X and in each adapter separately: exact up to rounding
    for name, P, G in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, d)) for d in P.shape)
            Pp, Pm = P.copy(), P.copy()
            # the oracle takes fp32 operands: use the perturbations fp32 can hold exactly
            Pp[idx] = np.float32(P[idx] + h)
            Pm[idx] = np.float32(P[idx] - h)
            hp, hm = Pp[idx] - P[idx], P[idx] - Pm[idx]
            args_p = {"X": X, "A": A, "B": B}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Pp, Pm
            fd = (loss(args_p["X"], args_p["A"], args_p["B"])
                  - loss(args_m["X"], args_m["A"], args_m["B"])) / (hp + hm)
            assert abs(fd - G[idx]) <= 1e-9 * max(1.0, abs(G[idx])), (name, idx, fd, G[idx])


def test_no_gradient_reaches_frozen_weight(orc, small):
    # the backward returns exactly dX, dA, dB: the 4-bit weights are constants
    out = orc.qlora_linear_bwd(small["Wd"], small["X"], small["dY"], small["A"], small["B"],
                               small["alpha"])
    assert len(out) == 3


def test_empty_token_batch(orc, small):
    s = small
    X0 = np.zeros((0, s["X"].shape[1]), np.float32)
    dY0 = np.zeros((0, s["dY"].shape[1]), np.float32)
    Y, T = orc.qlora_linear_fwd(s["Wd"], X0, s["A"], s["B"], s["alpha"])
    assert Y.shape == (0, s["Wd"].shape[0]) and T.shape == (0, s["A"].shape[0])
    dX, dA, dB = orc.qlora_linear_bwd(s["Wd"], X0, dY0, s["A"], s["B"], s["alpha"])
    assert dX.shape[0] == 0 and np.all(dA == 0) and np.all(dB == 0)
