"""GPU parity of the rank-r truncated SVD and the LoftQ-style initialisation.

"Paged optimizers, and QLoRA end to end" (zerotofrontier.app "sft/peft", closing remark
on LoftQ, Li et al. 2023): start the adapter so that dequant(W^NF4) + gamma B A is close
to W.  The GPU alternates the codec kernels with a randomized rank-r SVD of the
quantization error (subspace iteration with a caller-drawn Gaussian test matrix); the
oracle uses the exact truncated SVD (one-sided Jacobi, float64).

What is unique is compared: with a clear gap between the r-th and the next singular
value the rank-r approximation itself is unique and matched element by element; without
one (a quantization error is noise-like, its spectrum flat) only the singular values and
the residual norm are determined, and the randomized result captures at most the exact
energy (it approaches it from below) and is held to a small relative gap.  The codes of
the first alternation (the weight itself quantized) are bit-exact; the final quantized
weight and the bf16 adapter are evaluated on the host against W.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_09_amd as nf4
import oracle
from workloads import Draw, seed_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _omega(K, l, seed):
    return Draw(seed, DEV).normal((K, l), 1.0)


def _planted(m, n, s, noise, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    Qa, _ = np.linalg.qr(rng.standard_normal((m, len(s))))
    Qb, _ = np.linalg.qr(rng.standard_normal((n, len(s))))
    E = (Qa * s) @ Qb.T + noise * rng.standard_normal((m, n))
    return E.astype(np.float32)


@pytest.mark.parametrize("m,n,r,l", [(300, 200, 8, 24), (96, 700, 16, 40), (512, 320, 32, 48), (260, 260, 64, 96)])
def test_lowrank_svd_planted_gap(m, n, r, l):
    # singular values r.. fall by 10x below the r-th: the rank-r approximation is unique
    s = np.concatenate([np.linspace(40.0, 10.0, r), np.linspace(1.0, 0.5, 8)])
    E = _planted(m, n, s, 1e-3, seed_of(60, m, n))
    print("lowrank planted", m, n, r, l, flush=True)
    U, S, V = nf4.nf4_lowrank_svd(torch.from_numpy(E).to(DEV), r, _omega(n, l, seed_of(61, n, l)), power_iters=3)
    torch.cuda.synchronize()
    U, S, V = (t.cpu().numpy().astype(np.float64) for t in (U, S, V))
    So, Uo, Vto = oracle.svd_topr(E.astype(np.float64), r)
    np.testing.assert_allclose(S, So, rtol=2e-5)
    P, Po = (U * S) @ V.T, (Uo * So) @ Vto
    assert np.linalg.norm(P - Po) <= 1e-4 * np.linalg.norm(Po)
    np.testing.assert_allclose(U.T @ U, np.eye(r), atol=2e-5)
    np.testing.assert_allclose(V.T @ V, np.eye(r), atol=2e-5)


@pytest.mark.parametrize("m,n,r,l", [(256, 192, 8, 24), (200, 300, 16, 32)])
def test_lowrank_svd_flat_spectrum(m, n, r, l):
    # a Gaussian matrix: no gap, so only the energies are determined.  Subspace iteration
    # captures a share of the exact top-r energy that rises with the power iterations
    # (Halko et al. 2011, section 4.5): for these matrices and test matrices, evaluated in
    # float64, 0.947 / 0.953 after 2 and 0.9967 / 0.9971 after 6
    E = np.random.Generator(np.random.PCG64(seed_of(62, m, n))).standard_normal((m, n)).astype(np.float32)
    So, _, _ = oracle.svd_topr(E.astype(np.float64), r)
    caps = []
    for power, floor in ((2, 0.93), (6, 0.99)):
        U, S, V = nf4.nf4_lowrank_svd(torch.from_numpy(E).to(DEV), r, _omega(n, l, seed_of(63, n)), power_iters=power)
        torch.cuda.synchronize()
        U, S, V = (t.cpu().numpy().astype(np.float64) for t in (U, S, V))
        assert np.all(S <= So * (1 + 1e-5))                 # Ritz values approach from below
        cap = np.sum(S ** 2) / np.sum(So ** 2)
        assert cap >= floor, (power, cap)
        caps.append(cap)
        # the factors reproduce their own singular values: U^T E V = diag(S)
        np.testing.assert_allclose(U.T @ E.astype(np.float64) @ V, np.diag(S), atol=1e-4 * So[0])
    assert caps[1] > caps[0]


def test_lowrank_svd_rank_deficient():
    # rank 3 with r = 8: the 5 missing directions come out as zero singular values
    E = _planted(128, 96, np.array([5.0, 3.0, 1.0]), 0.0, seed_of(64))
    U, S, V = nf4.nf4_lowrank_svd(torch.from_numpy(E).to(DEV), 8, _omega(96, 16, seed_of(65)), power_iters=2)
    torch.cuda.synchronize()
    S = S.cpu().numpy()
    np.testing.assert_allclose(S[:3], [5.0, 3.0, 1.0], rtol=1e-5)
    assert np.all(np.abs(S[3:]) < 1e-4)
    P = (U.cpu().numpy() * S) @ V.cpu().numpy().T
    np.testing.assert_allclose(P, E, atol=1e-5)


def _host_error(W, Wq, A, B, gamma):
    Wd = nf4.nf4_dequantize(Wq, torch.float32).cpu().numpy().astype(np.float64)
    BA = B.float().cpu().numpy().astype(np.float64) @ A.float().cpu().numpy().astype(np.float64)
    return np.linalg.norm(W.astype(np.float64) - Wd - gamma * BA)


@pytest.mark.parametrize("N,K,r,l,iters", [(256, 192, 8, 24, 3), (192, 512, 16, 40, 4)])
def test_loftq_matches_oracle(N, K, r, l, iters):
    alpha = 16.0
    gamma = alpha / r
    W = Draw(seed_of(66, N, K), "cpu").normal((N, K), 0.02, outlier_frac=0.01).numpy()
    print("loftq", N, K, r, l, iters, flush=True)
    Wq, A, B, err = nf4.loftq_init(torch.from_numpy(W).to(DEV), r, alpha, _omega(K, l, seed_of(67, K)), iters=iters,
                                   power_iters=4)
    torch.cuda.synchronize()
    err = err.cpu().numpy()
    ref = oracle.loftq(W, r, gamma, iters)
    # first alternation: W itself quantized (bit-exact), then the SVD of its quantization error
    one = oracle.loftq(W, r, gamma, 1)
    Wq1, _, _, err1 = nf4.loftq_init(torch.from_numpy(W).to(DEV), r, alpha, _omega(K, l, seed_of(67, K)), iters=1,
                                     power_iters=4)
    torch.cuda.synchronize()
    assert np.array_equal(Wq1.codes.cpu().numpy(), one["codes"])
    assert np.array_equal(Wq1.q.cpu().numpy(), one["q"])
    assert np.array_equal(Wq1.c2.cpu().numpy().view(np.uint32), one["c2"].view(np.uint32))
    e1 = float(err1.cpu().numpy()[0])
    assert one["err"][0] * (1 - 1e-6) <= e1 <= one["err"][0] * (1 + 2e-3), (e1, one["err"][0])
    # the whole trajectory: each alternation's residual norm close to the exact method's
    np.testing.assert_allclose(err, ref["err"], rtol=5e-3)
    assert err[-1] < err[0]
    # the outputs as the layer will use them: dequant(Q) + gamma bf16(B) bf16(A) against W
    e_host = _host_error(W, Wq, A, B, gamma)
    plain = np.linalg.norm(W.astype(np.float64) - oracle.nf4_dequantize(
        one["codes"], one["q"], one["c2"], one["mean"], W.shape).astype(np.float64))
    assert e_host < plain                                   # the adapter absorbs part of the error
    assert abs(e_host - err[-1]) <= 0.02 * err[-1]          # bf16 rounding of the factors aside


def test_loftq_zero_weight():
    W = torch.zeros((64, 128), dtype=torch.float32, device=DEV)
    Wq, A, B, err = nf4.loftq_init(W, 8, 16.0, _omega(128, 16, seed_of(68)), iters=2)
    torch.cuda.synchronize()
    assert torch.all(err == 0).item() and torch.all(A.float() == 0).item() and torch.all(B.float() == 0).item()
    assert torch.all(Wq.codes == 0x77).item()
