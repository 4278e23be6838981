"""GPU parity of the QLoRA linear forward and backward against the float64
oracle ("Putting it together", prism.theerrors.in QLoRA explainer; "Paged
optimizers, and QLoRA end to end", zerotofrontier.app PEFT page):
Y = X W'^T + (alpha/r) (X A^T) B^T, dX = dY W' + s U A, dA = s U^T X,
dB = s dY^T T.  Element by element at sizes that span several 256-wide tiles
with ragged tails, and on sampled rows (the oracle computes them one by one)
at the full LLaMA-7B / LLaMA-65B shapes in the launch configuration the
benchmark times.  The NF4 codes of each weight are checked bit-exact first.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_09_amd as nf4
import oracle
from parity import assert_close, oracle_weight, to_np
from workloads import Draw, host_f32, linear_inputs, seed_of, tiny_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(W, X, A, B, dY, alpha, rows=None, check_codes=True, save_t=True, double_quant=True):
    """GPU fwd+bwd on device tensors, oracle on host copies; returns the metrics.  With
    double_quant=False the weight keeps plain fp32 constants on both sides."""
    print("linear case N=%d K=%d M=%d r=%d rows=%s dq=%s" % (W.shape[0], W.shape[1], X.shape[0],
                                                             A.shape[0], None if rows is None else len(rows),
                                                             double_quant), flush=True)
    ref = oracle_weight(W.cpu())
    Wq = nf4.quantize_weight(W, double_quant=double_quant)
    if not double_quant:
        ref = dict(ref)
        ref["Wd"] = oracle.nf4_dequantize_plain(ref["codes"], ref["absmax"], tuple(W.shape))
    if check_codes:
        assert np.array_equal(Wq.codes.cpu().numpy(), ref["codes"])
        if double_quant:
            assert np.array_equal(Wq.q.cpu().numpy(), ref["q"])
        else:
            assert np.array_equal(Wq.absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32))
    Y, T = nf4.qlora_linear_fwd(Wq, X, A, B, alpha, save_t=save_t)
    dX, dA, dB = nf4.qlora_linear_bwd(Wq, X, dY, A, B, alpha, T=T)
    torch.cuda.synchronize()
    Xh, Ah, Bh, dYh = (host_f32(t) for t in (X, A, B, dY))
    Yr, Tr = oracle.qlora_linear_fwd(ref["Wd"], Xh, Ah, Bh, alpha, rows=rows)
    dXr, dAr, dBr = oracle.qlora_linear_bwd(ref["Wd"], Xh, dYh, Ah, Bh, alpha, rows=rows)
    sel = slice(None) if rows is None else rows
    out = {}
    out["Y"] = assert_close("Y", to_np(Y)[sel], Yr)
    if T is not None:
        out["T"] = assert_close("T", to_np(T), Tr)
    out["dX"] = assert_close("dX", to_np(dX)[sel], dXr)
    out["dA"] = assert_close("dA", to_np(dA), dAr)
    out["dB"] = assert_close("dB", to_np(dB), dBr)
    return out


def test_tiny_layer():
    W, X, A, B, dY = (t.to(DEV) for t in tiny_inputs())
    _run(W, X, A, B, dY, alpha=16.0)


# Launches of a few tiles cut every tile into contraction pieces; (8, 64, 33, 8) has a
# single step (no pieces) and the 136-tile forward of (2048, 128, 4352, 16) runs whole
# tiles only, while its 17-tile dX runs pieces.
@pytest.mark.parametrize("N,K,M,r", [(328, 320, 300, 8), (256, 512, 257, 64), (520, 192, 513, 128),
                                     (264, 256, 40, 24), (8, 64, 33, 8), (2048, 128, 4352, 16)])
def test_ragged_gemm_path(N, K, M, r):
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(10, N, K, M, r)))
    _run(W, X, A, B, dY, alpha=16.0)


@pytest.mark.parametrize("M", [1, 2, 4, 5, 16])
@pytest.mark.parametrize("N,K", [(200, 512), (1032, 1088)])
def test_gemv_path(M, N, K):
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, 64, seed=seed_of(11, N, K, M)))
    _run(W, X, A, B, dY, alpha=16.0)


@pytest.mark.parametrize("M,N,K,r", [(3, 72, 576, 24), (1, 16, 65600, 8), (16, 48, 65600, 40),
                                     (7, 24, 1088, 120)])
def test_gemv_ranks_and_long_rows(M, N, K, r):
    # adapter ranks that are not a multiple of 32, rows whose 256-blocks of second-level
    # constants outnumber the per-workgroup cache (K > 64512), odd block counts per row
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(13, N, K, M, r)))
    _run(W, X, A, B, dY, alpha=16.0)


@pytest.mark.parametrize("M", [1, 5])
def test_gemv_second_level_groups(M):
    # an odd number of blocks per row (17) puts block pairs across the boundaries of the
    # 256-block groups of second-level constants; rows scaled over four decades give the
    # groups different constants, and every output row is held to the tolerance on its
    # own, so a block decoded with its neighbouring group's constant shows
    N, K, r = 256, 1088, 16
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(14, M)))
    g = torch.Generator().manual_seed(seed_of(15, M))
    scale = (10.0 ** (4.0 * torch.rand(N, 1, generator=g) - 2.0)).to(DEV)
    W = W * scale
    B = (B.float() * 1e-2).to(torch.bfloat16)      # keep the rank-r term below the smallest rows
    print("gemv groups", N, K, M, flush=True)
    ref = oracle_weight(W.cpu())
    Wq = nf4.quantize_weight(W)
    Y, T = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0)
    torch.cuda.synchronize()
    Yr, Tr = oracle.qlora_linear_fwd(ref["Wd"], host_f32(X), host_f32(A), host_f32(B), 16.0)
    err = np.abs(to_np(Y) - Yr).max(axis=0)
    # the natural size of output row n: the norm of its dequantized weight row (X ~ N(0, 1))
    row_norm = np.linalg.norm(ref["Wd"], axis=1)
    worst = int(np.argmax(err / row_norm))
    assert err[worst] <= 2e-2 * row_norm[worst], "row %d: error %.3e, row norm %.3e" % (
        worst, err[worst], row_norm[worst])


def test_backward_rows_stay_apart():
    # dX contracts over N = 72: the last 64-value step holds 8 real columns. An infinite
    # value at the start of dY's row 1 sits right after row 0's last column in memory; row 0
    # of dX (and every other row but 1) must not see it: the packed dY holds zeros past N.
    N, K, M, r = 72, 128, 40, 8
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(16)))
    dY[1, 0] = float("inf")
    ref = oracle_weight(W.cpu())
    Wq = nf4.quantize_weight(W)
    dX, dA, dB = nf4.qlora_linear_bwd(Wq, X, dY, A, B, 16.0)
    torch.cuda.synchronize()
    dXr, _, _ = oracle.qlora_linear_bwd(ref["Wd"], host_f32(X), host_f32(dY), host_f32(A), host_f32(B), 16.0,
                                        want_da=False, want_db=False)
    keep = [m for m in range(M) if m != 1]
    got = to_np(dX)[keep]
    assert np.all(np.isfinite(got)), "a row other than 1 saw the infinite value"
    assert_close("dX", got, dXr[keep])


def test_gemv_and_gemm_paths_agree():
    # 16 tokens run through the dequant-GEMV; the same 16 plus one more run through the GEMM
    N, K, r = 520, 1024, 64
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, 17, r, seed=seed_of(12)))
    Wq = nf4.quantize_weight(W)
    Y16, T16 = nf4.qlora_linear_fwd(Wq, X[:16].contiguous(), A, B, 16.0)
    Y17, T17 = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0)
    assert_close("gemv vs gemm", to_np(Y16), to_np(Y17[:16]), fro_tol=5e-3, elem_tol=2e-2)
    assert_close("T", to_np(T16), to_np(T17[:16]), fro_tol=5e-3, elem_tol=2e-2)


def test_special_cases():
    N, K, M, r = 256, 256, 64, 16
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(13)))
    # B = 0: the plain dequant product
    _run(W, X, A, torch.zeros_like(B), dY, alpha=16.0)
    # alpha = 0: no adapter contribution, zero adapter gradients
    Wq = nf4.quantize_weight(W)
    Y, _ = nf4.qlora_linear_fwd(Wq, X, A, B, 0.0)
    Y0, _ = nf4.qlora_linear_fwd(Wq, X, A, torch.zeros_like(B), 16.0)
    assert torch.equal(Y, Y0)
    _, dA, dB = nf4.qlora_linear_bwd(Wq, X, dY, A, B, 0.0)
    assert torch.all(dA == 0).item() and torch.all(dB == 0).item()
    # W = 0: pure LoRA
    _run(torch.zeros_like(W), X, A, B, dY, alpha=16.0)


def test_backward_recomputes_t_and_skips_dx():
    N, K, M, r = 264, 320, 96, 64
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(14)))
    Wq = nf4.quantize_weight(W)
    Y, T = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0)
    dX1, dA1, dB1 = nf4.qlora_linear_bwd(Wq, X, dY, A, B, 16.0, T=T)
    dX2, dA2, dB2 = nf4.qlora_linear_bwd(Wq, X, dY, A, B, 16.0, T=None)
    _, dA3, dB3 = nf4.qlora_linear_bwd(Wq, X, dY, A, B, 16.0, T=T, need_dx=False)
    assert torch.equal(dX1, dX2) and torch.equal(dA1, dA2) and torch.equal(dB1, dB2)
    assert torch.equal(dA1, dA3) and torch.equal(dB1, dB3)
    Y2, T2 = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0, save_t=False)
    assert T2 is None and torch.equal(Y, Y2)


def test_empty_token_batch():
    N, K, r = 256, 256, 8
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, 4, r, seed=seed_of(15)))
    Wq = nf4.quantize_weight(W)
    X0 = X[:0].contiguous()
    dY0 = dY[:0].contiguous()
    Y, T = nf4.qlora_linear_fwd(Wq, X0, A, B, 16.0)
    assert Y.shape == (0, N)
    dX, dA, dB = nf4.qlora_linear_bwd(Wq, X0, dY0, A, B, 16.0)
    torch.cuda.synchronize()
    assert dX.shape == (0, K) and torch.all(dA == 0).item() and torch.all(dB == 0).item()


def test_deterministic():
    N, K, M, r = 512, 512, 512, 64
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(16)))
    Wq = nf4.quantize_weight(W)
    a = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0) + nf4.qlora_linear_bwd(Wq, X, dY, A, B, 16.0)
    b = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0) + nf4.qlora_linear_bwd(Wq, X, dY, A, B, 16.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _sampled_rows(M, per_band, seed, band=32):
    """`per_band` random token rows out of every `band` consecutive rows, plus the first
    and the last.  With band = 32 every 32-row MFMA tile of every wave (a wave owns 128
    rows of a 512-row output tile) contributes a row; with band = 128, every wave of
    every output tile."""
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = [[0, M - 1]]
    for b0 in range(0, M, band):
        picks.append(b0 + rng.integers(0, min(band, M - b0), per_band))
    return np.unique(np.concatenate(picks)).astype(np.int64)


@pytest.mark.parametrize("proj", ["q", "gate", "down"])
def test_full_llama7b_shapes_sampled(proj):
    from workloads import LLAMA7B, layer_projections
    (name, N, K), = [p for p in layer_projections(LLAMA7B["d"], LLAMA7B["ffn"]) if p[0] == proj]
    M = 2048
    W, X, A, B, dY = linear_inputs(N, K, M, 64, seed=seed_of(20, N, K), device=DEV)
    _run(W, X, A, B, dY, alpha=16.0, rows=_sampled_rows(M, 1, 1))


@pytest.mark.parametrize("proj", ["q", "gate", "down"])
def test_full_llama65b_shapes_sampled(proj):
    # one row out of every 32-row MFMA tile of every wave and output tile (128 of 4096)
    from workloads import LLAMA65B, layer_projections
    (name, N, K), = [p for p in layer_projections(LLAMA65B["d"], LLAMA65B["ffn"]) if p[0] == proj]
    M = 4096
    W, X, A, B, dY = linear_inputs(N, K, M, 64, seed=seed_of(21, N, K), device=DEV)
    _run(W, X, A, B, dY, alpha=16.0, rows=_sampled_rows(M, 1, 2))


def test_llama65b_layer_chain_sampled():
    # The 65B layer as the benchmark runs it: the seven forwards in layer order (q, k, v,
    # o, gate, up, down), each saving T, then the seven backwards in reverse order with
    # the saved T; every output against the oracle, Y and dX on two rows of every wave of
    # every 512-row output tile, T, dA and dB in full
    from workloads import LLAMA65B, layer_projections
    M, r, alpha = 4096, 64, 16.0
    projs = layer_projections(LLAMA65B["d"], LLAMA65B["ffn"])
    rows = _sampled_rows(M, 2, 25, band=128)
    layer = []
    for i, (name, N, K) in enumerate(projs):
        W, X, A, B, dY = linear_inputs(N, K, M, r, seed=seed_of(25, i), device=DEV)
        layer.append(dict(name=name, W=W, Wq=nf4.quantize_weight(W), X=X, A=A, B=B, dY=dY))
    for p in layer:
        print("chain forward", p["name"], flush=True)
        p["Y"], p["T"] = nf4.qlora_linear_fwd(p["Wq"], p["X"], p["A"], p["B"], alpha)
    for p in reversed(layer):
        print("chain backward", p["name"], flush=True)
        p["dX"], p["dA"], p["dB"] = nf4.qlora_linear_bwd(p["Wq"], p["X"], p["dY"], p["A"], p["B"], alpha, T=p["T"])
    torch.cuda.synchronize()
    for p in layer:
        print("chain oracle", p["name"], flush=True)
        ref = oracle_weight(p["W"].cpu())
        assert np.array_equal(p["Wq"].codes.cpu().numpy(), ref["codes"]), p["name"]
        assert np.array_equal(p["Wq"].q.cpu().numpy(), ref["q"]), p["name"]
        Xh, Ah, Bh, dYh = (host_f32(t) for t in (p["X"], p["A"], p["B"], p["dY"]))
        Yr, Tr = oracle.qlora_linear_fwd(ref["Wd"], Xh, Ah, Bh, alpha, rows=rows)
        dXr, dAr, dBr = oracle.qlora_linear_bwd(ref["Wd"], Xh, dYh, Ah, Bh, alpha, rows=rows)
        assert_close(p["name"] + " Y", to_np(p["Y"])[rows], Yr)
        assert_close(p["name"] + " T", to_np(p["T"]), Tr)
        assert_close(p["name"] + " dX", to_np(p["dX"])[rows], dXr)
        assert_close(p["name"] + " dA", to_np(p["dA"]), dAr)
        assert_close(p["name"] + " dB", to_np(p["dB"]), dBr)
        for k in ("W", "Wq", "X", "dY", "Y", "dX"):
            p[k] = None


@pytest.mark.parametrize("N,K", [(8, (1 << 22) - 64), ((1 << 22) - 8, 64)])
def test_longest_operand_rows(N, K):
    # The largest N and K the ABI accepts (below 2^22): X rows of length K (forward) and dY
    # rows of length N (backward) as long as they get, with every byte offset of every kernel
    # below 2^31 (an earlier form of the fused product read its token operand through one
    # 2^31-byte range, and the last rows of its 512-row tiles lost their products past it);
    # eight rows of every wave of the 512-row tile are compared
    M = 512
    W, X, A, B, dY = linear_inputs(N, K, M, 8, seed=seed_of(24, N, K), device=DEV)
    _run(W, X, A, B, dY, alpha=16.0, rows=_sampled_rows(M, 8, 3, band=128))


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("N,K", [(8, (1 << 22) - 64), ((1 << 22) - 8, 64)])
def test_gemv_longest_rows(M, N, K):
    # the few-token forward at the largest N and K the ABI accepts: token rows of 2^22 - 64
    # values (every byte offset below 2^31), and rows of a single block (one block pair
    # whose second block lies past the row); every output compared
    W, X, A, B, dY = linear_inputs(N, K, M, 8, seed=seed_of(25, N, K, M), device=DEV)
    print("gemv longest", N, K, M, flush=True)
    ref = oracle_weight(W.cpu())
    Wq = nf4.quantize_weight(W)
    Y, T = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0)
    torch.cuda.synchronize()
    Yr, Tr = oracle.qlora_linear_fwd(ref["Wd"], host_f32(X), host_f32(A), host_f32(B), 16.0)
    assert_close("Y", to_np(Y), Yr)
    assert_close("T", to_np(T), Tr)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("N,K", [(8192, 8192), (22016, 8192), (8192, 22016)])
def test_full_gemv_shapes(M, N, K):
    W, X, A, B, dY = linear_inputs(N, K, M, 64, seed=seed_of(22, N, K, M), device=DEV)
    print("gemv full", N, K, M, flush=True)
    ref = oracle_weight(W.cpu())
    Wq = nf4.quantize_weight(W)
    Y, T = nf4.qlora_linear_fwd(Wq, X, A, B, 16.0)
    torch.cuda.synchronize()
    Yr, Tr = oracle.qlora_linear_fwd(ref["Wd"], host_f32(X), host_f32(A), host_f32(B), 16.0)
    assert_close("Y", to_np(Y), Yr)
    assert_close("T", to_np(T), Tr)


@pytest.mark.parametrize("M,N,K,r", [(300, 328, 320, 8), (257, 256, 512, 64), (1, 200, 512, 64),
                                     (4, 1032, 1088, 16), (16, 1032, 1088, 64), (5, 48, 65600, 40)])
def test_double_quantization_off(M, N, K, r):
    # [DQ] off: plain fp32 constants through the fused GEMM (M > 16) and the few-token
    # forward (M <= 16), against the oracle with w' = level * absmax
    W, X, A, B, dY = (t.to(DEV) for t in linear_inputs(N, K, M, r, seed=seed_of(40, N, K, M, r)))
    _run(W, X, A, B, dY, alpha=16.0, double_quant=False)
