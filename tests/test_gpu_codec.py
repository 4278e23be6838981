"""GPU parity of the codec kernels against the oracle: NF4 codes, absmax, the
double-quantized constants (q, c2, mean) and their decode bit-exact; the
dequantized weight bit-exact in fp32 and equal to its round-to-nearest-even
bf16 value in bf16.  Covers ragged sizes, odd n, partial blocks, zero blocks,
exact midpoint ties, outliers, bf16 input, and the full LLaMA weight shapes.
"""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_09_amd as nf4
import oracle
from parity import oracle_weight
from workloads import Draw, bf16_bits, host_f32, seed_of

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_tuple(w_dev):
    codes, absmax = nf4.nf4_quantize(w_dev)
    q, c2, mean = nf4.nf4_double_quantize(absmax)
    return codes, absmax, q, c2, mean


def _assert_codec_equal(w_host, w_dev, check_dequant=True):
    ref = oracle_weight(w_host)
    codes, absmax, q, c2, mean = _gpu_tuple(w_dev)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ref["codes"]), "codes"
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32)), "absmax"
    assert np.array_equal(mean.cpu().numpy().view(np.uint32), ref["mean"].view(np.uint32)), "mean"
    assert np.array_equal(c2.cpu().numpy().view(np.uint32), ref["c2"].view(np.uint32)), "c2"
    assert np.array_equal(q.cpu().numpy(), ref["q"]), "q"
    if check_dequant:
        c1p = nf4.nf4_double_dequantize(q, c2, mean).cpu().numpy()
        c1p_ref = oracle.double_dequantize(ref["q"], ref["c2"], ref["mean"])
        assert np.array_equal(c1p.view(np.uint32), c1p_ref.view(np.uint32)), "c1'"
        if w_host.dim() == 2:
            W = nf4.NF4Weight(codes, q, c2, mean, tuple(w_host.shape))
            wd = nf4.nf4_dequantize(W, torch.float32).cpu().numpy()
            assert np.array_equal(wd.view(np.uint32), ref["Wd"].view(np.uint32)), "dequant fp32"
            wb = nf4.nf4_dequantize(W, torch.bfloat16)
            wb_ref = torch.from_numpy(ref["Wd"]).to(torch.bfloat16)
            assert torch.equal(wb.cpu().view(torch.int16), wb_ref.view(torch.int16)), "dequant bf16"
    return ref


@pytest.mark.parametrize("shape", [(1, 64), (3, 64), (7, 192), (256, 256), (300, 448), (1000, 1088)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_codec_small_shapes(shape, dtype):
    d = Draw(seed_of(1, shape[0], shape[1]), "cpu")
    w = d.normal(shape, 0.02, outlier_frac=0.01).to(dtype)
    _assert_codec_equal(w, w.to(DEV))


@pytest.mark.parametrize("n", [1, 2, 63, 65, 127, 1001, 64 * 256 + 3, 64 * 2048 * 3 + 17])
def test_codec_flat_ragged(n):
    d = Draw(seed_of(2, n), "cpu")
    w = d.normal((n,), 0.05)
    _assert_codec_equal(w, w.to(DEV), check_dequant=False)
    # dequantize a flat ragged tensor through a 1 x n view
    ref = oracle_weight(w.view(1, n))
    codes, absmax, q, c2, mean = _gpu_tuple(w.to(DEV))
    wd = nf4.nf4_dequantize(nf4.NF4Weight(codes, q, c2, mean, (1, n)), torch.float32).cpu().numpy()
    assert np.array_equal(wd.view(np.uint32), ref["Wd"].view(np.uint32))


def test_codec_special_values():
    lv = oracle.nf4_codebook().astype(np.float64)
    rows = []
    rows.append(np.zeros(64, np.float32))                                 # zero block
    blk = np.zeros(64, np.float32)
    ties = [(lv[j] + lv[j + 1]) / 2 for j in (2, 6, 7, 14)]              # exact fp32 midpoints
    blk[: len(ties)] = np.array(ties, np.float32)
    blk[10] = 1.0
    blk[11] = -0.0
    rows.append(blk)
    rows.append(np.linspace(-3, 2, 64).astype(np.float32))               # absmax from the negative side
    big = np.full(64, 1e-30, np.float32)
    big[5] = 3e30
    rows.append(big)                                                     # huge dynamic range
    w = torch.from_numpy(np.stack(rows))
    _assert_codec_equal(w, w.to(DEV))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_codec_extreme_absmax(dtype):
    # blocks whose absmax lies outside [2^-126, 2^126): subnormal (its reciprocal would
    # overflow), above 2^126 (a subnormal reciprocal) and the largest finite value.  The
    # codes must still be those of the IEEE quotient w / absmax, e.g. 0xC2 for the pair
    # (+0.5, -0.5) x absmax at absmax 2e-39
    ramp = np.linspace(-1.0, 1.0, 64)
    rows = []
    amaxes = [2e-39, 1e-44, 1.1754942e-38, 1e38, 3.0e38]
    if dtype == torch.float32:
        amaxes.append(float(np.finfo(np.float32).max))     # rounds to inf in bf16
    for amax in amaxes:
        blk = (ramp * amax).astype(np.float32)
        blk[0] = np.float32(-amax)
        blk[1] = np.float32(amax)
        blk[2] = np.float32(0.5 * amax)
        blk[3] = np.float32(-0.5 * amax)
        rows.append(blk)
    w = torch.from_numpy(np.stack(rows)).to(dtype)
    ref = _assert_codec_equal(w, w.to(DEV), check_dequant=False)
    assert ref["codes"][0] == 0xF0 and ref["codes"][1] == 0x2C, "oracle codes of -1, 1, 0.5, -0.5 x absmax"


def test_codec_non_finite_values():
    # outside the linear layer's domain, but the codec's codes and constants still follow
    # the IEEE arithmetic of the definition: an infinite value makes the block's absmax
    # infinite, finite values then divide to zero (code 7) and the infinite one to NaN,
    # which no threshold is below (code 0); a NaN value is no larger than the others, so
    # the absmax comes from the finite values, and its quotient takes code 0; an all-NaN
    # block has absmax 0 and the zero code
    rng = np.random.Generator(np.random.PCG64(17))
    rows = [rng.standard_normal(64).astype(np.float32) * 0.02 for _ in range(5)]
    rows[0][3] = np.inf
    rows[1][60] = -np.inf
    rows[2][7] = np.nan
    rows[2][8] = np.nan
    rows[3][:] = np.nan
    rows[4][0] = np.inf
    rows[4][1] = np.nan
    rows[4][2] = -np.inf
    w = torch.from_numpy(np.stack(rows))
    for dt in (torch.float32, torch.bfloat16):
        wt = w.to(dt)
        h = bf16_bits(wt).reshape(-1) if dt == torch.bfloat16 else host_f32(wt).reshape(-1)
        rc, ra = oracle.nf4_quantize(h)
        codes, absmax = nf4.nf4_quantize(wt.to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), rc), "codes (%s)" % dt
        assert np.array_equal(absmax.cpu().numpy().view(np.uint32), ra.view(np.uint32)), "absmax (%s)" % dt
    assert (rc[1] >> 4) == 0 and rc[3 * 32] == 0x77           # inf (element 3) -> code 0; all-NaN block -> 7


def test_double_quant_constant_and_mean_tree():
    # a constant absmax vector gives c2 = 0, q = 0 and c1' == mean exactly
    c1 = torch.full((5000,), 0.0625)
    q, c2, mean = nf4.nf4_double_quantize(c1.to(DEV))
    assert torch.all(c2 == 0).item() and torch.all(q == 0).item()
    assert mean.item() == 0.0625
    assert torch.all(nf4.nf4_double_dequantize(q, c2, mean) == 0.0625).item()
    # a length that needs three passes of the chunk tree
    rng = np.random.Generator(np.random.PCG64(9))
    c1 = np.abs(rng.standard_normal(2048 * 2048 + 12345)).astype(np.float32)
    rq, rc2, rmean = oracle.double_quantize(c1)
    q, c2, mean = nf4.nf4_double_quantize(torch.from_numpy(c1).to(DEV))
    assert mean.cpu().numpy().view(np.uint32)[0] == rmean.view(np.uint32)[0]
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(c2.cpu().numpy().view(np.uint32), rc2.view(np.uint32))


def test_double_quantize_batch():
    # the batched double quantization equals the oracle, tensor by tensor, bit for bit: sizes
    # that are empty, one constant, one ragged block, whole and ragged chunks, the largest a
    # batch takes (2048 chunks), and more tensors than one launch pair holds (32)
    rng = np.random.Generator(np.random.PCG64(21))
    sizes = [0, 1, 255, 256, 2047, 2048, 2049, 70001, 2048 * 2048] + [int(x) for x in rng.integers(1, 9000, 40)]
    host = [np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(rng.uniform(1e-3, 10.0))
            for n in sizes]
    host[3][:] = np.float32(0.0625)                        # a constant vector: c2 = 0, q = 0
    dev = [torch.from_numpy(h).to(DEV) for h in host]
    outs = nf4.nf4_double_quantize_batch(dev)
    torch.cuda.synchronize()
    assert len(outs) == len(sizes)
    for n, h, (q, c2, mean) in zip(sizes, host, outs):
        rq, rc2, rmean = oracle.double_quantize(h)
        where = "n1=%d" % n
        assert mean.cpu().numpy().view(np.uint32)[0] == np.asarray(rmean, np.float32).view(np.uint32).reshape(-1)[0], where
        assert np.array_equal(q.cpu().numpy(), rq), where
        assert np.array_equal(c2.cpu().numpy().view(np.uint32), np.asarray(rc2, np.float32).view(np.uint32)), where


@pytest.mark.parametrize("name,N,K", [("q7b", 4096, 4096), ("gate7b", 11008, 4096),
                                      ("down65b", 8192, 22016)])
def test_codec_full_llama_shapes(name, N, K):
    print("codec full shape", name, N, K, flush=True)
    d = Draw(seed_of(3, N, K), DEV)
    w_dev = d.normal((N, K), 0.02, outlier_frac=0.01)
    _assert_codec_equal(w_dev.cpu(), w_dev, check_dequant=(N * K <= 64 * 10 ** 6))


def test_codec_bf16_full_shape():
    d = Draw(seed_of(4), DEV)
    w_dev = d.normal((11008, 4096), 0.02, outlier_frac=0.01).to(torch.bfloat16)
    _assert_codec_equal(w_dev.cpu(), w_dev)


def test_codec_deterministic():
    d = Draw(seed_of(5), DEV)
    w = d.normal((4096, 4096), 0.02)
    a = _gpu_tuple(w)
    b = _gpu_tuple(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("shape", [(64, 64), (328, 320), (1000, 1088), (4096, 4096)])
def test_dequantize_plain_constants(shape):
    # [DQ] off: nf4_dequantize with the plain constants gives fp32(level * absmax) bit for
    # bit, and its round-to-nearest-even bf16 value
    w = Draw(seed_of(41, *shape), DEV).normal(shape, 0.02, outlier_frac=0.01)
    W = nf4.quantize_weight(w, double_quant=False)
    ref = oracle_weight(w.cpu())
    exp = oracle.nf4_dequantize_plain(ref["codes"], ref["absmax"], shape)
    got = nf4.nf4_dequantize(W, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))
    gb = nf4.nf4_dequantize(W, torch.bfloat16)
    assert torch.equal(gb.cpu().view(torch.int16), torch.from_numpy(exp).bfloat16().view(torch.int16))


# Chunks of 2048 (fp32 out) or 4096 (bf16 out) values per wave, 8192 waves at most: these
# sizes give more whole chunks than waves (waves run 2 or 3 chunks, so the pipelined loop
# leaves through both register sets) plus a partial last chunk.
@pytest.mark.parametrize("out_dtype,n", [(torch.float32, (2 * 8192 + 3) * 2048 + 777),
                                         (torch.bfloat16, (2 * 8192 + 5) * 4096 + 1001)])
@pytest.mark.parametrize("double_quant", [True, False])
def test_dequantize_more_chunks_than_waves(out_dtype, n, double_quant):
    print("dequantize", out_dtype, n, "double_quant", double_quant, flush=True)
    w = Draw(seed_of(42, n), DEV).normal((1, n), 0.02, outlier_frac=0.01)
    W = nf4.quantize_weight(w, double_quant=double_quant)
    ref = oracle_weight(w.cpu())
    if double_quant:
        exp = ref["Wd"]
    else:
        exp = oracle.nf4_dequantize_plain(ref["codes"], ref["absmax"], (1, n))
    got = nf4.nf4_dequantize(W, out_dtype)
    if out_dtype == torch.float32:
        assert np.array_equal(got.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    else:
        assert torch.equal(got.cpu().view(torch.int16), torch.from_numpy(exp).bfloat16().view(torch.int16))
