"""CPU oracle for the QLoRA NF4 linear layer (numpy in, numpy out).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The arithmetic lives in
``nf4_oracle.c`` (plain C, float64 accumulation, no fused multiply-adds); this
module only marshals numpy arrays.  It shares nothing with the GPU library.

Function names follow the pages' stubs ("NF4, derived from normal quantiles"
and "Double quantization" on the zerotofrontier.app PEFT page) and the layer
formula ("Putting it together" on the prism.theerrors.in QLoRA explainer).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    src_mtime = os.path.getmtime(_build.SRC)
    if not os.path.exists(path) or os.path.getmtime(path) < src_mtime:
        _build.build()
    lib = ctypes.CDLL(path)
    lib.orc_norm_ppf.restype = ctypes.c_double
    lib.orc_norm_ppf.argtypes = [ctypes.c_double]
    lib.orc_nf4_codebook.argtypes = [_f32p]
    lib.orc_nf4_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64, _u8p, _f32p]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_double_quantize.argtypes = [_f32p, _i64, _u8p, _f32p, _f32p]
    lib.orc_double_dequantize.argtypes = [_u8p, _f32p, _f32p, _i64, _f32p]
    lib.orc_nf4_dequantize.argtypes = [_u8p, _u8p, _f32p, _f32p, _i64, _f32p]
    lib.orc_qlora_linear_fwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                                         ctypes.c_double, _i64p, _i64, _f64p, _f64p]
    lib.orc_qlora_linear_bwd.argtypes = [_f32p, _f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64,
                                         _i64, ctypes.c_double, _i64p, _i64, _f64p, _f64p, _f64p]
    lib.orc_nf4_dequantize_plain.argtypes = [_u8p, _f32p, _i64, _f32p]
    lib.orc_quantize_levels.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64, _f32p, _u8p, _f32p]
    lib.orc_codebook_stats.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64, _u8p, _f32p, _f32p, _i64p,
                                       _f64p, _f64p]
    _d = ctypes.c_double
    lib.orc_adamw_step.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _d, _d, _d, _d, _d, _i64,
                                   _f64p, _f64p, _f64p]
    lib.orc_svd_topr.argtypes = [_f64p, _i64, _i64, _i64, _f64p, _f64p, _f64p]
    lib.orc_loftq.argtypes = [_f32p, _i64, _i64, _i64, _d, ctypes.c_int, _u8p, _u8p, _f32p, _f32p,
                              _f64p, _f64p, _f64p]
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_pairwise_sum.restype = ctypes.c_double
    lib.orc_pairwise_sum.argtypes = [_f32p, _i64]
    _lib = lib
    return lib


def _p(a, t):
    return a.ctypes.data_as(t) if a is not None else None


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().orc_num_threads()


def norm_ppf(p: float) -> float:
    """Inverse standard-normal CDF (Wichura AS 241, float64)."""
    return _load().orc_norm_ppf(float(p))


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels, ascending, fp32 ("NF4, derived from normal quantiles")."""
    out = np.zeros(16, np.float32)
    _load().orc_nf4_codebook(_p(out, _f32p))
    return out


def nf4_quantize(w: np.ndarray, block: int = 64):
    """Blockwise-absmax NF4 quantization ("Block-wise quantization in one page").

    w: float32 array, or uint16 array of bf16 bit patterns, flattened row-major.
    Returns (codes uint8[ceil(n/2)], absmax float32[ceil(n/64)]).
    """
    if block != 64:
        raise ValueError("blocksize 64 only")
    w = np.ascontiguousarray(w).reshape(-1)
    if w.dtype == np.float32:
        is_bf16 = 0
    elif w.dtype == np.uint16:
        is_bf16 = 1
    else:
        raise TypeError("float32 or bf16 bit patterns (uint16)")
    n = w.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    absmax = np.zeros((n + 63) // 64, np.float32)
    _load().orc_nf4_quantize(w.ctypes.data_as(ctypes.c_void_p), is_bf16, n,
                             _p(codes, _u8p), _p(absmax, _f32p))
    return codes, absmax


def pairwise_sum(x: np.ndarray) -> float:
    """Aligned pairwise float64 sum used for the double-quantization mean."""
    x = np.ascontiguousarray(x, np.float32).reshape(-1)
    return float(_load().orc_pairwise_sum(_p(x, _f32p), x.size))


def e4m3_encode(v: float) -> int:
    """OCP E4M3 code of v (|v| <= 448), nearest value, ties to even code."""
    return int(_load().orc_e4m3_encode(float(v)))


def e4m3_decode(b: int) -> float:
    """Exact value of an E4M3 code (no NaN codes expected)."""
    return float(_load().orc_e4m3_decode(int(b)))


def double_quantize(c1: np.ndarray, block: int = 256):
    """Double quantization of first-level constants ("Double quantization").

    Returns (q uint8[n1], c2 float32[ceil(n1/256)], mean float32[1]).
    """
    if block != 256:
        raise ValueError("blocksize 256 only")
    c1 = np.ascontiguousarray(c1, np.float32).reshape(-1)
    n1 = c1.size
    q = np.zeros(n1, np.uint8)
    c2 = np.zeros((n1 + 255) // 256, np.float32)
    mean = np.zeros(1, np.float32)
    _load().orc_double_quantize(_p(c1, _f32p), n1, _p(q, _u8p), _p(c2, _f32p), _p(mean, _f32p))
    return q, c2, mean


def double_dequantize(q: np.ndarray, c2: np.ndarray, mean: np.ndarray) -> np.ndarray:
    """c1' = fma(E4M3(q), fp32(c2/448), mean), one rounding per constant."""
    q = np.ascontiguousarray(q, np.uint8).reshape(-1)
    c2 = np.ascontiguousarray(c2, np.float32).reshape(-1)
    mean = np.ascontiguousarray(mean, np.float32).reshape(-1)
    out = np.zeros(q.size, np.float32)
    _load().orc_double_dequantize(_p(q, _u8p), _p(c2, _f32p), _p(mean, _f32p), q.size,
                                  _p(out, _f32p))
    return out


def nf4_dequantize(codes, q, c2, mean, shape) -> np.ndarray:
    """w' = fp32(level[code] * c1') over the whole tensor; returns float32 `shape`."""
    n = int(np.prod(shape)) if len(shape) else 1
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1)
    q = np.ascontiguousarray(q, np.uint8).reshape(-1)
    c2 = np.ascontiguousarray(c2, np.float32).reshape(-1)
    mean = np.ascontiguousarray(mean, np.float32).reshape(-1)
    out = np.zeros(n, np.float32)
    _load().orc_nf4_dequantize(_p(codes, _u8p), _p(q, _u8p), _p(c2, _f32p), _p(mean, _f32p), n,
                               _p(out, _f32p))
    return out.reshape(shape)


def _f32(a):
    return np.ascontiguousarray(a, np.float32)


def qlora_linear_fwd(Wd, X, A, B, alpha, rows=None):
    """Y = X W'^T + (alpha/r) (X A^T) B^T and T = X A^T, in float64.

    Wd: dequantized weight float32 (N, K); X (M, K); A (r, K); B (N, r) as
    float32 arrays holding the exact bf16 values.  rows: optional row indices
    of Y to compute.  Returns (Y float64 (len(rows) or M, N), T float64 (M, r)).
    """
    Wd, X, A, B = _f32(Wd), _f32(X), _f32(A), _f32(B)
    N, K = Wd.shape
    M = X.shape[0]
    r = A.shape[0]
    rows_a = None if rows is None else np.ascontiguousarray(rows, np.int64)
    nr = M if rows_a is None else rows_a.size
    Y = np.zeros((nr, N), np.float64)
    T = np.zeros((M, r), np.float64)
    _load().orc_qlora_linear_fwd(_p(Wd, _f32p), _p(X, _f32p), _p(A, _f32p), _p(B, _f32p), M, N,
                                 K, r, float(alpha), _p(rows_a, _i64p), nr, _p(Y, _f64p),
                                 _p(T, _f64p))
    return Y, T


def qlora_linear_bwd(Wd, X, dY, A, B, alpha, rows=None, want_dx=True, want_da=True,
                     want_db=True):
    """dX = dY W' + s U A, dA = s U^T X, dB = s dY^T (X A^T), U = dY B, in float64.

    Returns (dX or None, dA or None, dB or None).
    """
    Wd, X, dY, A, B = _f32(Wd), _f32(X), _f32(dY), _f32(A), _f32(B)
    N, K = Wd.shape
    M = X.shape[0]
    r = A.shape[0]
    rows_a = None if rows is None else np.ascontiguousarray(rows, np.int64)
    nr = M if rows_a is None else rows_a.size
    dX = np.zeros((nr, K), np.float64) if want_dx else None
    dA = np.zeros((r, K), np.float64) if want_da else None
    dB = np.zeros((N, r), np.float64) if want_db else None
    _load().orc_qlora_linear_bwd(_p(Wd, _f32p), _p(X, _f32p), _p(dY, _f32p), _p(A, _f32p),
                                 _p(B, _f32p), M, N, K, r, float(alpha), _p(rows_a, _i64p), nr,
                                 _p(dX, _f64p), _p(dA, _f64p), _p(dB, _f64p))
    return dX, dA, dB


def adamw_step(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step on fp32 state (p, g, m, v); returns (p', m', v') in float64.

    The pages ("Paged optimizers, and QLoRA end to end", zerotofrontier.app
    "sft/peft") page the adapters' Adam states and give the learning rates; the
    update is Kingma & Ba (2015) Algorithm 1 with Loshchilov & Hutter (2019)
    decoupled weight decay, evaluated in float64.
    """
    p, g, m, v = (_f32(a).ravel() for a in (p, g, m, v))
    n = p.size
    assert g.size == n and m.size == n and v.size == n and int(step) >= 1
    po, mo, vo = (np.empty(n, np.float64) for _ in range(3))
    _load().orc_adamw_step(_p(p, _f32p), _p(g, _f32p), _p(m, _f32p), _p(v, _f32p), n,
                           float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                           int(step), _p(po, _f64p), _p(mo, _f64p), _p(vo, _f64p))
    return po, mo, vo


def quantize_levels(w: np.ndarray, levels: np.ndarray):
    """Blockwise absmax quantization (blocks of 64) onto an ascending 16-level codebook
    ("Block-wise quantization in one page"); returns (codes uint8[ceil(n/2)], absmax)."""
    levels = np.ascontiguousarray(levels, np.float32).ravel()
    assert levels.size == 16 and np.all(np.diff(levels.astype(np.float64)) > 0)
    is_bf16 = 1 if w.dtype == np.uint16 else 0
    w = np.ascontiguousarray(w).ravel()
    n = w.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    absmax = np.zeros((n + 63) // 64, np.float32)
    _load().orc_quantize_levels(w.ctypes.data_as(ctypes.c_void_p), is_bf16, n, _p(levels, _f32p),
                                _p(codes, _u8p), _p(absmax, _f32p))
    return codes, absmax


def codebook_stats(w: np.ndarray, codes: np.ndarray, absmax: np.ndarray, levels: np.ndarray):
    """(count int64[16], sum_x float64[16], sse float64) of a blockwise quantization:
    values per code, sum of x = fp32(w/absmax) per code, and the float64 sum of
    (w - fp32(level[code] * absmax))^2 ("NF4, derived from normal quantiles")."""
    levels = np.ascontiguousarray(levels, np.float32).ravel()
    is_bf16 = 1 if w.dtype == np.uint16 else 0
    w = np.ascontiguousarray(w).ravel()
    codes = np.ascontiguousarray(codes, np.uint8)
    absmax = np.ascontiguousarray(absmax, np.float32)
    count = np.zeros(16, np.int64)
    sum_x = np.zeros(16, np.float64)
    sse = np.zeros(1, np.float64)
    _load().orc_codebook_stats(w.ctypes.data_as(ctypes.c_void_p), is_bf16, w.size, _p(codes, _u8p),
                               _p(absmax, _f32p), _p(levels, _f32p), _p(count, _i64p), _p(sum_x, _f64p),
                               _p(sse, _f64p))
    return count, sum_x, float(sse[0])


def nf4_dequantize_plain(codes, absmax, shape) -> np.ndarray:
    """w' = fp32(level[code] * absmax[i/64]) with plain constants (double quantization
    off, "Double quantization"); returns float32 `shape`."""
    n = int(np.prod(shape))
    codes = np.ascontiguousarray(codes, np.uint8)
    absmax = np.ascontiguousarray(absmax, np.float32)
    out = np.empty(n, np.float32)
    _load().orc_nf4_dequantize_plain(_p(codes, _u8p), _p(absmax, _f32p), n, _p(out, _f32p))
    return out.reshape(shape)


def svd_topr(E, r):
    """Top r singular triplets of E (float64 m x n) by one-sided Jacobi: (S descending,
    U m x r, Vt r x n), so that U diag(S) Vt is the best rank-r approximation of E."""
    E = np.ascontiguousarray(E, np.float64)
    m, n = E.shape
    assert 0 < r <= min(m, n)
    S = np.zeros(r, np.float64)
    U = np.zeros((m, r), np.float64)
    Vt = np.zeros((r, n), np.float64)
    _load().orc_svd_topr(_p(E, _f64p), m, n, r, _p(S, _f64p), _p(U, _f64p), _p(Vt, _f64p))
    return S, U, Vt


def loftq(W, r, gamma, iters):
    """LoftQ-style initialisation ("Paged optimizers, and QLoRA end to end": start the
    adapter so that dequant(W^NF4) + gamma B A is close to W): `iters` alternations of
    NF4 + double quantization of the residual W - gamma B A and a rank-r truncated SVD of
    the quantization error.  Returns dict(codes, q, c2, mean, B (N x r), A (r x K) float64,
    err (per iteration ||W - dequant(Q_t) - gamma B_t A_t||_F))."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    n = N * K
    n1 = (n + 63) // 64
    codes = np.zeros((n + 1) // 2, np.uint8)
    q = np.zeros(n1, np.uint8)
    c2 = np.zeros((n1 + 255) // 256, np.float32)
    mean = np.zeros(1, np.float32)
    B = np.zeros((N, r), np.float64)
    A = np.zeros((r, K), np.float64)
    err = np.zeros(iters, np.float64)
    _load().orc_loftq(_p(W, _f32p), N, K, r, float(gamma), int(iters), _p(codes, _u8p), _p(q, _u8p),
                      _p(c2, _f32p), _p(mean, _f32p), _p(B, _f64p), _p(A, _f64p), _p(err, _f64p))
    return dict(codes=codes, q=q, c2=c2, mean=mean, B=B, A=A, err=err)
