"""QLoRA NF4 linear layer for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libqlora_nf4.so`` (declared in
``include/qlora_nf4.h``).  This module only marshals arguments: it checks
dtypes and shapes, allocates outputs and workspaces with torch, and passes raw
device pointers plus the current HIP stream.  Every step of the computation
runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and a
missing library raises ``NF4Error``.

Names follow the stubs on the zerotofrontier.app PEFT page ("NF4, derived from
normal quantiles": nf4_quantize / nf4_dequantize; "Double quantization":
double_quantize / double_dequantize) and the layer formula of "Putting it
together" (prism.theerrors.in QLoRA explainer).
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

__all__ = [
    "NF4Error", "NF4Weight", "lib_path", "load_library", "nf4_quantize", "nf4_double_quantize",
    "nf4_double_dequantize", "nf4_double_quantize_batch", "nf4_dequantize", "quantize_weight", "qlora_linear_fwd",
    "qlora_linear_bwd", "nf4_storage_bytes", "nf4_codebook", "nf4_workspace_bytes",
    "nf4_profile_next_fused", "adamw_step", "adamw_step_paged", "PagedAdamW",
    "nf4_quantize_codebook", "nf4_codebook_stats", "qlora_linear_fwd_noalloc", "codebook_int4_symmetric", "codebook_uniform16",
    "lloyd_codebook", "NF4_OP_CODEBOOK_STATS",
    "NF4_OP_DOUBLE_QUANTIZE", "NF4_OP_LINEAR_FWD", "NF4_OP_LINEAR_BWD", "NF4_OP_LOWRANK_SVD", "NF4_OP_LOFTQ",
    "nf4_lowrank_svd", "loftq_init",
]

NF4_OK, NF4_ERR_ARG, NF4_ERR_UNSUPPORTED, NF4_ERR_WORKSPACE, NF4_ERR_HIP = range(5)
NF4_F32, NF4_BF16 = 0, 1
NF4_OP_DOUBLE_QUANTIZE, NF4_OP_LINEAR_FWD, NF4_OP_LINEAR_BWD, NF4_OP_CODEBOOK_STATS = 1, 2, 3, 4
NF4_OP_LOWRANK_SVD, NF4_OP_LOFTQ = 5, 6
_STATUS = {1: "NF4_ERR_ARG", 2: "NF4_ERR_UNSUPPORTED", 3: "NF4_ERR_WORKSPACE", 4: "NF4_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "_lib", "libqlora_nf4.so")


class NF4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, status), message))
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("q", ctypes.c_void_p), ("c2", ctypes.c_void_p),
                ("mean", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("absmax", ctypes.c_void_p)]


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


def load_library():
    """Load libqlora_nf4.so (raises NF4Error if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise NF4Error(NF4_ERR_HIP, "HIP library not built (%s); run __graft_entry__.build()" % path)
    L = ctypes.CDLL(path)
    L.nf4_quantize.restype = ctypes.c_int
    L.nf4_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i32, _vp, _vp, _vp]
    L.nf4_double_quantize.restype = ctypes.c_int
    L.nf4_double_quantize.argtypes = [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    L.nf4_double_quantize_batch.restype = ctypes.c_int
    L.nf4_double_quantize_batch.argtypes = [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.nf4_double_quantize_batch_workspace_bytes.restype = _sz
    L.nf4_double_quantize_batch_workspace_bytes.argtypes = [_i32, _vp]
    L.nf4_double_dequantize.restype = ctypes.c_int
    L.nf4_double_dequantize.argtypes = [_vp, _vp, _vp, _i64, _i32, _vp, _vp]
    L.nf4_dequantize.restype = ctypes.c_int
    L.nf4_dequantize.argtypes = [ctypes.POINTER(_Weight), _vp, ctypes.c_int, _vp]
    L.qlora_linear_fwd.restype = ctypes.c_int
    L.qlora_linear_fwd.argtypes = [ctypes.POINTER(_Weight), _vp, _i64, _vp, _vp, _i32, ctypes.c_float,
                                   _vp, _vp, _vp, _sz, _vp]
    L.qlora_linear_fwd_noalloc.restype = ctypes.c_int
    L.qlora_linear_fwd_noalloc.argtypes = [ctypes.POINTER(_Weight), _vp, _i64, _vp, _vp, _i32, ctypes.c_float,
                                           _vp, _vp, _vp]
    L.qlora_linear_bwd.restype = ctypes.c_int
    L.qlora_linear_bwd.argtypes = [ctypes.POINTER(_Weight), _vp, _vp, _i64, _vp, _vp, _i32,
                                   ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.nf4_workspace_bytes.restype = _sz
    L.nf4_workspace_bytes.argtypes = [_i32, _i64, _i64, _i64, _i32]
    L.nf4_storage_bytes.restype = None
    L.nf4_storage_bytes.argtypes = [_i64, _i32, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                    ctypes.POINTER(_sz)]
    L.nf4_codebook.restype = None
    L.nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.nf4_profile_next_fused.restype = None
    L.nf4_profile_next_fused.argtypes = [_vp, _vp]
    _f = ctypes.c_float
    _fp = ctypes.POINTER(ctypes.c_float)
    L.nf4_quantize_codebook.restype = ctypes.c_int
    L.nf4_quantize_codebook.argtypes = [_vp, ctypes.c_int, _i64, _i32, _fp, _vp, _vp, _vp]
    L.nf4_codebook_stats.restype = ctypes.c_int
    L.nf4_codebook_stats.argtypes = [_vp, ctypes.c_int, _i64, _vp, _vp, _fp, _vp, _vp, _sz, _vp]
    L.nf4_adamw_step.restype = ctypes.c_int
    L.nf4_adamw_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _f, _f, _f, _f, _f, _i64, _vp]
    L.nf4_adamw_step_paged.restype = ctypes.c_int
    L.nf4_adamw_step_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _f, _f, _f, _f, _f, _i64,
                                       _vp, _sz, _vp]
    L.nf4_lowrank_svd.restype = ctypes.c_int
    L.nf4_lowrank_svd.argtypes = [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.nf4_loftq_init.restype = ctypes.c_int
    L.nf4_loftq_init.argtypes = [_vp, _i64, _i64, _i32, _f, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _sz, _vp]
    L.nf4_last_error.restype = ctypes.c_char_p
    L.nf4_last_error.argtypes = []
    _lib = L
    return L


def _check(status: int):
    if status != NF4_OK:
        raise NF4Error(status, load_library().nf4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


def _numel(t: Optional[torch.Tensor], name: str, n: int, dtype):
    """Size and dtype of a 1-D operand, checked before anything reaches the device."""
    if t is None:
        raise ValueError("%s is missing" % name)
    if t.dtype != dtype or t.numel() != n:
        raise ValueError("%s must hold %d values of %s, got %d of %s" % (name, n, dtype, t.numel(), t.dtype))


def _same_device(*named):
    devs = {(name, t.device) for name, t in named if t is not None}
    if len({d for _, d in devs}) > 1:
        raise ValueError("operands on different devices: %s" % sorted((n, str(d)) for n, d in devs))


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off: off + nbytes]


@dataclass
class NF4Weight:
    """A frozen weight as NF4 on the GPU: codes with double-quantized constants (q, c2,
    mean), or, with double quantization off, with the plain fp32 constants (absmax;
    q, c2 and mean None)."""
    codes: torch.Tensor             # uint8 [ceil(n/2)]
    q: Optional[torch.Tensor]       # uint8 [ceil(n/64)]
    c2: Optional[torch.Tensor]      # float32 [ceil(n1/256)]
    mean: Optional[torch.Tensor]    # float32 [1]
    shape: Tuple[int, int]
    absmax: Optional[torch.Tensor] = None   # float32 [ceil(n/64)], when q is None

    def validate(self):
        """Sizes, dtypes and device of the tuple against its shape (raises ValueError)."""
        rows, cols = self.shape
        if rows < 0 or cols < 0:
            raise ValueError("negative weight shape")
        n = rows * cols
        n1 = (n + 63) // 64
        _numel(self.codes, "codes", (n + 1) // 2, torch.uint8)
        if self.q is not None:
            _numel(self.q, "q", n1, torch.uint8)
            _numel(self.c2, "c2", (n1 + 255) // 256, torch.float32)
            _numel(self.mean, "mean", 1, torch.float32)
            parts = (("codes", self.codes), ("q", self.q), ("c2", self.c2), ("mean", self.mean))
        else:
            _numel(self.absmax, "absmax", n1, torch.float32)
            parts = (("codes", self.codes), ("absmax", self.absmax))
        for name, t in parts:
            _dev(t, name)
        _same_device(*parts)

    def descriptor(self) -> _Weight:
        self.validate()
        rows, cols = self.shape
        ptr = lambda t: t.data_ptr() if t is not None else None
        return _Weight(self.codes.data_ptr(), ptr(self.q), ptr(self.c2), ptr(self.mean), rows, cols,
                       ptr(self.absmax) if self.q is None else None)

    @property
    def device(self):
        return self.codes.device

    def nbytes(self) -> int:
        parts = (self.codes, self.q, self.c2, self.mean) if self.q is not None else (self.codes, self.absmax)
        return sum(t.numel() * t.element_size() for t in parts)


def nf4_profile_next_fused(start: "torch.cuda.Event", stop: "torch.cuda.Event"):
    """Arm the library's profiling hook: the next fused dequant kernel launched on this
    thread records `start` before and `stop` after itself on its stream."""
    start_h = ctypes.c_void_p(start.cuda_event) if start is not None else None
    stop_h = ctypes.c_void_p(stop.cuda_event) if stop is not None else None
    load_library().nf4_profile_next_fused(start_h, stop_h)


def nf4_codebook():
    """The 16 NF4 levels (host copy)."""
    out = (ctypes.c_float * 16)()
    load_library().nf4_codebook(out)
    return list(out)


def nf4_storage_bytes(n: int, blocksize: int = 64, blocksize2: int = 256):
    """(codes, q, c2) bytes of a double-quantized NF4 tensor of n values."""
    a, b, c = _sz(), _sz(), _sz()
    load_library().nf4_storage_bytes(n, blocksize, blocksize2, ctypes.byref(a), ctypes.byref(b),
                                     ctypes.byref(c))
    return a.value, b.value, c.value


def nf4_workspace_bytes(op: int, M: int, N: int, K: int, r: int) -> int:
    return int(load_library().nf4_workspace_bytes(op, M, N, K, r))


def nf4_quantize(w: torch.Tensor, blocksize: int = 64):
    """Blockwise-absmax NF4 codes of a fp32/bf16 tensor: (codes uint8, absmax fp32)."""
    L = load_library()
    _dev(w, "w")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    n = w.numel()
    codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=w.device)
    absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=w.device)
    _check(L.nf4_quantize(_ptr(w), NF4_BF16 if w.dtype == torch.bfloat16 else NF4_F32, n, blocksize,
                          _ptr(codes), _ptr(absmax), _stream(w.device)))
    return codes, absmax


def nf4_double_quantize(absmax: torch.Tensor, blocksize2: int = 256):
    """Double quantization of the first-level constants: (q uint8, c2 fp32, mean fp32[1])."""
    L = load_library()
    _dev(absmax, "absmax", torch.float32)
    n1 = absmax.numel()
    q = torch.empty(n1, dtype=torch.uint8, device=absmax.device)
    c2 = torch.empty((n1 + 255) // 256, dtype=torch.float32, device=absmax.device)
    mean = torch.empty(1, dtype=torch.float32, device=absmax.device)
    wsb = L.nf4_workspace_bytes(NF4_OP_DOUBLE_QUANTIZE, 0, n1, 0, 0)
    ws = _workspace(wsb, absmax.device)
    _check(L.nf4_double_quantize(_ptr(absmax), n1, blocksize2, _ptr(q), _ptr(c2), _ptr(mean),
                                 _ptr(ws), wsb, _stream(absmax.device)))
    return q, c2, mean


def nf4_double_quantize_batch(absmax_list):
    """Double quantization of many first-level constant vectors at once (same device):
    a list of (q, c2, mean), each exactly what nf4_double_quantize gives for that vector,
    from two kernel launches per 32 vectors."""
    L = load_library()
    absmax_list = list(absmax_list)
    count = len(absmax_list)
    if count == 0:
        return []
    for i, a in enumerate(absmax_list):
        _dev(a, "absmax[%d]" % i, torch.float32)
    _same_device(*(("absmax[%d]" % i, a) for i, a in enumerate(absmax_list)))
    dev = absmax_list[0].device
    outs = []
    for a in absmax_list:
        n1 = a.numel()
        outs.append((torch.empty(n1, dtype=torch.uint8, device=dev),
                     torch.empty((n1 + 255) // 256, dtype=torch.float32, device=dev),
                     torch.empty(1, dtype=torch.float32, device=dev)))
    arr = lambda vals, ct: (ct * count)(*vals)
    n1s = arr([a.numel() for a in absmax_list], ctypes.c_int64)
    c1p = arr([_ptr(a) for a in absmax_list], ctypes.c_void_p)
    qp = arr([_ptr(o[0]) for o in outs], ctypes.c_void_p)
    c2p = arr([_ptr(o[1]) for o in outs], ctypes.c_void_p)
    mp = arr([_ptr(o[2]) for o in outs], ctypes.c_void_p)
    wsb = L.nf4_double_quantize_batch_workspace_bytes(count, n1s)
    ws = _workspace(wsb, dev)
    _check(L.nf4_double_quantize_batch(count, c1p, n1s, qp, c2p, mp, _ptr(ws), wsb, _stream(dev)))
    return outs


def nf4_double_dequantize(q: torch.Tensor, c2: torch.Tensor, mean: torch.Tensor,
                          blocksize2: int = 256) -> torch.Tensor:
    """c1' = fma(E4M3(q), fp32(c2/448), mean) per constant."""
    L = load_library()
    n1 = q.numel()
    _numel(q, "q", n1, torch.uint8)
    _numel(c2, "c2", (n1 + 255) // 256, torch.float32)
    _numel(mean, "mean", 1, torch.float32)
    for name, t in (("q", q), ("c2", c2), ("mean", mean)):
        _dev(t, name)
    _same_device(("q", q), ("c2", c2), ("mean", mean))
    out = torch.empty(q.numel(), dtype=torch.float32, device=q.device)
    _check(L.nf4_double_dequantize(_ptr(q), _ptr(c2), _ptr(mean), q.numel(), blocksize2, _ptr(out),
                                   _stream(q.device)))
    return out


def quantize_weight(w: torch.Tensor, double_quant: bool = True) -> NF4Weight:
    """Quantize a 2-D (out x in) fp32/bf16 weight to NF4: the double-quantized tuple, or
    with double_quant=False the codes and plain fp32 constants."""
    if w.dim() != 2:
        raise ValueError("weight must be 2-D (out x in)")
    codes, absmax = nf4_quantize(w)
    shape = (int(w.shape[0]), int(w.shape[1]))
    if not double_quant:
        return NF4Weight(codes, None, None, None, shape, absmax)
    q, c2, mean = nf4_double_quantize(absmax)
    return NF4Weight(codes, q, c2, mean, shape)


def nf4_dequantize(W: NF4Weight, dtype=torch.float32) -> torch.Tensor:
    """Dequantized weight (rows x cols) as float32 or bfloat16."""
    L = load_library()
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dtype must be float32 or bfloat16")
    out = torch.empty(W.shape, dtype=dtype, device=W.device)
    d = W.descriptor()
    _check(L.nf4_dequantize(ctypes.byref(d), _ptr(out), NF4_BF16 if dtype == torch.bfloat16 else NF4_F32,
                            _stream(W.device)))
    return out


def qlora_linear_fwd(W: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, alpha: float,
                     save_t: bool = True):
    """Y = X dequant(W)^T + (alpha/r) (X A^T) B^T.  Returns (Y bf16 [M, N], T bf16 [M, r] or None)."""
    L = load_library()
    N, K = W.shape
    _dev(X, "X", torch.bfloat16)
    _dev(A, "A", torch.bfloat16)
    _dev(B, "B", torch.bfloat16)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M, %d]" % K)
    r = A.shape[0]
    if tuple(A.shape) != (r, K) or tuple(B.shape) != (N, r):
        raise ValueError("A must be [r, K] and B [N, r]")
    M = X.shape[0]
    _same_device(("W", W.codes), ("X", X), ("A", A), ("B", B))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    T = torch.empty((M, r), dtype=torch.bfloat16, device=X.device) if save_t else None
    wsb = L.nf4_workspace_bytes(NF4_OP_LINEAR_FWD, M, N, K, r)
    ws = _workspace(wsb, X.device)
    d = W.descriptor()
    _check(L.qlora_linear_fwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(Y),
                              _ptr(T), _ptr(ws), wsb, _stream(X.device)))
    return Y, T


def qlora_linear_fwd_noalloc(W: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, alpha: float,
                             Y: Optional[torch.Tensor] = None, T: Optional[torch.Tensor] = None,
                             save_t: bool = True):
    """qlora_linear_fwd through the allocation-free entry point: no workspace (the library's
    fixed device scratch serves instead).  Y and T may be given (bf16 [M, N], [M, r]); then
    the call allocates nothing at all.  Returns (Y, T or None)."""
    L = load_library()
    N, K = W.shape
    _dev(X, "X", torch.bfloat16)
    _dev(A, "A", torch.bfloat16)
    _dev(B, "B", torch.bfloat16)
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [M, %d]" % K)
    r = A.shape[0]
    if tuple(A.shape) != (r, K) or tuple(B.shape) != (N, r):
        raise ValueError("A must be [r, K] and B [N, r]")
    M = X.shape[0]
    _same_device(("W", W.codes), ("X", X), ("A", A), ("B", B))
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    elif Y.dtype != torch.bfloat16 or tuple(Y.shape) != (M, N) or not Y.is_contiguous() or Y.device != X.device:
        raise ValueError("Y must be a contiguous bf16 [%d, %d] tensor on %s" % (M, N, X.device))
    if T is None and save_t:
        T = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    elif T is not None and (T.dtype != torch.bfloat16 or tuple(T.shape) != (M, r) or not T.is_contiguous()
                            or T.device != X.device):
        raise ValueError("T must be a contiguous bf16 [%d, %d] tensor on %s" % (M, r, X.device))
    d = W.descriptor()
    _check(L.qlora_linear_fwd_noalloc(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, float(alpha), _ptr(Y),
                                      _ptr(T), _stream(X.device)))
    return Y, T


def qlora_linear_bwd(W: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, alpha: float, T: Optional[torch.Tensor] = None,
                     need_dx: bool = True):
    """Backward of qlora_linear_fwd: (dX bf16 [M, K] or None, dA fp32 [r, K], dB fp32 [N, r])."""
    L = load_library()
    N, K = W.shape
    _dev(X, "X", torch.bfloat16)
    _dev(dY, "dY", torch.bfloat16)
    _dev(A, "A", torch.bfloat16)
    _dev(B, "B", torch.bfloat16)
    M = X.shape[0]
    r = A.shape[0]
    if tuple(dY.shape) != (M, N) or tuple(X.shape) != (M, K):
        raise ValueError("X must be [M, K] and dY [M, N]")
    if tuple(A.shape) != (r, K) or tuple(B.shape) != (N, r):
        raise ValueError("A must be [r, K] and B [N, r]")
    if T is not None:
        _dev(T, "T", torch.bfloat16)
        if tuple(T.shape) != (M, r):
            raise ValueError("T must be [M, r]")
    _same_device(("W", W.codes), ("X", X), ("dY", dY), ("A", A), ("B", B), ("T", T))
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=X.device) if need_dx else None
    dA = torch.empty((r, K), dtype=torch.float32, device=X.device)
    dB = torch.empty((N, r), dtype=torch.float32, device=X.device)
    wsb = L.nf4_workspace_bytes(NF4_OP_LINEAR_BWD, M, N, K, r)
    ws = _workspace(wsb, X.device)
    d = W.descriptor()
    _check(L.qlora_linear_bwd(ctypes.byref(d), _ptr(X), _ptr(dY), M, _ptr(A), _ptr(B), r, float(alpha),
                              _ptr(T), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), wsb, _stream(X.device)))
    return dX, dA, dB


# ---------------------------------------------------------------------------
# Adapter optimizer ("Paged optimizers, and QLoRA end to end", zerotofrontier.app
# "sft/peft"): AdamW over fp32 master copies of the adapters, states paged between
# GPU and host memory.
# ---------------------------------------------------------------------------
def _check_state(name, t, n, device=None):
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
        raise ValueError("%s must be a contiguous float32 tensor of %d values" % (name, n))
    if device == "cuda" and not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device == "host" and (t.is_cuda or not t.is_pinned()):
        raise ValueError("%s must be a page-locked host tensor" % name)


def adamw_step(p: torch.Tensor, g: torch.Tensor, m: torch.Tensor, v: torch.Tensor, lr: float,
               step: int, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
               weight_decay: float = 0.0, p_bf16: Optional[torch.Tensor] = None):
    """One AdamW step in place on fp32 GPU state p, m, v with gradient g (all the same
    size); writes bf16(p) into p_bf16 when given (the layer's A or B)."""
    L = load_library()
    n = p.numel()
    for name, t in (("p", p), ("g", g), ("m", m), ("v", v)):
        _check_state(name, t, n, "cuda")
    if p_bf16 is not None:
        _dev(p_bf16, "p_bf16", torch.bfloat16)
        if p_bf16.numel() != n:
            raise ValueError("p_bf16 must have %d values" % n)
    _check(L.nf4_adamw_step(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(p_bf16), n, float(lr), float(beta1),
                            float(beta2), float(eps), float(weight_decay), int(step), _stream(p.device)))


def adamw_step_paged(p: torch.Tensor, g: torch.Tensor, m: torch.Tensor, v: torch.Tensor, lr: float,
                     step: int, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                     weight_decay: float = 0.0, p_bf16: Optional[torch.Tensor] = None,
                     stage: Optional[torch.Tensor] = None):
    """adamw_step for state paged out to page-locked host tensors p, m, v; g (and
    p_bf16) on the GPU.  The state streams through `stage` (a GPU uint8 buffer,
    64 MiB by default) in stream order; the host tensors must not be touched until
    the stream has run the step."""
    L = load_library()
    n = p.numel()
    for name, t in (("p", p), ("m", m), ("v", v)):
        _check_state(name, t, n, "host")
    _check_state("g", g, n, "cuda")
    if p_bf16 is not None:
        _dev(p_bf16, "p_bf16", torch.bfloat16)
        if p_bf16.numel() != n:
            raise ValueError("p_bf16 must have %d values" % n)
    if stage is None:
        stage = _workspace(64 << 20, g.device)
    _dev(stage, "stage", torch.uint8)
    _check(L.nf4_adamw_step_paged(_ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(p_bf16), n, float(lr),
                                  float(beta1), float(beta2), float(eps), float(weight_decay), int(step),
                                  _ptr(stage), stage.numel(), _stream(g.device)))


class PagedAdamW:
    """AdamW for the adapter tensors with paged optimizer state.

    Each parameter (a bf16 GPU tensor: a layer's A or B) gets an fp32 master copy and
    fp32 moments m, v.  That state lives on the GPU while the total fits
    `device_budget_bytes` (None: no limit) and in page-locked host memory past it;
    `page_out(i)` / `page_in(i)` move one parameter's state between the two.  step()
    updates every parameter from its fp32 gradient and writes the bf16 copy back into
    the parameter tensor: device state in one kernel, host state through a staging
    buffer of `stage_bytes`.  Both paths give identical bits.
    """

    def __init__(self, params, lr: float, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0, device_budget_bytes: Optional[int] = None,
                 stage_bytes: int = 64 << 20):
        self.params = list(params)
        self.lr, self.betas, self.eps, self.weight_decay = float(lr), tuple(betas), float(eps), float(weight_decay)
        self.t = 0
        self.state = []
        used = 0
        for q in self.params:
            _dev(q, "param", torch.bfloat16)
            nb = q.numel() * 12
            on_gpu = device_budget_bytes is None or used + nb <= device_budget_bytes
            p32 = q.detach().float().reshape(-1)
            st = {"p": p32, "m": torch.zeros_like(p32), "v": torch.zeros_like(p32), "host": False}
            if on_gpu:
                used += nb
            else:
                self._to_host(st)
            self.state.append(st)
        self._stage_bytes = int(stage_bytes)
        self._stage = None

    @staticmethod
    def _to_host(st):
        for k in ("p", "m", "v"):
            h = torch.empty(st[k].numel(), dtype=torch.float32, pin_memory=True)
            h.copy_(st[k])
            st[k] = h
        st["host"] = True

    def page_out(self, i: int):
        """Move parameter i's fp32 state to page-locked host memory."""
        st = self.state[i]
        if not st["host"]:
            torch.cuda.current_stream(self.params[i].device).synchronize()
            self._to_host(st)

    def page_in(self, i: int):
        """Move parameter i's fp32 state back to the GPU."""
        st = self.state[i]
        if st["host"]:
            torch.cuda.current_stream(self.params[i].device).synchronize()
            dev = self.params[i].device
            for k in ("p", "m", "v"):
                st[k] = st[k].to(dev)
            st["host"] = False

    def on_host(self, i: int) -> bool:
        return self.state[i]["host"]

    def step(self, grads):
        """One AdamW step for every parameter; grads are fp32 GPU tensors (dA, dB)."""
        grads = list(grads)
        if len(grads) != len(self.params):
            raise ValueError("one gradient per parameter")
        self.t += 1
        b1, b2 = self.betas
        for q, g, st in zip(self.params, grads, self.state):
            gq = g.reshape(-1)
            if st["host"]:
                if self._stage is None:
                    self._stage = _workspace(self._stage_bytes, q.device)
                adamw_step_paged(st["p"], gq, st["m"], st["v"], self.lr, self.t, b1, b2, self.eps,
                                 self.weight_decay, p_bf16=q, stage=self._stage)
            else:
                adamw_step(st["p"], gq, st["m"], st["v"], self.lr, self.t, b1, b2, self.eps,
                           self.weight_decay, p_bf16=q)


# ---------------------------------------------------------------------------
# Codebook comparison ("NF4, derived from normal quantiles", zerotofrontier.app
# "sft/peft"): the same blockwise quantization onto other 16-level tables, and the
# statistics the page compares them by.
# ---------------------------------------------------------------------------
def codebook_int4_symmetric():
    """The symmetric int4 grid {-7..7}/7, with an unused 16th level above 1."""
    return [k / 7 for k in range(-7, 8)] + [2.0]


def codebook_uniform16():
    """The 16-level grid {-8..7}/8."""
    return [k / 8 for k in range(-8, 8)]


def _levels16(levels):
    lv = [float(x) for x in levels]
    if len(lv) != 16:
        raise ValueError("a codebook has 16 levels")
    return (ctypes.c_float * 16)(*lv)


def nf4_quantize_codebook(w: torch.Tensor, levels, blocksize: int = 64):
    """nf4_quantize onto a caller's 16 ascending levels: (codes uint8, absmax fp32)."""
    L = load_library()
    _dev(w, "w")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    n = w.numel()
    codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=w.device)
    absmax = torch.empty((n + blocksize - 1) // blocksize, dtype=torch.float32, device=w.device)
    dt = NF4_BF16 if w.dtype == torch.bfloat16 else NF4_F32
    _check(L.nf4_quantize_codebook(_ptr(w), dt, n, blocksize, _levels16(levels), _ptr(codes), _ptr(absmax),
                                   _stream(w.device)))
    return codes, absmax


def nf4_codebook_stats(w: torch.Tensor, codes: torch.Tensor, absmax: torch.Tensor, levels):
    """Per-code counts, per-code sums of x = w/absmax and the squared error of a
    blockwise quantization, computed on the GPU: (count int64[16], sum_x float64[16],
    sse float) as host values."""
    L = load_library()
    n = w.numel()
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("w must be float32 or bfloat16")
    _numel(codes, "codes", (n + 1) // 2, torch.uint8)
    _numel(absmax, "absmax", (n + 63) // 64, torch.float32)
    _dev(w, "w")
    _dev(codes, "codes")
    _dev(absmax, "absmax")
    _same_device(("w", w), ("codes", codes), ("absmax", absmax))
    dt = NF4_BF16 if w.dtype == torch.bfloat16 else NF4_F32
    out = torch.empty(33, dtype=torch.float64, device=w.device)
    wsb = L.nf4_workspace_bytes(NF4_OP_CODEBOOK_STATS, 0, n, 0, 0)
    ws = _workspace(wsb, w.device)
    _check(L.nf4_codebook_stats(_ptr(w), dt, n, _ptr(codes), _ptr(absmax), _levels16(levels), _ptr(out),
                                _ptr(ws), wsb, _stream(w.device)))
    host = out.cpu()
    count = host[:16].view(torch.int64).numpy().copy()
    return count, host[16:32].numpy().copy(), float(host[32])


def lloyd_codebook(w: torch.Tensor, levels, iters: int = 30):
    """Lloyd's algorithm (one-dimensional k-means) for the squared error of the blockwise
    quantization of w, from `levels`: each step quantizes on the GPU and moves every used
    level to the mean x = w/absmax of its values.  Returns the 16 levels (ascending)."""
    lv = sorted(float(x) for x in levels)
    for _ in range(iters):
        codes, absmax = nf4_quantize_codebook(w, lv)
        count, sum_x, _ = nf4_codebook_stats(w, codes, absmax, lv)
        new = [float(torch.tensor(sum_x[j] / count[j], dtype=torch.float32)) if count[j] > 0 else lv[j]
               for j in range(16)]
        new.sort()
        if new == lv:
            break
        lv = new
    return lv


def nf4_lowrank_svd(E: torch.Tensor, r: int, omega: torch.Tensor, power_iters: int = 2):
    """Rank-r truncated SVD of an fp32 matrix by randomized subspace iteration with the
    K x l test matrix omega: (U [N, r], S [r], V [K, r]), E ~ U diag(S) V^T."""
    L = load_library()
    _dev(E, "E", torch.float32)
    _dev(omega, "omega", torch.float32)
    if E.dim() != 2 or omega.dim() != 2 or omega.shape[0] != E.shape[1]:
        raise ValueError("E must be [N, K] and omega [K, l]")
    _same_device(("E", E), ("omega", omega))
    N, K = E.shape
    l = omega.shape[1]
    U = torch.empty((N, r), dtype=torch.float32, device=E.device)
    S = torch.empty(r, dtype=torch.float32, device=E.device)
    V = torch.empty((K, r), dtype=torch.float32, device=E.device)
    wsb = L.nf4_workspace_bytes(NF4_OP_LOWRANK_SVD, l, N, K, r)
    ws = _workspace(wsb, E.device)
    _check(L.nf4_lowrank_svd(_ptr(E), N, K, r, l, power_iters, _ptr(omega), _ptr(U), _ptr(S), _ptr(V), _ptr(ws),
                             wsb, _stream(E.device)))
    return U, S, V


def loftq_init(W: torch.Tensor, r: int, alpha: float, omega: torch.Tensor, iters: int = 5, power_iters: int = 2):
    """LoftQ-style initialisation for a weight W (fp32 [N, K]): `iters` alternations of
    quantizing the residual W - (alpha/r) B A and a rank-r truncated SVD of the quantization
    error.  Returns (NF4Weight, A bf16 [r, K], B bf16 [N, r], err float64 [iters] on the
    device: ||W - dequant(Q_t) - (alpha/r) B_t A_t||_F per alternation)."""
    L = load_library()
    _dev(W, "W", torch.float32)
    _dev(omega, "omega", torch.float32)
    if W.dim() != 2 or omega.dim() != 2 or omega.shape[0] != W.shape[1]:
        raise ValueError("W must be [N, K] and omega [K, l]")
    _same_device(("W", W), ("omega", omega))
    N, K = W.shape
    l = omega.shape[1]
    n = N * K
    n1 = (n + 63) // 64
    dev = W.device
    codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev)
    q = torch.empty(n1, dtype=torch.uint8, device=dev)
    c2 = torch.empty((n1 + 255) // 256, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    A = torch.empty((r, K), dtype=torch.bfloat16, device=dev)
    B = torch.empty((N, r), dtype=torch.bfloat16, device=dev)
    err = torch.empty(iters, dtype=torch.float64, device=dev)
    wsb = L.nf4_workspace_bytes(NF4_OP_LOFTQ, l, N, K, r)
    ws = _workspace(wsb, dev)
    _check(L.nf4_loftq_init(_ptr(W), N, K, r, float(alpha), iters, l, power_iters, _ptr(omega), _ptr(codes),
                            _ptr(q), _ptr(c2), _ptr(mean), _ptr(A), _ptr(B), _ptr(err), _ptr(ws), wsb,
                            _stream(dev)))
    return NF4Weight(codes, q, c2, mean, (int(N), int(K))), A, B, err
